/* The pages' attention-state correction for folded rows, built as a comparison variant.

   [SpecFold summary, App. B and §A.1]: a folded position starts from its parent's retained
   streaming-softmax state (running maximum, denominator and unnormalised numerator per
   head), removes the parent's terms at the block positions the child recomputed and adds
   the child's terms there; [§A.3]: branches are visited in topological order, so the parent's
   state is already corrected when the child needs it.

   This library is separate from libspecfold: the layer itself reaches the same exact state by
   a prefix-partial + block merge (specfold_folded_attention), and this variant exists only so
   tests and the benchmark can compare the two methods' cost and numerics.  It uses the layout
   types of include/specfold.h.

   State buffer: float [R][Hq][head_dim + 2] with R = n_branch * block; per (row, head) the
   running maximum m (base-2 units of the scaled score), the denominator l and the numerator
   acc[head_dim].  Every pointer is a device pointer to caller-owned memory, except
   parent_host (host, n_branch int32, parent[0] = -1, 0 <= parent[i] < i).  Calls enqueue on
   `stream` and return the library's status codes (0 OK, -1 null pointer, -2 bad shape,
   -3 bad parent tree, -8 launch error); nothing is enqueued on an error.  Shapes: head_dim in
   {16, 32, 64, 128}, at most 8 query heads per KV head (one wave each in a workgroup), the
   library's branch and block limits. */
#ifndef SPECFOLD_CORRECTION_H
#define SPECFOLD_CORRECTION_H

#include <stdint.h>

#include "specfold.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Depth levels of the parent tree: masks[d - 1] has bit i set for every branch i at depth d
   (depth of branch 0 is 0); *n_levels = maximum depth.  masks holds n_branch entries.
   Host only. */
int specfold_variant_correction_levels(const specfold_shape* shape, const int32_t* parent_host,
                                       uint64_t* masks, int32_t* n_levels);

/* Fresh state of every recompute row (slot s < rec_count, row rec_rows[s]): streaming softmax
   over [prefix keys ; the row's branch block keys K_i[m] = k_c[src_slot[i * block + m]]], in
   key order, fp32.  q_c/k_c/v_c are slot-indexed bf16 [R][H][head_dim] as produced by
   specfold_sparse_qkv. */
int specfold_variant_correction_fresh(const specfold_shape* shape, const specfold_bf16* q_c,
                                      const specfold_bf16* k_c, const specfold_bf16* v_c,
                                      const int32_t* rec_rows, const int32_t* rec_count,
                                      const int32_t* src_slot, const specfold_prefix_kv* prefix,
                                      float* state, void* stream);

/* One depth level: every folded row (fold[r] != 0) of a branch in branch_mask takes its
   parent's state at the same position and replaces the parent's terms at the child's
   recomputed positions (fold[i * block + m] == 0) by the child's: with mx = max(m_parent,
   the child's new scores), l = l_parent 2^(m_parent - mx) - sum 2^(s_old - mx)
   + sum 2^(s_new - mx), and the numerator likewise with the value rows. */
int specfold_variant_correction_level(const specfold_shape* shape, const int32_t* parent_host,
                                      uint64_t branch_mask, const specfold_bf16* q_c,
                                      const specfold_bf16* k_c, const specfold_bf16* v_c,
                                      const int32_t* src_slot, const uint8_t* fold, float* state,
                                      void* stream);

/* out[r][h][j] = acc / l for every row and head, fp32 [R][Hq][head_dim]. */
int specfold_variant_correction_finalize(const specfold_shape* shape, const float* state, float* out,
                                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECFOLD_CORRECTION_H */
