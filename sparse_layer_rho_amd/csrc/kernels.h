// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace specfold {

// ------------------------------------------------------------------ gate / compaction / sources
struct GateParams {
    const uint16_t* H;       // [R][D]
    ParentMap par;
    int nb, N, D;
    float delta;
    const float* rho_in;     // nullable
    float* rho;              // [R]
    uint8_t* fold;           // [R]
    float* inv_rms;          // nullable
    float eps;
    const uint16_t* ln;      // nullable: with xn, also write xn[r] = H[r] * inv_rms * ln (bf16)
    uint16_t* xn;            // nullable [R][D]
    uint8_t* fold_copy;      // nullable second copy of the fold flags
};

struct CompactParams {
    const uint8_t* fold;
    int R, N, nb;
    int32_t* rec_rows;
    int32_t* rec_count;
    int32_t* branch_off;
    int32_t* row_slot;
};

struct ResolveParams {
    const uint8_t* fold;
    ParentMap par;
    int nb, N, R;
    const int32_t* row_slot;
    int32_t* src_branch;
    int32_t* src_slot;
};

hipError_t launch_gate(const GateParams& p, hipStream_t st);
// ws: compact_workspace_bytes(R) bytes (may be NULL when that is 0), any contents
size_t compact_workspace_bytes(int R);
hipError_t launch_compact(const CompactParams& p, void* ws, hipStream_t st);
hipError_t launch_resolve(const ResolveParams& p, hipStream_t st);

// xn[r] = X[r] * s_r * ln (bf16), s_r = inv_rms[r] or, when inv_rms is NULL, 1/sqrt(mean(X[r]^2)+eps)
hipError_t launch_row_norm(const uint16_t* X, int R, int D, const float* inv_rms, float eps, const uint16_t* ln,
                           uint16_t* xn, hipStream_t st);

// ------------------------------------------------------------------ gathered-row GEMM
// C[m][n] = sum_k A[row(m)][k] W[n][k] for m < M; row(m) = a_rows[m], m, or the m-th
// recompute row of the fold flags (fused compaction).
struct GemmArgs {
    const uint16_t* A;
    int64_t lda;
    const int32_t* a_rows;   // nullable: identity
    int a_row_limit;         // gathered indices outside [0, limit) read as zero rows
    const int32_t* m_count;  // nullable: use m_fixed
    int m_fixed;
    int m_cap;               // M is clamped to [0, m_cap]; outputs have m_cap rows
    const uint16_t* W;       // [Nout][K]
    int K, Nout;
    int n_groups, m_chunks;  // set by the launcher
    int min_chunks;          // set by the launcher: rows split over at least this many workgroups
    float* partial;          // [splits][m_cap][Nout]   (partial-sum epilogue)
    uint16_t* act;           // [m_cap][F]              (SwiGLU epilogue)
    int F;
    // fused compaction (fc_fold non-NULL): rows = recompute rows of the fold flags, compacted
    // in LDS by every workgroup; the grid's last workgroup (an idle one) publishes the list and
    // the fold sources
    const uint8_t* fc_fold;
    int fc_R, fc_N, fc_nb;
    ParentMap fc_par;
    int32_t* fc_rec_rows;
    int32_t* fc_rec_count;
    int32_t* fc_branch_off;
    int32_t* fc_row_slot;
    int32_t* fc_src_branch;
    int32_t* fc_src_slot;
    int32_t* fc_count_copy;      // nullable extra copies (per-call statistics)
    int32_t* fc_src_slot_copy;
    // greedy-token epilogue: per (column group, row) the best output and its column
    float* arg_val;              // [group_base + n_groups][m_cap]
    int32_t* arg_idx;            // column + col_base, or -1 when the group has no candidate
    int col_base, group_base;
    int xcd_split;               // set by the launcher from GemmCfg::xcd_split
};

// Tile shape of one launch: a workgroup covers the output columns of one of `groups` even
// column groups (at most gemm_group_cols), a chunk of gemm_chunk_rows rows and one of `splits`
// K ranges (grid.y; the partial buffer holds splits * m_cap * Nout floats).  Its 4 waves form a
// wn x (4/wn) grid; a wave owns ntw 16-row weight tiles and tm 16-row activation tiles; a weight
// stage spans ksub compute stages of 64 K; nbw weight and nba activation slots form the LDS rings.  swiglu: the gate/up GEMM (Nout = 2F, gate rows then up rows, no K
// split) writing act = silu(g) * u.
struct GemmCfg {
    int ntw, wn, tm, ksub, nbw, nba, groups, splits;
    bool swiglu;
    int min_chunks;          // row workgroups per column group used at least (when there are that many)
    bool argmax;             // greedy-token epilogue (wn must be 1, no K split)
    int lw;                  // 0, or 4 load waves beside the compute waves (one workgroup per CU)
    bool xcd_split;          // K-splits placed by XCD (partial-sum epilogue, S a multiple of 8)
};
// the (ntw, wn, tm, ksub, nbw, nba, lw) shapes compiled
#define SPECFOLD_GEMM_CASES(X)                                                                     \
    X(4, 1, 1, 2, 2, 2, 0) X(4, 1, 1, 1, 3, 2, 0) X(4, 1, 2, 1, 4, 2, 0) X(2, 2, 2, 2, 2, 2, 0)         \
    X(8, 1, 2, 1, 3, 2, 0) X(4, 1, 2, 1, 4, 3, 4) X(6, 1, 2, 1, 4, 2, 0) X(4, 1, 2, 1, 4, 3, 0)
int gemm_chunk_rows(const GemmCfg& c);
int gemm_group_cols(const GemmCfg& c);
size_t gemm_lds_bytes(const GemmCfg& c);
hipError_t launch_gemm(const GemmArgs& a, const GemmCfg& c, hipStream_t st);
// SwiGLU projection with three tile shapes in one launch: c[0] for M <= upto[0] rows, c[1] for
// M <= upto[1], c[2] above, chosen on the device (no fused compaction).  Every shape forms each
// output's sum in the same order.  The (c[0] ; c[1] ; c[2] ; lw, the same for all three)
// triples compiled:
#define SPECFOLD_GEMM_TRIPLES(X)                                                                   \
    X(6, 1, 1, 1, 3, 2, 6, 1, 2, 1, 3, 2, 8, 1, 2, 1, 3, 2, 0)                                     \
    X(8, 1, 1, 1, 3, 2, 8, 1, 2, 1, 3, 2, 8, 1, 2, 1, 3, 2, 0)                                     \
    X(6, 1, 1, 1, 4, 3, 6, 1, 2, 1, 4, 3, 8, 1, 2, 1, 3, 2, 4)
hipError_t launch_gemm_shapes(const GemmArgs& a, const GemmCfg* c, const int* upto, hipStream_t st);

// ------------------------------------------------------------------ GEMM epilogues
struct QkvEpiArgs {
    const float* part; int splits, m_cap;
    const int32_t* m_count;
    const int32_t* rec_rows;
    int R, N, Hq, Hkv, hd, P;
    double inv_freq[64];     // theta^(-2j/d), j < d/2
    uint16_t* q_c; uint16_t* k_c; uint16_t* v_c;
};
hipError_t launch_qkv_epilogue(const QkvEpiArgs& a, hipStream_t st);

// h_mid = H + sum of partials (bf16); with xn, also xn = RMSNorm(h_mid) * ln (bf16)
hipError_t launch_oproj_epilogue(const float* part, int splits, int R, int D, const uint16_t* H,
                                 uint16_t* h_mid, const uint16_t* ln, float eps, uint16_t* xn,
                                 hipStream_t st);

// f[m] = sum of partials of slot m; H_out[r] = h_mid[r] + f[src_slot[r]] for every row that
// inherits from slot m (rows with an invalid slot get NaN)
hipError_t launch_down_epilogue(const float* part, int splits, int m_cap, const int32_t* m_count,
                                const int32_t* rec_rows, const int32_t* src_slot, int nb, int N, int D,
                                const uint16_t* h_mid, uint16_t* H_out, hipStream_t st);

// ------------------------------------------------------------------ attention
struct AttnArgs {
    const uint16_t* q_c; const uint16_t* k_c; const uint16_t* v_c;
    const int32_t* m_count; int m_cap;
    const int32_t* src_slot;
    int nb, N, Hq, Hkv, hd, P;
    const uint16_t* pk; const uint16_t* pv;
    int64_t pk_st, pk_sh, pv_st, pv_sh;
    int chunk_len, n_chunks;
    float* part_o;           // [n_chunks][m_cap][Hq][hd]
    float* part_ml;          // [n_chunks][m_cap][Hq][2]
    uint16_t* attn;          // [R][Hq*hd]
    float* lse;              // nullable [R][Hq]
    float scale_log2;        // log2(e) / sqrt(hd)
    int plan_rows;           // recompute rows the prefix tiles are planned for (0: half of m_cap)
};
hipError_t launch_attn_prefix(const AttnArgs& a, hipStream_t st);
// rows kernels either side of the stack
hipError_t launch_rmsnorm_rows(const uint16_t* H, int R, int D, const uint16_t* ln, float eps, uint16_t* xn,
                               hipStream_t st);
hipError_t launch_embed(const int32_t* tokens, int R, const uint16_t* E, int V, int D, uint16_t* H, hipStream_t st);
hipError_t launch_argmax_merge(const float* arg_val, const int32_t* arg_idx, int groups, int R, int32_t* token,
                               float* logit, hipStream_t st);
hipError_t launch_attn_block(const AttnArgs& a, hipStream_t st);

}  // namespace specfold
