/*
 * specfold.h -- C ABI of the folded multi-branch verification layer (MI355X / gfx950).
 *
 * One verification pass runs a main branch (index 0) and B draft branches (1..B),
 * arranged as a parent tree, through a transformer layer.  Per layer the library:
 *   - gates every draft position by its parent-child relative residual and folds the
 *     positions at or below the threshold  (specfold_gate);
 *   - compacts the recompute positions of all branches into one list (specfold_compact);
 *   - resolves each folded position to the branch that actually computed it
 *     (specfold_resolve_sources);
 *   - runs RMSNorm + packed QKV + rotary embedding on recompute rows only
 *     (specfold_sparse_qkv);
 *   - computes exact attention for every branch query against that branch's own keys
 *     over the shared prefix cache (specfold_folded_attention);
 *   - applies the output projection and residual to every row (specfold_out_proj);
 *   - runs RMSNorm + SwiGLU FFN on recompute rows only and adds each row's source FFN
 *     output to the row's own residual stream (specfold_sparse_ffn);
 *   - or does all of the above in one call (specfold_verify_layer).
 *
 * Pages defining the method, cited by title and section:
 *   [SpecFold summary]  "SpecFold: Folding Multi-Branch Redundancy for Faster Speculative
 *                        Decoding in Diffusion Language Models", paperlayer.ai summary of
 *                        arXiv 2610.04875v2.
 *   [SpecFold review]   "SpecFold가 확산 언어모델 추측 디코딩의 분기 중복을 접어 속도를
 *                        높인다", onedev.kr/papers/830.
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer to caller-owned memory, except the parent
 *     map, which is a HOST array (copied into kernel arguments).  The library never
 *     allocates, frees or synchronizes; it enqueues kernels on `stream` (a hipStream_t,
 *     NULL = the default stream) and returns.  Device faults surface at the caller's next
 *     synchronization.
 *   - All argument checks run on the host before anything is enqueued; on any error the
 *     call returns a negative status and enqueues nothing.
 *   - bfloat16 tensors are passed as `specfold_bf16` (the raw 16-bit pattern); storage is
 *     row-major and dense unless a stride is given.  Device pointers must be 16-byte
 *     aligned (SPECFOLD_ERR_ALIGN otherwise).
 *   - Rows: R = n_branch * block, row r = i * block + n for branch i, position n.
 *   - Arithmetic: bf16 storage, fp32 accumulation, softmax, RMSNorm, rotary embedding and
 *     residual adds; every bf16 store rounds to nearest even.  Results are deterministic:
 *     two identical calls give bitwise identical outputs (no float atomics).
 *   - Workspace: `ws` is caller-owned device memory of at least
 *     specfold_workspace_bytes(shape) bytes (scratch for intermediates; any initial
 *     contents).  One workspace must not be used by two calls that may run concurrently.
 *   - Data-dependent sizes (the recompute count M) stay on the device: kernels are sized
 *     for the worst case M = R, so no call synchronizes with the host and the whole
 *     layer can be captured in a HIP graph.
 */
#ifndef SPECFOLD_H
#define SPECFOLD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPECFOLD_VERSION 1

/* status codes */
#define SPECFOLD_OK               0
#define SPECFOLD_ERR_NULL        -1  /* a required pointer is NULL                            */
#define SPECFOLD_ERR_SHAPE       -2  /* sizes out of range or inconsistent                     */
#define SPECFOLD_ERR_TREE        -3  /* parent map invalid: need par[0] = -1, 0 <= par[i] < i  */
#define SPECFOLD_ERR_ALIGN       -4  /* a device pointer or stride is not 16-byte aligned      */
#define SPECFOLD_ERR_WORKSPACE   -5  /* workspace NULL or smaller than specfold_workspace_bytes */
#define SPECFOLD_ERR_UNSUPPORTED -6  /* shape outside what the kernels implement (see below)  */
#define SPECFOLD_ERR_ALIAS       -7  /* an output overlaps an input it must not overlap        */
#define SPECFOLD_ERR_HIP         -8  /* the HIP runtime rejected a launch                      */

/* limits (SPECFOLD_ERR_UNSUPPORTED outside them) */
#define SPECFOLD_MAX_BRANCHES 64     /* n_branch = B + 1                                       */
#define SPECFOLD_MAX_BLOCK    64     /* block positions N per branch (attention keeps the N    */
                                     /* block keys of a branch in LDS)                         */
#define SPECFOLD_MAX_HIDDEN   5120   /* D: the gate keeps a whole row in one wave's registers  */
#define SPECFOLD_MAX_QKV_WIDTH 8192  /* (n_q_heads + 2 n_kv_heads) * head_dim                  */
/* head_dim in {16, 32, 64, 128}; hidden, ffn and n_q_heads*head_dim multiples of 64;
   n_q_heads a multiple of n_kv_heads. */

typedef uint16_t specfold_bf16;

/* Sizes of one verification layer. */
typedef struct specfold_shape {
    int32_t n_branch;    /* B + 1: main + drafts, 1..SPECFOLD_MAX_BRANCHES            */
    int32_t block;       /* N positions per branch, 1..SPECFOLD_MAX_BLOCK             */
    int32_t hidden;      /* D                                                          */
    int32_t n_q_heads;   /* Hq                                                         */
    int32_t n_kv_heads;  /* Hkv (grouped-query attention: head h uses KV head          */
                         /*      h / (Hq / Hkv))                                       */
    int32_t head_dim;    /* d                                                          */
    int32_t ffn;         /* F (SwiGLU intermediate width)                              */
    int32_t prefix_len;  /* P shared prefix tokens (>= 0)                               */
    float rms_eps;       /* RMSNorm epsilon                                            */
    float rope_theta;    /* rotary base; block position n sits at absolute position P+n */
} specfold_shape;

/* The shared prefix KV cache of one layer, as a zero-copy strided view
   [SpecFold review, "어떻게 쓰나": the prefix cache is expanded over all branches as a
   strided view, never copied per branch].  Element (t, g, e) of K is
   k[t * k_stride_tok + g * k_stride_head + e] (strides in elements, multiples of 8);
   keys are already rotary-embedded.  The same view serves every branch. */
typedef struct specfold_prefix_kv {
    const specfold_bf16* k;
    const specfold_bf16* v;
    int64_t k_stride_tok, k_stride_head;
    int64_t v_stride_tok, v_stride_head;
} specfold_prefix_kv;

/* Weights of one layer, torch Linear layout ([out][in], row-major, bf16):
   ln1, ln2  [D]                RMSNorm weights
   w_qkv     [(Hq+2Hkv)*d][D]   Q heads, then K heads, then V heads
   w_o       [D][Hq*d]
   w_gate_up [2F][D]            gate rows, then up rows
   w_down    [D][F]                                                              */
typedef struct specfold_layer_weights {
    const specfold_bf16* ln1;
    const specfold_bf16* w_qkv;
    const specfold_bf16* w_o;
    const specfold_bf16* ln2;
    const specfold_bf16* w_gate_up;
    const specfold_bf16* w_down;
} specfold_layer_weights;

/* Optional per-call outputs of specfold_verify_layer (each member may be NULL). */
typedef struct specfold_layer_stats {
    float*   rho;        /* [R] relative residual, 0 for main                      */
    uint8_t* fold;       /* [R] 1 = folded                                          */
    int32_t* rec_count;  /* [1] M, the number of recompute rows                     */
    int32_t* src_slot;   /* [R] slot of each row's source in the recompute list     */
} specfold_layer_stats;

/* Optional per-kernel timing: `events` holds n_events hipEvent_t created by the caller
   (specfold_event_create); launch k of a call is bracketed by events[2k] and
   events[2k+1] when 2k+1 < n_events.  specfold_stage_name(k) names launch k. */
typedef struct specfold_trace {
    void* const* events;
    int32_t n_events;
} specfold_trace;

int         specfold_version(void);
const char* specfold_status_str(int status);
/* Name and text of the HIP error behind the calling thread's last SPECFOLD_ERR_HIP. */
const char* specfold_last_error(void);
/* Bytes of workspace every entry point of this shape needs (0 if the shape is invalid). */
size_t      specfold_workspace_bytes(const specfold_shape* shape);
/* Number and names of the kernel launches of specfold_verify_layer. */
int         specfold_stage_count(void);
const char* specfold_stage_name(int stage);
/* hipEvent helpers for specfold_trace (host-side wrappers of the HIP runtime). */
int specfold_event_create(void** event);
int specfold_event_destroy(void* event);
int specfold_event_elapsed_ms(void* start, void* stop, float* ms);

/* ---------------------------------------------------------------- step 1: the gate
 * [SpecFold review, "무엇과 다른가"]: rho = |H_i[n] - H_par(i)[n]| / |H_par(i)[n]|
 * (Euclidean norms over D); position (i,n) folds when rho <= delta.
 * [SpecFold summary, App. B]: main bypasses the gate (fold = 0, rho = 0).
 * Zero parent row: rho = 0 if the child row is zero too, +inf otherwise; NaN never folds.
 * Norms accumulate in fp32; sqrt and division are IEEE correctly rounded.
 *   parent_host [n_branch] host int32: par[0] = -1, 0 <= par[i] < i
 *   H      [R][D] bf16 layer-input hidden states (the raw residual stream); when H is read
 *          (rho_in NULL or inv_rms given) it must be smaller than 1 GB, i.e. 2 R D < 2^30
 *          (SPECFOLD_ERR_UNSUPPORTED otherwise)
 *   rho_in [R] fp32 or NULL: when given, threshold these values instead of computing rho
 *          (H is then read only for inv_rms)
 *   rho    [R] fp32 out;  fold [R] u8 out (1 = folded)
 *   inv_rms [R] fp32 out or NULL: 1/sqrt(mean(H[r]^2) + eps), the RMSNorm scale of each row
 */
int specfold_gate(const specfold_shape* shape, const int32_t* parent_host,
                  const specfold_bf16* H, float delta, const float* rho_in,
                  float* rho, uint8_t* fold, float* inv_rms, void* stream);

/* ---------------------------------------------------------------- step 2: compaction
 * [SpecFold summary, App. B]: recompute indices of all branches are compacted into a global
 * list and per-branch lists.  rec_rows[0..M) holds the recompute rows (fold == 0) in
 * ascending row order; branch i's list is rec_rows[branch_off[i] .. branch_off[i+1]).
 *   fold       [R] u8 in
 *   rec_rows   [R] int32 out (entries >= M untouched)
 *   rec_count  [1] int32 out: M
 *   branch_off [n_branch + 1] int32 out
 *   row_slot   [R] int32 out: slot of row r in rec_rows, -1 when folded
 *   ws         device scratch of specfold_compact_workspace_bytes(shape) bytes, any contents
 *              (may be NULL when that is 0).  Past 8192 rows the scan is one pass over 32768-row
 *              tiles with a decoupled look-back between them; its status words live here and
 *              are cleared by the call itself.  One workspace must not serve two calls that may
 *              run concurrently.
 */
int specfold_compact(const specfold_shape* shape, const uint8_t* fold, int32_t* rec_rows,
                     int32_t* rec_count, int32_t* branch_off, int32_t* row_slot, void* ws, size_t ws_bytes,
                     void* stream);
/* Bytes of workspace specfold_compact needs for this shape (0 if the shape is invalid or needs
   none: up to 8192 rows one workgroup scans them all). */
size_t specfold_compact_workspace_bytes(const specfold_shape* shape);

/* ---------------------------------------------------------------- step 3: fold sources
 * [SpecFold summary, App. B and §A.3]: each folded position follows its fold chain to the
 * nearest ancestor that recomputed it, in one order-free launch.
 * src(i,n) = i if (i,n) is recomputed else src(par(i), n); branch 0 always terminates.
 *   fold [R] u8, row_slot [R] int32 (from specfold_compact) in
 *   src_branch [R] int32 out, src_slot [R] int32 out (= row_slot[src*N + n])
 */
int specfold_resolve_sources(const specfold_shape* shape, const int32_t* parent_host,
                             const uint8_t* fold, const int32_t* row_slot,
                             int32_t* src_branch, int32_t* src_slot, void* stream);

/* ---------------------------------------------------------------- step 4: sparse QKV
 * [SpecFold summary, App. B]: recompute positions get RMSNorm, the packed QKV projection and
 * rotary embedding; folded positions inherit [SpecFold review, "무엇과 다른가"].
 * For slot m < M, row r = rec_rows[m], position n = r % N:
 *   x = H[r] * inv_rms[r] * ln1;  [q|k|v] = x W_qkv^T;  q, k rotated (rotate-half, angle
 *   (P+n) * theta^(-2j/d)) ;  stored as q_c[m][Hq][d], k_c[m][Hkv][d], v_c[m][Hkv][d] bf16.
 *   inv_rms [R] fp32 from specfold_gate.  rec_count is read on the device; q_c/k_c/v_c need
 *   capacity R rows.
 */
int specfold_sparse_qkv(const specfold_shape* shape, const specfold_bf16* H,
                        const float* inv_rms, const int32_t* rec_rows, const int32_t* rec_count,
                        const specfold_bf16* ln1, const specfold_bf16* w_qkv,
                        specfold_bf16* q_c, specfold_bf16* k_c, specfold_bf16* v_c,
                        void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- step 5: folded attention
 * [SpecFold review, "무엇과 다른가"]: attention is exact with respect to each branch's own
 * KV; [SpecFold summary, §A.1]: a folded query's state equals the child's exact state.
 * For every row (i,n) and head h, with s(i,m) = src_slot[i*N+m] and g = h / (Hq/Hkv):
 *   attn[i*N+n][h*d : (h+1)*d] = softmax(q K^T / sqrt(d)) V over the keys
 *   [prefix K[:, g] ; k_c[s(i,0..N-1)][g]], q = q_c[s(i,n)][h]; no mask.
 * The prefix part is computed once per recompute slot (a folded row's query and the
 * prefix equal its source's) and merged with the per-branch block part by log-sum-exp.
 *   lse [R][Hq] fp32 out or NULL: natural log of the softmax denominator of the scaled
 *   scores (the retained per-head softmax statistics).
 *   A row whose src_slot is outside [0, M) gets NaN outputs.
 */
int specfold_folded_attention(const specfold_shape* shape, const specfold_bf16* q_c,
                              const specfold_bf16* k_c, const specfold_bf16* v_c,
                              const int32_t* rec_rows, const int32_t* rec_count,
                              const int32_t* src_slot, const specfold_prefix_kv* prefix,
                              specfold_bf16* attn, float* lse,
                              void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- step 6: output projection
 * Not described by the pages; read as dense over all R rows (folded rows' attention outputs
 * differ from their parents').  h_mid[r] = H[r] + attn[r] W_o^T for every row.
 *   attn [R][Hq*d], H [R][D] in; h_mid [R][D] out (must not alias H or attn).
 */
int specfold_out_proj(const specfold_shape* shape, const specfold_bf16* attn,
                      const specfold_bf16* H, const specfold_bf16* w_o, specfold_bf16* h_mid,
                      void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- step 7: sparse FFN + inherit
 * [SpecFold summary, §A.2 and App. B]: the FFN runs on recompute rows; every position adds
 * its own residual stream, which is never folded; folded positions reuse their source's
 * FFN output.  For slot m < M: y = RMSNorm(h_mid[rec_rows[m]]) * ln2;
 * f[m] = (silu(y W_gate^T) * (y W_up^T)) W_down^T.  For every row r:
 * H_out[r] = h_mid[r] + f[src_slot[r]]  (NaN when src_slot[r] is outside [0, M)).
 *   H_out [R][D] out (must not alias h_mid).
 */
int specfold_sparse_ffn(const specfold_shape* shape, const specfold_bf16* h_mid,
                        const int32_t* rec_rows, const int32_t* rec_count,
                        const int32_t* src_slot, const specfold_bf16* ln2,
                        const specfold_bf16* w_gate_up, const specfold_bf16* w_down,
                        specfold_bf16* H_out, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- the whole layer
 * [SpecFold summary, §3.2, App. A.3 and App. B]: steps 1-7 on the caller's stream, with the
 * gate, compaction and resolution fused into one launch.  delta = 0 folds only rows with
 * rho == 0 (dense verification on perturbed inputs).  H_out must not alias H_in.
 *   stats NULL or per-call outputs; trace NULL or per-launch events.
 */
int specfold_verify_layer(const specfold_shape* shape, const int32_t* parent_host,
                          const specfold_layer_weights* weights,
                          const specfold_prefix_kv* prefix, const specfold_bf16* H_in,
                          float delta, specfold_bf16* H_out, specfold_layer_stats* stats,
                          const specfold_trace* trace, void* ws, size_t ws_bytes,
                          void* stream);

/* ---------------------------------------------------------------- the whole layer, no workspace
 * For callers that cannot allocate device memory or pass a workspace (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): specfold_verify_layer with
 * its workspace taken from a device array inside the library instead of `ws`.  The array holds
 * SPECFOLD_NOALLOC_SCRATCH_BYTES on every device the library runs on, from the first call on
 * that device (which looks its address up, with that device current) until the process ends.
 * Nothing is allocated or freed by any call.  Arguments, outputs and errors are those of
 * specfold_verify_layer (same kernels, same bits); a shape whose workspace
 * (specfold_workspace_bytes) exceeds SPECFOLD_NOALLOC_SCRATCH_BYTES returns
 * SPECFOLD_ERR_WORKSPACE before anything is enqueued.  The calling thread's current device must
 * be the stream's device.  Every call on one device shares the array: calls that may overlap on
 * one device (concurrent streams, threads) race and must be serialized by the caller.
 */
#define SPECFOLD_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

int specfold_verify_layer_noalloc(const specfold_shape* shape, const int32_t* parent_host,
                                  const specfold_layer_weights* weights,
                                  const specfold_prefix_kv* prefix, const specfold_bf16* H_in,
                                  float delta, specfold_bf16* H_out, specfold_layer_stats* stats,
                                  const specfold_trace* trace, void* stream);

/* ---------------------------------------------------------------- either side of the stack
 * [SpecFold summary, App. B]: the folded kernels cover the transformer layers; the token
 * embedding before the first layer and the language-model head after the last one stay
 * outside them and are not folded -- every row of every branch gets its logits.
 * R = n_branch * block rows, D = hidden; vocab V >= 1.
 *
 * specfold_embed: H[r] = E[tokens[r]] for every row; a token id outside [0, V) gives a row of
 * NaN.  tokens [R] int32 device, E [V][D] bf16 device, H [R][D] bf16 out.
 */
int specfold_embed(const specfold_shape* shape, const int32_t* tokens, const specfold_bf16* E,
                   int32_t vocab, specfold_bf16* H, void* stream);

/* Bytes of workspace specfold_lm_head needs for this shape and vocabulary (0 if invalid). */
size_t specfold_head_workspace_bytes(const specfold_shape* shape, int32_t vocab);

/* specfold_lm_head: final RMSNorm, LM head and greedy token of every row:
 *   xn = RMSNorm(H[r]) * ln_f (rms_eps of the shape);  logits[r][v] = xn . W_lm[v] (fp32
 *   accumulation, no bias);  token[r] = the lowest index among the maximal logits, logit[r]
 *   that maximum.  The logits are never stored: each workgroup keeps its columns' best per
 *   row and a second launch merges them in column order.  NaN logits are never chosen; a
 *   row without a finite or infinite candidate gets token -1 and logit NaN.
 *   H [R][D] bf16, ln_f [D] bf16, W_lm [V][D] bf16 (torch Linear layout; any size -- the
 *   vocabulary is streamed in pieces under 1 GB); token [R] int32 out, logit [R] fp32 out;
 *   ws: specfold_head_workspace_bytes(shape, vocab) bytes, any contents.
 */
int specfold_lm_head(const specfold_shape* shape, const specfold_bf16* H, const specfold_bf16* ln_f,
                     const specfold_bf16* w_lm, int32_t vocab, int32_t* token, float* logit,
                     void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SPECFOLD_H */
