// C ABI of the folded verification layer: argument checks, workspace layout and the launch
// sequence of each entry point.  Every check runs before the first launch, so a call that
// returns an error has enqueued nothing.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <cmath>
#include <mutex>

#include "../../include/specfold.h"
#include "kernels.h"

using namespace specfold;

namespace {

static_assert(kMaxBranches == SPECFOLD_MAX_BRANCHES, "branch limit mismatch");

constexpr int kMaxGateBlock = 1 << 20;   // positions per branch accepted by gate/compact/resolve

struct Dims {
    int nb, N, R, D, Hq, Hkv, hd, F, P, Nq, Do;
    float eps, theta;
};

struct Layout {
    GemmCfg c_qkv, c_o, c_gu, c_down;
    GemmCfg c_down_few;          // the down projection when few rows are expected to recompute (delta > 0)
    GemmCfg c_gu_shapes[3];      // gate/up tile shapes for up to gu_upto[0], up to gu_upto[1], and more rows
    int gu_upto[2];
    GemmCfg c_gu_shapes_few[3];  // the same when few rows are expected to recompute (delta > 0)
    bool gu_multi;               // false: c_gu for every row count
    size_t rho, fold, inv_rms, rec_rows, rec_count, branch_off, row_slot, src_branch, src_slot;
    size_t xn1, xn2, q_c, k_c, v_c, attn, h_mid, act, gemm_part, attn_o, attn_ml;
    size_t total;
    int s_qkv, s_o, s_down, chunk_len, n_chunks;
};

inline size_t align_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

Dims dims_of(const specfold_shape& s) {
    Dims d;
    d.nb = s.n_branch; d.N = s.block; d.R = s.n_branch * s.block; d.D = s.hidden;
    d.Hq = s.n_q_heads; d.Hkv = s.n_kv_heads; d.hd = s.head_dim; d.F = s.ffn; d.P = s.prefix_len;
    d.Nq = (s.n_q_heads + 2 * s.n_kv_heads) * s.head_dim; d.Do = s.n_q_heads * s.head_dim;
    d.eps = s.rms_eps; d.theta = s.rope_theta;
    return d;
}

// Tile shape, column groups and K split of one projection.  A workgroup streams 64 or 128
// weight rows against a chunk of activation rows through small LDS rings, so two or three
// workgroups share a CU and hide each other's waits.  The tile shape is performance only (every
// shape forms each sum in the same order); the K-splits come from the projection's shape alone.
enum GemmKind { GEMM_QKV, GEMM_O, GEMM_GATE_UP, GEMM_DOWN };

// K-splits of a partial-sum projection as a function of (kind, output columns, K) only -- not
// of the row count -- so every output's sum is formed in the same order whatever the batch:
// a batched verification pass matches serialized verification (each branch alone) bit for bit
// [SpecFold summary, App. C: the drift of batched matmuls comes from shape-dependent
// accumulation order].  The counts aim at about 512 (QKV), 768 (o_proj) and 384 (down) busy
// workgroups with the row workgroups a 288-row layer has (2, 5 and 1 per column group), as
// measured best on the 1.5B layer.
constexpr int kNumCUs = 256;                        // compute units of the GPU (MI355X)

int splits_for(GemmKind kind, int n_cols, int k) {
    if (kind == GEMM_GATE_UP) return 1;             // SwiGLU needs the whole sum
    const int rows = kind == GEMM_QKV ? 2 : kind == GEMM_O ? 5 : 1;
    int cols = 64;
    if (kind != GEMM_DOWN && ((n_cols + 63) / 64) * rows < 128) cols = 32;
    const int busy = ((n_cols + cols - 1) / cols) * rows;
    const int target = kind == GEMM_DOWN ? 384 : kind == GEMM_O ? 768 : 512;
    int s = (target + busy / 2) / busy;
    int smax = (k + 127) / 128 / 2;                  // two 128-element units per split at least
    if (smax > 32) smax = 32;                        // the epilogues batch up to 32 splits
    if (s > smax) s = smax;
    return s < 1 ? 1 : s;
}

// Measured on the 1.5B, 7B and 14B layers (each projection alone, cold weights, and whole layers):
//   * QKV, the recompute rows (M ~ 100 folded): 64-column groups, two 64-row chunks; 1.5B
//     6.9 us against 7.7 with 32-column groups;
//   * o_proj, all R rows: 128-row chunks, three at R = 288 instead of five of 64, so the weights
//     are re-read least; 1.5B 8.5 against 9.2 us, 7B 19.7 against 28.4, 14B 35 against 51; three
//     activation slots (two stages in flight) and four load waves when the grid fits one
//     workgroup per CU: 1.5B 9.1 against 9.4 us (7B, 504 workgroups: 20.05 against 20.08 with
//     them, so it keeps two slots);
//   * gate/up up to 128 rows (above, gemm_shapes_kernel's three shapes): weight stages of 256 bytes
//     per row;
//   * down: 128-row chunks; 128-column groups when a K-split spans at least 1024 elements (the
//     7B and 14B shapes: 38 against 44 us at M = 108), else 64 (1.5B, 560 elements per split,
//     where the wider tiles lose 4 us at M = 288) with three activation slots (80 KB, two
//     workgroups per CU: 1.5B dense 28.9 against 30.1-30.4 us).
GemmCfg pick_gemm(GemmKind kind, int n_cols, int k, int max_rows) {
    GemmCfg c{};
    c.swiglu = kind == GEMM_GATE_UP;
    c.wn = 1;
    c.splits = splits_for(kind, n_cols, k);
    switch (kind) {
    case GEMM_QKV: c.ntw = 4; c.tm = 1; c.ksub = 1; c.nbw = 3; c.nba = 2; break;
    case GEMM_O: c.ntw = 4; c.tm = 2; c.ksub = 1; c.nbw = 4; c.nba = 2; break;
    case GEMM_GATE_UP: c.ntw = 4; c.tm = 1; c.ksub = 2; c.nbw = 2; c.nba = 2; break;
    case GEMM_DOWN:
        if (k / c.splits >= 1024) { c.ntw = 8; c.tm = 2; c.ksub = 1; c.nbw = 3; c.nba = 2; }
        else { c.ntw = 4; c.tm = 2; c.ksub = 1; c.nbw = 4; c.nba = 3; }
        break;
    }
    if (max_rows <= 64) { c.ntw = 2; c.wn = 2; c.tm = 2; c.ksub = 2; c.nbw = 2; c.nba = 2; }
    const int cap = gemm_group_cols(c);
    c.groups = (n_cols + cap - 1) / cap;
    // o_proj: a third activation slot while its workgroups fit one per CU (the 80 KB rings leave
    // no room for a second)
    if (kind == GEMM_O && c.wn == 1) {
        const int rows = gemm_chunk_rows(c);
        const long wgs = static_cast<long>(c.groups) * ((max_rows + rows - 1) / rows) * c.splits;
        c.nba = wgs <= kNumCUs ? 3 : 2;
        c.lw = wgs <= kNumCUs ? 4 : 0;
    }
    // the recompute-row projections keep two row workgroups per column group however small M
    // is (the split counts assume them)
    c.min_chunks = (kind == GEMM_QKV || kind == GEMM_GATE_UP) ? 2 : 1;
    return c;
}

// Gate/up tiles for more than 128 rows (R > 128): one launch holds three tile shapes and the
// device picks by the recompute count M (gemm_shapes_kernel).  Each group's weights stream once
// per row chunk; the CU count sets the group counts.
//   * many rows: 64-column groups (ntw 8), the fewest groups, so the activations -- read again
//     by every group -- cost least; 128-row chunks, three of <= 96 rows at M = 288.
//   * few rows: 256 k groups, k the fewest workgroups per CU that keeps a group within 64
//     columns, so every CU ingests the same weight bytes; the narrowest tile (ntw 6 for <= 48
//     columns, else 8) that covers a group; one 128-row chunk up to 256 rows when k = 1 (two
//     chunks still fill two workgroups per CU), else up to 128.
//   * up to 64 rows: the few-rows groups with a 64-row tile (no MFMAs on empty row tiles).
// Measured (gate/up alone, cold weights, us; few-rows / many-rows shape against the single
// 32-column shape pick_gemm uses up to 128 rows): 1.5B M 108: 21.9 / 24.8, M 288: 32.4 / 39.8;
// 7B M 108: 66.1 / 88.7, M 288: 121 / 155; 14B M 108: 65.9 / 104, M 288: 133 / 162.  At M = 60
// the 64-row tile against the 128-row one: 1.5B 18.2 / 21.1, 7B 54.7 / 59.1, 14B 57.6 / 62.0.
void pick_gate_up_shapes(int F, GemmCfg* c, int* upto) {
    const int k = (F + 256 * 64 - 1) / (256 * 64);
    const int tiles = (F + 15) / 16;
    const int g_few = 256 * k < tiles ? 256 * k : tiles;
    const int ntw = (F + g_few - 1) / g_few <= 48 ? 6 : 8;
    c[0] = GemmCfg{ntw, 1, 1, 1, 3, 2, g_few, 1, true, 1, false};
    c[1] = GemmCfg{ntw, 1, 2, 1, 3, 2, g_few, 1, true, 1, false};
    c[2] = GemmCfg{8, 1, 2, 1, 3, 2, (F + 63) / 64, 1, true, 1, false};
    upto[0] = 64;
    upto[1] = k == 1 ? 256 : 128;
}

// The gate/up shapes when few rows are expected to recompute (the layer's threshold folds
// rows): where the few-rows grid is one workgroup per CU (k = 1) and the 48-column tiles cover
// a group, the shapes with four load waves beside the compute waves and three activation slots
// (1.5B, M = 108-118: 19.1 against 20.2 us); otherwise those of pick_gate_up_shapes.  The
// device still picks by M, so more rows than expected stay correct, only slower.
void pick_gate_up_shapes_few(int F, const GemmCfg* dense, GemmCfg* c) {
    for (int i = 0; i < 3; ++i) c[i] = dense[i];
    const int k = (F + 256 * 64 - 1) / (256 * 64);
    if (k != 1 || dense[0].ntw != 6) return;
    c[0].nbw = 4; c[0].nba = 3; c[0].lw = 4;
    c[1].nbw = 4; c[1].nba = 3; c[1].lw = 4;
    c[2].lw = 4;
}

// The down projection when few rows are expected to recompute (the layer's threshold folds
// rows): where the dense plan has 64-column groups and 96-column groups times the K-splits
// still fit one workgroup per CU, the 96-column groups -- each CU then streams its share of the
// weights in one workgroup with one row chunk (1.5B, M = 108-115: 13.8-14.0 against
// 15.2-15.3 us; at M = 288 the 96-column groups lose 0.3-0.6 us, so the dense plan keeps 64).
// Its K-splits are placed by XCD, so each XCD reads only its own columns of the activations
// (13.4 against 13.75 us; the dense plan lost 2.6 us with it, so it keeps the plain placement).
// The split count is the dense plan's, so the choice never changes a bit.
GemmCfg pick_down_few(const GemmCfg& dense, int n_cols) {
    GemmCfg c = dense;
    if (dense.ntw != 4 || dense.wn != 1 || dense.tm != 2) return c;
    const int groups = (n_cols + 95) / 96;
    if (static_cast<long>(groups) * dense.splits > kNumCUs) return c;
    c.ntw = 6;
    c.nba = 2;                                    // 80 KB: two workgroups per CU above 128 rows
    c.groups = groups;
    c.xcd_split = dense.splits % 8 == 0;
    return c;
}

Layout layout_of(const Dims& d) {
    Layout L;
    // the recompute projections expect about 128 busy rows (folded M); o_proj has all R rows
    L.c_qkv = pick_gemm(GEMM_QKV, d.Nq, d.D, d.R);
    L.c_o = pick_gemm(GEMM_O, d.D, d.Do, d.R);
    L.c_gu = pick_gemm(GEMM_GATE_UP, d.F, d.D, d.R);
    L.gu_multi = d.R > 128;
    if (L.gu_multi) {
        pick_gate_up_shapes(d.F, L.c_gu_shapes, L.gu_upto);
        pick_gate_up_shapes_few(d.F, L.c_gu_shapes, L.c_gu_shapes_few);
    }
    L.c_down = pick_gemm(GEMM_DOWN, d.D, d.F, d.R);
    L.c_down_few = pick_down_few(L.c_down, d.D);
    L.s_qkv = L.c_qkv.splits; L.s_o = L.c_o.splits; L.s_down = L.c_down.splits;
    L.chunk_len = d.P <= 1024 ? 128 : 512;
    L.n_chunks = d.P > 0 ? (d.P + L.chunk_len - 1) / L.chunk_len : 0;
    const size_t R = static_cast<size_t>(d.R);
    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
    L.rho = take(R * 4);
    L.fold = take(R);
    L.inv_rms = take(R * 4);
    L.rec_rows = take(R * 4);
    L.rec_count = take(4);
    L.branch_off = take((static_cast<size_t>(d.nb) + 1) * 4);
    L.row_slot = take(R * 4);
    L.src_branch = take(R * 4);
    L.src_slot = take(R * 4);
    L.xn1 = take(R * d.D * 2);
    L.xn2 = take(R * d.D * 2);
    L.q_c = take(R * d.Hq * d.hd * 2);
    L.k_c = take(R * d.Hkv * d.hd * 2);
    L.v_c = take(R * d.Hkv * d.hd * 2);
    L.attn = take(R * d.Do * 2);
    L.h_mid = take(R * d.D * 2);
    L.act = take(R * d.F * 2);
    size_t part = static_cast<size_t>(L.s_qkv) * R * d.Nq;
    const size_t po = static_cast<size_t>(L.s_o) * R * d.D;
    const size_t pd = static_cast<size_t>(L.s_down) * R * d.D;
    if (po > part) part = po;
    if (pd > part) part = pd;
    L.gemm_part = take(part * 4);
    L.attn_o = take(static_cast<size_t>(L.n_chunks) * R * d.Hq * d.hd * 4);
    L.attn_ml = take(static_cast<size_t>(L.n_chunks) * R * d.Hq * 2 * 4);
    L.total = off;
    return L;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int dev(const void* p) {
    if (!p) return SPECFOLD_ERR_NULL;
    return aligned16(p) ? SPECFOLD_OK : SPECFOLD_ERR_ALIGN;
}

int opt_dev(const void* p) { return p ? dev(p) : SPECFOLD_OK; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

// sizes every entry point relies on
int check_rows_shape(const specfold_shape* s, int max_block) {
    if (!s) return SPECFOLD_ERR_NULL;
    if (s->n_branch < 1 || s->block < 1 || s->hidden < 1) return SPECFOLD_ERR_SHAPE;
    if (s->n_branch > SPECFOLD_MAX_BRANCHES || s->block > max_block) return SPECFOLD_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(s->n_branch) * s->block > (1 << 24)) return SPECFOLD_ERR_UNSUPPORTED;
    if (s->hidden % 64 != 0 || s->hidden > SPECFOLD_MAX_HIDDEN) return SPECFOLD_ERR_UNSUPPORTED;
    if (!(s->rms_eps >= 0.f) || !std::isfinite(s->rms_eps)) return SPECFOLD_ERR_SHAPE;
    return SPECFOLD_OK;
}

// full layer sizes (attention and projections)
int check_layer_shape(const specfold_shape* s) {
    int e = check_rows_shape(s, SPECFOLD_MAX_BLOCK);
    if (e) return e;
    if (s->n_q_heads < 1 || s->n_kv_heads < 1 || s->head_dim < 1 || s->ffn < 1 || s->prefix_len < 0)
        return SPECFOLD_ERR_SHAPE;
    if (s->n_q_heads % s->n_kv_heads != 0) return SPECFOLD_ERR_SHAPE;
    if (!(s->rope_theta > 0.f) || !std::isfinite(s->rope_theta)) return SPECFOLD_ERR_SHAPE;
    const int hd = s->head_dim;
    if (hd != 16 && hd != 32 && hd != 64 && hd != 128) return SPECFOLD_ERR_UNSUPPORTED;
    if (s->ffn % 64 != 0 || (s->n_q_heads * hd) % 64 != 0) return SPECFOLD_ERR_UNSUPPORTED;
    if (((s->n_q_heads + 2 * s->n_kv_heads) * hd) % 32 != 0) return SPECFOLD_ERR_UNSUPPORTED;
    if ((s->n_q_heads + 2 * s->n_kv_heads) * hd > SPECFOLD_MAX_QKV_WIDTH) return SPECFOLD_ERR_UNSUPPORTED;
    // every weight matrix and activation buffer a GEMM streams must stay below 1 GB (the
    // kernels address them with 32-bit buffer offsets and out-of-range sentinels above 1 GB)
    const int64_t gb = int64_t(1) << 30;
    const int64_t R = static_cast<int64_t>(s->n_branch) * s->block;
    const int64_t nq = static_cast<int64_t>(s->n_q_heads + 2 * s->n_kv_heads) * hd;
    if (4 * static_cast<int64_t>(s->hidden) * s->ffn >= gb || 2 * nq * s->hidden >= gb ||
        2 * static_cast<int64_t>(s->hidden) * s->n_q_heads * hd >= gb || 2 * R * s->ffn >= gb ||
        2 * R * s->hidden >= gb || 2 * R * nq >= gb)
        return SPECFOLD_ERR_UNSUPPORTED;
    // prefix chunk states [n_chunks][R][Hq][hd] fp32 (chunks of 512 past 1024 prefix tokens)
    const int64_t chunks = s->prefix_len <= 1024 ? (s->prefix_len + 127) / 128 : (s->prefix_len + 511) / 512;
    if (4 * chunks * R * s->n_q_heads * hd >= gb) return SPECFOLD_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(s->prefix_len) > (int64_t(1) << 24)) return SPECFOLD_ERR_UNSUPPORTED;
    return SPECFOLD_OK;
}

int check_tree(const int32_t* par, int nb, ParentMap& out) {
    if (!par) return SPECFOLD_ERR_NULL;
    if (par[0] != -1) return SPECFOLD_ERR_TREE;
    out.p[0] = -1;
    for (int i = 1; i < nb; ++i) {
        if (par[i] < 0 || par[i] >= i) return SPECFOLD_ERR_TREE;
        out.p[i] = par[i];
    }
    for (int i = nb; i < kMaxBranches; ++i) out.p[i] = -1;
    return SPECFOLD_OK;
}

int check_ws(const void* ws, size_t ws_bytes, const Layout& L) {
    if (!ws) return SPECFOLD_ERR_WORKSPACE;
    if (!aligned16(ws)) return SPECFOLD_ERR_ALIGN;
    if (ws_bytes < L.total) return SPECFOLD_ERR_WORKSPACE;
    return SPECFOLD_OK;
}

int check_prefix(const specfold_prefix_kv* pf, const Dims& d) {
    if (d.P == 0) return SPECFOLD_OK;
    if (!pf) return SPECFOLD_ERR_NULL;
    int e;
    if ((e = dev(pf->k)) || (e = dev(pf->v))) return e;
    const int64_t st[4] = {pf->k_stride_tok, pf->k_stride_head, pf->v_stride_tok, pf->v_stride_head};
    for (int64_t x : st) {
        if (x < 0) return SPECFOLD_ERR_SHAPE;
        if (x % 8 != 0) return SPECFOLD_ERR_ALIGN;
    }
    if (d.P > 1 && (pf->k_stride_tok == 0 || pf->v_stride_tok == 0)) return SPECFOLD_ERR_SHAPE;
    // the attention kernels address each view with 32-bit offsets below 1 GB
    const int64_t gb = int64_t(1) << 30;
    const int64_t ek = ((d.P - 1) * pf->k_stride_tok + (d.Hkv - 1) * pf->k_stride_head + d.hd) * 2;
    const int64_t ev = ((d.P - 1) * pf->v_stride_tok + (d.Hkv - 1) * pf->v_stride_head + d.hd) * 2;
    if (ek >= gb || ev >= gb) return SPECFOLD_ERR_UNSUPPORTED;
    return SPECFOLD_OK;
}

template <typename T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<uint8_t*>(ws) + off); }

thread_local char g_last_error[256] = "";

int hip_status(hipError_t e) {
    if (e == hipSuccess) return SPECFOLD_OK;
    snprintf(g_last_error, sizeof g_last_error, "%s (%d): %s", hipGetErrorName(e), static_cast<int>(e),
             hipGetErrorString(e));
    return SPECFOLD_ERR_HIP;
}

struct Tracer {
    const specfold_trace* t;
    hipStream_t st;
    int k = 0;
    void begin() {
        if (t && t->events && 2 * k + 1 < t->n_events && t->events[2 * k])
            (void)hipEventRecord(static_cast<hipEvent_t>(t->events[2 * k]), st);
    }
    void end() {
        if (t && t->events && 2 * k + 1 < t->n_events && t->events[2 * k + 1])
            (void)hipEventRecord(static_cast<hipEvent_t>(t->events[2 * k + 1]), st);
        ++k;
    }
};

const char* const kStageNames[] = {
    "gate_rmsnorm", "qkv_gemm_compact_resolve", "qkv_rope_epilogue", "attn_prefix", "attn_block_merge",
    "oproj_gemm", "oproj_residual_rmsnorm", "gate_up_swiglu_gemm", "down_gemm", "down_inherit_epilogue",
};
constexpr int kStages = sizeof(kStageNames) / sizeof(kStageNames[0]);

// ---------------------------------------------------------------- launch sequences (no checks)

// QKV projection of the recompute rows of xn (RMSNorm'd rows): rows come from a device list
// (rec_rows/rec_count) or, when fc is given, from the fold flags compacted in the GEMM itself.
hipError_t run_qkv(const Dims& d, const Layout& L, const uint16_t* xn, const int32_t* rec_rows,
                   const int32_t* rec_count, const uint16_t* w_qkv, uint16_t* q_c, uint16_t* k_c, uint16_t* v_c,
                   void* ws, hipStream_t st, Tracer* tr, const GemmArgs* fc) {
    GemmArgs g = fc ? *fc : GemmArgs{};
    g.A = xn; g.lda = d.D; g.a_rows = rec_rows; g.a_row_limit = d.R; g.m_count = rec_count;
    g.m_cap = d.R; g.W = w_qkv; g.K = d.D; g.Nout = d.Nq;
    g.partial = at<float>(ws, L.gemm_part);
    if (tr) tr->begin();
    hipError_t e = launch_gemm(g, L.c_qkv, st);
    if (tr) tr->end();
    if (e != hipSuccess) return e;
    QkvEpiArgs q{};
    q.part = g.partial; q.splits = L.s_qkv; q.m_cap = d.R; q.m_count = rec_count; q.rec_rows = rec_rows;
    q.R = d.R; q.N = d.N; q.Hq = d.Hq; q.Hkv = d.Hkv; q.hd = d.hd; q.P = d.P;
    for (int j = 0; j < d.hd / 2; ++j)
        q.inv_freq[j] = std::pow(static_cast<double>(d.theta), -2.0 * j / static_cast<double>(d.hd));
    q.q_c = q_c; q.k_c = k_c; q.v_c = v_c;
    if (tr) tr->begin();
    e = launch_qkv_epilogue(q, st);
    if (tr) tr->end();
    return e;
}

hipError_t run_attention(const Dims& d, const Layout& L, const uint16_t* q_c, const uint16_t* k_c,
                         const uint16_t* v_c, const int32_t* rec_count, const int32_t* src_slot,
                         const specfold_prefix_kv* pf, uint16_t* attn, float* lse, void* ws,
                         hipStream_t st, Tracer* tr, int plan_rows = 0) {
    AttnArgs a{};
    a.plan_rows = plan_rows;
    a.q_c = q_c; a.k_c = k_c; a.v_c = v_c; a.m_count = rec_count; a.m_cap = d.R; a.src_slot = src_slot;
    a.nb = d.nb; a.N = d.N; a.Hq = d.Hq; a.Hkv = d.Hkv; a.hd = d.hd; a.P = d.P;
    if (d.P > 0) {
        a.pk = pf->k; a.pv = pf->v;
        a.pk_st = pf->k_stride_tok; a.pk_sh = pf->k_stride_head;
        a.pv_st = pf->v_stride_tok; a.pv_sh = pf->v_stride_head;
    }
    a.chunk_len = L.chunk_len; a.n_chunks = L.n_chunks;
    a.part_o = at<float>(ws, L.attn_o); a.part_ml = at<float>(ws, L.attn_ml);
    a.attn = attn; a.lse = lse;
    a.scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(d.hd)));
    if (tr) tr->begin();
    hipError_t e = launch_attn_prefix(a, st);
    if (tr) tr->end();
    if (e != hipSuccess) return e;
    if (tr) tr->begin();
    e = launch_attn_block(a, st);
    if (tr) tr->end();
    return e;
}

hipError_t run_out_proj(const Dims& d, const Layout& L, const uint16_t* attn, const uint16_t* H,
                        const uint16_t* w_o, uint16_t* h_mid, const uint16_t* ln2, uint16_t* xn2, void* ws,
                        hipStream_t st, Tracer* tr) {
    GemmArgs g{};
    g.A = attn; g.lda = d.Do; g.a_rows = nullptr; g.a_row_limit = d.R; g.m_count = nullptr;
    g.m_fixed = d.R; g.m_cap = d.R; g.W = w_o; g.K = d.Do; g.Nout = d.D;
    g.partial = at<float>(ws, L.gemm_part);
    if (tr) tr->begin();
    hipError_t e = launch_gemm(g, L.c_o, st);
    if (tr) tr->end();
    if (e != hipSuccess) return e;
    if (tr) tr->begin();
    e = launch_oproj_epilogue(g.partial, L.s_o, d.R, d.D, H, h_mid, ln2, d.eps, xn2, st);
    if (tr) tr->end();
    return e;
}

// FFN of the recompute rows of xn2 (RMSNorm'd h_mid) + fold-inherit + residual.
// Above 128 rows the gate/up projection is one launch with three tile shapes, the device picking
// by the recompute count (layout_of).  Every shape forms each output's sum in the same order, so
// the choice never changes a bit.
hipError_t run_ffn(const Dims& d, const Layout& L, const uint16_t* xn2, const uint16_t* h_mid,
                   const int32_t* rec_rows, const int32_t* rec_count, const int32_t* src_slot,
                   const uint16_t* w_gate_up, const uint16_t* w_down, uint16_t* H_out, void* ws, hipStream_t st,
                   Tracer* tr, bool few_rows = false) {
    GemmArgs g{};
    g.A = xn2; g.lda = d.D; g.a_rows = rec_rows; g.a_row_limit = d.R; g.m_count = rec_count;
    g.m_cap = d.R; g.W = w_gate_up; g.K = d.D; g.Nout = 2 * d.F;
    g.act = at<uint16_t>(ws, L.act); g.F = d.F;
    if (tr) tr->begin();
    hipError_t e = L.gu_multi ? launch_gemm_shapes(g, few_rows ? L.c_gu_shapes_few : L.c_gu_shapes, L.gu_upto, st)
                              : launch_gemm(g, L.c_gu, st);
    if (tr) tr->end();
    if (e != hipSuccess) return e;
    GemmArgs h{};
    h.A = g.act; h.lda = d.F; h.a_rows = nullptr; h.a_row_limit = d.R; h.m_count = rec_count;
    h.m_cap = d.R; h.W = w_down; h.K = d.F; h.Nout = d.D;
    h.partial = at<float>(ws, L.gemm_part);
    if (tr) tr->begin();
    e = launch_gemm(h, few_rows ? L.c_down_few : L.c_down, st);
    if (tr) tr->end();
    if (e != hipSuccess) return e;
    if (tr) tr->begin();
    e = launch_down_epilogue(h.partial, L.s_down, d.R, rec_count, rec_rows, src_slot, d.nb, d.N, d.D, h_mid,
                             H_out, st);
    if (tr) tr->end();
    return e;
}

// Checks of specfold_verify_layer's arguments other than the shape and the workspace.
int check_layer_args(const Dims& d, const int32_t* parent_host, const specfold_layer_weights* w,
                     const specfold_prefix_kv* prefix, const specfold_bf16* H_in, const specfold_bf16* H_out,
                     const specfold_layer_stats* stats, ParentMap& par) {
    int e;
    if ((e = check_tree(parent_host, d.nb, par))) return e;
    if (!w) return SPECFOLD_ERR_NULL;
    if ((e = dev(w->ln1)) || (e = dev(w->w_qkv)) || (e = dev(w->w_o)) || (e = dev(w->ln2)) ||
        (e = dev(w->w_gate_up)) || (e = dev(w->w_down)) || (e = dev(H_in)) || (e = dev(H_out)))
        return e;
    if (stats && ((e = opt_dev(stats->rho)) || (e = opt_dev(stats->fold)) || (e = opt_dev(stats->rec_count)) ||
                  (e = opt_dev(stats->src_slot))))
        return e;
    if ((e = check_prefix(prefix, d))) return e;
    const size_t nh = static_cast<size_t>(d.R) * d.D * 2;
    if (overlaps(H_out, nh, H_in, nh)) return SPECFOLD_ERR_ALIAS;
    return SPECFOLD_OK;
}

// The launch sequence of one layer on workspace ws (checked by the caller).
int launch_layer(const Dims& d, const Layout& L, const ParentMap& par, const specfold_layer_weights* w,
                 const specfold_prefix_kv* prefix, const specfold_bf16* H_in, float delta, specfold_bf16* H_out,
                 specfold_layer_stats* stats, const specfold_trace* trace, void* ws, hipStream_t st) {
    Tracer tr{trace, st};
    GateParams g{};
    g.H = H_in; g.par = par; g.nb = d.nb; g.N = d.N; g.D = d.D; g.delta = delta; g.rho_in = nullptr;
    g.rho = (stats && stats->rho) ? stats->rho : at<float>(ws, L.rho);
    g.fold = at<uint8_t>(ws, L.fold); g.inv_rms = at<float>(ws, L.inv_rms); g.eps = d.eps;
    g.ln = w->ln1; g.xn = at<uint16_t>(ws, L.xn1); g.fold_copy = stats ? stats->fold : nullptr;
    tr.begin();
    hipError_t he = launch_gate(g, st);
    tr.end();
    if (he != hipSuccess) return hip_status(he);

    // the QKV GEMM compacts the fold flags itself and publishes the recompute list and sources
    int32_t* rec_rows = at<int32_t>(ws, L.rec_rows);
    int32_t* rec_count = at<int32_t>(ws, L.rec_count);
    int32_t* src_slot = at<int32_t>(ws, L.src_slot);
    GemmArgs fc{};
    fc.fc_fold = g.fold; fc.fc_R = d.R; fc.fc_N = d.N; fc.fc_nb = d.nb; fc.fc_par = par;
    fc.fc_rec_rows = rec_rows; fc.fc_rec_count = rec_count; fc.fc_branch_off = at<int32_t>(ws, L.branch_off);
    fc.fc_row_slot = at<int32_t>(ws, L.row_slot); fc.fc_src_branch = at<int32_t>(ws, L.src_branch);
    fc.fc_src_slot = src_slot;
    fc.fc_count_copy = stats ? stats->rec_count : nullptr;
    fc.fc_src_slot_copy = stats ? stats->src_slot : nullptr;

    uint16_t* q_c = at<uint16_t>(ws, L.q_c);
    uint16_t* k_c = at<uint16_t>(ws, L.k_c);
    uint16_t* v_c = at<uint16_t>(ws, L.v_c);
    uint16_t* attn = at<uint16_t>(ws, L.attn);
    uint16_t* h_mid = at<uint16_t>(ws, L.h_mid);
    uint16_t* xn2 = at<uint16_t>(ws, L.xn2);
    if ((he = run_qkv(d, L, g.xn, rec_rows, rec_count, w->w_qkv, q_c, k_c, v_c, ws, st, &tr, &fc)) != hipSuccess)
        return hip_status(he);
    // a threshold that folds only exact copies (delta <= 0, or NaN) leaves every row recomputing
    const int plan_rows = delta > 0.0f ? (d.R + 1) / 2 : d.R;
    if ((he = run_attention(d, L, q_c, k_c, v_c, rec_count, src_slot, prefix, attn, nullptr, ws, st, &tr,
                            plan_rows)) != hipSuccess)
        return hip_status(he);
    if ((he = run_out_proj(d, L, attn, H_in, w->w_o, h_mid, w->ln2, xn2, ws, st, &tr)) != hipSuccess)
        return hip_status(he);
    if ((he = run_ffn(d, L, xn2, h_mid, rec_rows, rec_count, src_slot, w->w_gate_up, w->w_down, H_out, ws, st,
                      &tr, delta > 0.0f)) != hipSuccess)
        return hip_status(he);
    return SPECFOLD_OK;
}

// ---------------------------------------------------------------- allocation-free scratch
// specfold_verify_layer_noalloc's workspace: a file-scope device array, so callers that cannot
// allocate (graph capture, serving loops) need no workspace.  Each device holds its own copy
// at its own address; host code never uses the array's name as an address (on the host it is
// only a stand-in for the symbol): the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept.  Every call on a device shares the
// array, so calls that overlap on one device race.
__device__ __align__(256) uint8_t scratch[SPECFOLD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// the current device's copy of `scratch` (looked up on the first call on that device)
int device_scratch(void** out) {
    int device = -1;
    hipError_t he = hipGetDevice(&device);
    if (he != hipSuccess) return hip_status(he);
    if (device < 0 || device >= kMaxDevices) return SPECFOLD_ERR_UNSUPPORTED;
    void* p = g_scratch[device].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[device].load(std::memory_order_relaxed);
        if (!p) {
            he = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (he != hipSuccess) return hip_status(he);
            if (!p || !aligned16(p)) return SPECFOLD_ERR_HIP;
            g_scratch[device].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return SPECFOLD_OK;
}

}  // namespace


// ---------------------------------------------------------------- LM head layout
// Vocabulary pieces: the GEMM addresses its weights with 32-bit buffer offsets below 1 GB, so
// W_lm streams in pieces of at most this many rows (a multiple of 64).
struct HeadLayout {
    GemmCfg cfg;
    int piece;                   // vocabulary rows per launch
    int groups;                  // column groups over all pieces
    size_t xn, val, idx, total;
};

int head_piece_rows(int D) {
    const int64_t rows = ((int64_t(1) << 30) - 1) / (2 * static_cast<int64_t>(D));
    return static_cast<int>(rows / 64 * 64);
}

HeadLayout head_layout(const specfold_shape& s, int V) {
    HeadLayout h{};
    const int R = s.n_branch * s.block, D = s.hidden;
    // 128 columns by 128 rows per workgroup (64 x 64 for small R), no K split: every column
    // group reads all R activation rows and every row chunk the group's weights, so the widest
    // tile re-reads least (M = 288, V = 151936: 293 against 311 us with 64-column groups)
    h.cfg = R > 64 ? GemmCfg{8, 1, 2, 1, 3, 2, 0, 1, false, 1, true} : GemmCfg{4, 1, 1, 1, 3, 2, 0, 1, false, 1, true};
    h.piece = head_piece_rows(D);
    const int cap = gemm_group_cols(h.cfg);
    h.groups = 0;
    for (int v0 = 0; v0 < V; v0 += h.piece) {
        const int n = V - v0 < h.piece ? V - v0 : h.piece;
        h.groups += (n + cap - 1) / cap;
    }
    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
    h.xn = take(static_cast<size_t>(R) * D * 2);
    h.val = take(static_cast<size_t>(h.groups) * R * 4);
    h.idx = take(static_cast<size_t>(h.groups) * R * 4);
    h.total = off;
    return h;
}

int check_head_shape(const specfold_shape* s, int32_t vocab) {
    int e = check_rows_shape(s, SPECFOLD_MAX_BLOCK);
    if (e) return e;
    if (vocab < 1) return SPECFOLD_ERR_SHAPE;
    if (2 * static_cast<int64_t>(s->n_branch) * s->block * s->hidden >= (int64_t(1) << 30))
        return SPECFOLD_ERR_UNSUPPORTED;
    return SPECFOLD_OK;
}

extern "C" {

int specfold_version(void) { return SPECFOLD_VERSION; }

const char* specfold_last_error(void) { return g_last_error; }

const char* specfold_status_str(int status) {
    switch (status) {
        case SPECFOLD_OK: return "ok";
        case SPECFOLD_ERR_NULL: return "required pointer is NULL";
        case SPECFOLD_ERR_SHAPE: return "sizes out of range or inconsistent";
        case SPECFOLD_ERR_TREE: return "invalid parent map (need par[0] = -1 and 0 <= par[i] < i)";
        case SPECFOLD_ERR_ALIGN: return "device pointer or stride not 16-byte aligned";
        case SPECFOLD_ERR_WORKSPACE: return "workspace missing or too small";
        case SPECFOLD_ERR_UNSUPPORTED: return "shape outside the implemented kernels";
        case SPECFOLD_ERR_ALIAS: return "output overlaps an input";
        case SPECFOLD_ERR_HIP: return "HIP runtime rejected a launch";
        default: return "unknown status";
    }
}

size_t specfold_workspace_bytes(const specfold_shape* shape) {
    if (check_layer_shape(shape) != SPECFOLD_OK) return 0;
    return layout_of(dims_of(*shape)).total;
}

int specfold_stage_count(void) { return kStages; }

const char* specfold_stage_name(int stage) {
    return (stage >= 0 && stage < kStages) ? kStageNames[stage] : nullptr;
}

int specfold_event_create(void** event) {
    if (!event) return SPECFOLD_ERR_NULL;
    hipEvent_t e;
    // timing only: no system-scope fence at record, so the event does not add a cache
    // writeback/invalidate to the launch it brackets
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return SPECFOLD_ERR_HIP;
    *event = e;
    return SPECFOLD_OK;
}

int specfold_event_destroy(void* event) {
    if (!event) return SPECFOLD_ERR_NULL;
    return hip_status(hipEventDestroy(static_cast<hipEvent_t>(event)));
}

int specfold_event_elapsed_ms(void* start, void* stop, float* ms) {
    if (!start || !stop || !ms) return SPECFOLD_ERR_NULL;
    return hip_status(hipEventElapsedTime(ms, static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(stop)));
}

int specfold_gate(const specfold_shape* shape, const int32_t* parent_host, const specfold_bf16* H,
                  float delta, const float* rho_in, float* rho, uint8_t* fold, float* inv_rms,
                  void* stream) {
    int e = check_rows_shape(shape, kMaxGateBlock);
    if (e) return e;
    ParentMap par;
    if ((e = check_tree(parent_host, shape->n_branch, par))) return e;
    const bool need_h = (rho_in == nullptr) || (inv_rms != nullptr);
    if (need_h && (e = dev(H))) return e;
    // the gate addresses H with 32-bit buffer offsets and reads zeros past 1 GB (rows past the
    // end, the parent of a main row), so H must stay below 1 GB
    if (need_h && 2 * static_cast<int64_t>(shape->n_branch) * shape->block * shape->hidden >= (int64_t(1) << 30))
        return SPECFOLD_ERR_UNSUPPORTED;
    if ((e = opt_dev(rho_in)) || (e = dev(rho)) || (e = dev(fold)) || (e = opt_dev(inv_rms))) return e;
    const size_t R = static_cast<size_t>(shape->n_branch) * shape->block;
    if (overlaps(rho, R * 4, fold, R) || (inv_rms && (overlaps(inv_rms, R * 4, rho, R * 4) ||
                                                      overlaps(inv_rms, R * 4, fold, R))))
        return SPECFOLD_ERR_ALIAS;
    if (need_h && (overlaps(H, R * shape->hidden * 2, rho, R * 4) || overlaps(H, R * shape->hidden * 2, fold, R)))
        return SPECFOLD_ERR_ALIAS;
    GateParams p{};
    p.H = H; p.par = par; p.nb = shape->n_branch; p.N = shape->block; p.D = shape->hidden;
    p.delta = delta; p.rho_in = rho_in; p.rho = rho; p.fold = fold; p.inv_rms = inv_rms;
    p.eps = shape->rms_eps; p.ln = nullptr; p.xn = nullptr; p.fold_copy = nullptr;
    return hip_status(launch_gate(p, static_cast<hipStream_t>(stream)));
}

size_t specfold_compact_workspace_bytes(const specfold_shape* shape) {
    if (check_rows_shape(shape, kMaxGateBlock) != SPECFOLD_OK) return 0;
    return compact_workspace_bytes(shape->n_branch * shape->block);
}

int specfold_compact(const specfold_shape* shape, const uint8_t* fold, int32_t* rec_rows,
                     int32_t* rec_count, int32_t* branch_off, int32_t* row_slot, void* ws, size_t ws_bytes,
                     void* stream) {
    int e = check_rows_shape(shape, kMaxGateBlock);
    if (e) return e;
    if ((e = dev(fold)) || (e = dev(rec_rows)) || (e = dev(rec_count)) || (e = dev(branch_off)) ||
        (e = dev(row_slot)))
        return e;
    const size_t R = static_cast<size_t>(shape->n_branch) * shape->block;
    const size_t need = compact_workspace_bytes(static_cast<int>(R));
    if (need > 0) {
        if (!ws || ws_bytes < need) return SPECFOLD_ERR_WORKSPACE;
        if (!aligned16(ws)) return SPECFOLD_ERR_ALIGN;
    }
    const size_t nbo = (static_cast<size_t>(shape->n_branch) + 1) * 4;
    if (overlaps(rec_rows, R * 4, row_slot, R * 4) || overlaps(rec_rows, R * 4, branch_off, nbo) ||
        overlaps(row_slot, R * 4, branch_off, nbo) || overlaps(rec_count, 4, rec_rows, R * 4) ||
        overlaps(rec_count, 4, row_slot, R * 4) || overlaps(rec_count, 4, branch_off, nbo) ||
        overlaps(fold, R, rec_rows, R * 4) || overlaps(fold, R, row_slot, R * 4))
        return SPECFOLD_ERR_ALIAS;
    if (need > 0) {
        const void* outs[5] = {fold, rec_rows, rec_count, branch_off, row_slot};
        const size_t sizes[5] = {R, R * 4, 4, nbo, R * 4};
        for (int k = 0; k < 5; ++k)
            if (overlaps(ws, need, outs[k], sizes[k])) return SPECFOLD_ERR_ALIAS;
    }
    CompactParams p{};
    p.fold = fold; p.R = static_cast<int>(R); p.N = shape->block; p.nb = shape->n_branch;
    p.rec_rows = rec_rows; p.rec_count = rec_count; p.branch_off = branch_off; p.row_slot = row_slot;
    return hip_status(launch_compact(p, need > 0 ? ws : nullptr, static_cast<hipStream_t>(stream)));
}

int specfold_resolve_sources(const specfold_shape* shape, const int32_t* parent_host,
                             const uint8_t* fold, const int32_t* row_slot, int32_t* src_branch,
                             int32_t* src_slot, void* stream) {
    int e = check_rows_shape(shape, kMaxGateBlock);
    if (e) return e;
    ParentMap par;
    if ((e = check_tree(parent_host, shape->n_branch, par))) return e;
    if ((e = dev(fold)) || (e = dev(row_slot)) || (e = dev(src_branch)) || (e = dev(src_slot))) return e;
    const size_t R = static_cast<size_t>(shape->n_branch) * shape->block;
    if (overlaps(src_branch, R * 4, src_slot, R * 4) || overlaps(src_branch, R * 4, row_slot, R * 4) ||
        overlaps(src_slot, R * 4, row_slot, R * 4) || overlaps(src_branch, R * 4, fold, R) ||
        overlaps(src_slot, R * 4, fold, R))
        return SPECFOLD_ERR_ALIAS;
    ResolveParams p{};
    p.fold = fold; p.par = par; p.nb = shape->n_branch; p.N = shape->block; p.R = static_cast<int>(R);
    p.row_slot = row_slot; p.src_branch = src_branch; p.src_slot = src_slot;
    return hip_status(launch_resolve(p, static_cast<hipStream_t>(stream)));
}

int specfold_sparse_qkv(const specfold_shape* shape, const specfold_bf16* H, const float* inv_rms,
                        const int32_t* rec_rows, const int32_t* rec_count, const specfold_bf16* ln1,
                        const specfold_bf16* w_qkv, specfold_bf16* q_c, specfold_bf16* k_c,
                        specfold_bf16* v_c, void* ws, size_t ws_bytes, void* stream) {
    int e = check_layer_shape(shape);
    if (e) return e;
    const Dims d = dims_of(*shape);
    const Layout L = layout_of(d);
    if ((e = dev(H)) || (e = dev(inv_rms)) || (e = dev(rec_rows)) || (e = dev(rec_count)) || (e = dev(ln1)) ||
        (e = dev(w_qkv)) || (e = dev(q_c)) || (e = dev(k_c)) || (e = dev(v_c)))
        return e;
    if ((e = check_ws(ws, ws_bytes, L))) return e;
    const size_t R = d.R, nq = R * d.Hq * d.hd * 2, nk = R * d.Hkv * d.hd * 2;
    if (overlaps(q_c, nq, k_c, nk) || overlaps(q_c, nq, v_c, nk) || overlaps(k_c, nk, v_c, nk) ||
        overlaps(q_c, nq, H, R * d.D * 2) || overlaps(k_c, nk, H, R * d.D * 2) || overlaps(v_c, nk, H, R * d.D * 2) ||
        overlaps(ws, ws_bytes, q_c, nq) || overlaps(ws, ws_bytes, k_c, nk) || overlaps(ws, ws_bytes, v_c, nk))
        return SPECFOLD_ERR_ALIAS;
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint16_t* xn = at<uint16_t>(ws, L.xn1);
    hipError_t he = launch_row_norm(H, d.R, d.D, inv_rms, d.eps, ln1, xn, st);
    if (he != hipSuccess) return hip_status(he);
    return hip_status(run_qkv(d, L, xn, rec_rows, rec_count, w_qkv, q_c, k_c, v_c, ws, st, nullptr, nullptr));
}

int specfold_folded_attention(const specfold_shape* shape, const specfold_bf16* q_c,
                              const specfold_bf16* k_c, const specfold_bf16* v_c,
                              const int32_t* rec_rows, const int32_t* rec_count, const int32_t* src_slot,
                              const specfold_prefix_kv* prefix, specfold_bf16* attn, float* lse,
                              void* ws, size_t ws_bytes, void* stream) {
    int e = check_layer_shape(shape);
    if (e) return e;
    const Dims d = dims_of(*shape);
    const Layout L = layout_of(d);
    (void)rec_rows;
    if ((e = dev(q_c)) || (e = dev(k_c)) || (e = dev(v_c)) || (e = dev(rec_count)) || (e = dev(src_slot)) ||
        (e = dev(attn)) || (e = opt_dev(lse)))
        return e;
    if ((e = check_prefix(prefix, d))) return e;
    if ((e = check_ws(ws, ws_bytes, L))) return e;
    const size_t R = d.R, na = R * d.Do * 2;
    if (overlaps(attn, na, q_c, R * d.Hq * d.hd * 2) || overlaps(attn, na, k_c, R * d.Hkv * d.hd * 2) ||
        overlaps(attn, na, v_c, R * d.Hkv * d.hd * 2) || overlaps(attn, na, ws, ws_bytes) ||
        (lse && (overlaps(lse, R * d.Hq * 4, attn, na) || overlaps(lse, R * d.Hq * 4, ws, ws_bytes))))
        return SPECFOLD_ERR_ALIAS;
    return hip_status(run_attention(d, L, q_c, k_c, v_c, rec_count, src_slot, prefix, attn, lse, ws,
                                    static_cast<hipStream_t>(stream), nullptr));
}

int specfold_out_proj(const specfold_shape* shape, const specfold_bf16* attn, const specfold_bf16* H,
                      const specfold_bf16* w_o, specfold_bf16* h_mid, void* ws, size_t ws_bytes,
                      void* stream) {
    int e = check_layer_shape(shape);
    if (e) return e;
    const Dims d = dims_of(*shape);
    const Layout L = layout_of(d);
    if ((e = dev(attn)) || (e = dev(H)) || (e = dev(w_o)) || (e = dev(h_mid))) return e;
    if ((e = check_ws(ws, ws_bytes, L))) return e;
    const size_t nh = static_cast<size_t>(d.R) * d.D * 2;
    if (overlaps(h_mid, nh, H, nh) || overlaps(h_mid, nh, attn, static_cast<size_t>(d.R) * d.Do * 2) ||
        overlaps(h_mid, nh, ws, ws_bytes))
        return SPECFOLD_ERR_ALIAS;
    return hip_status(run_out_proj(d, L, attn, H, w_o, h_mid, nullptr, nullptr, ws, static_cast<hipStream_t>(stream),
                                   nullptr));
}

int specfold_sparse_ffn(const specfold_shape* shape, const specfold_bf16* h_mid, const int32_t* rec_rows,
                        const int32_t* rec_count, const int32_t* src_slot, const specfold_bf16* ln2,
                        const specfold_bf16* w_gate_up, const specfold_bf16* w_down, specfold_bf16* H_out,
                        void* ws, size_t ws_bytes, void* stream) {
    int e = check_layer_shape(shape);
    if (e) return e;
    const Dims d = dims_of(*shape);
    const Layout L = layout_of(d);
    if ((e = dev(h_mid)) || (e = dev(rec_rows)) || (e = dev(rec_count)) || (e = dev(src_slot)) || (e = dev(ln2)) ||
        (e = dev(w_gate_up)) || (e = dev(w_down)) || (e = dev(H_out)))
        return e;
    if ((e = check_ws(ws, ws_bytes, L))) return e;
    const size_t nh = static_cast<size_t>(d.R) * d.D * 2;
    if (overlaps(H_out, nh, h_mid, nh) || overlaps(H_out, nh, ws, ws_bytes) || overlaps(h_mid, nh, ws, ws_bytes))
        return SPECFOLD_ERR_ALIAS;
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint16_t* xn = at<uint16_t>(ws, L.xn2);
    hipError_t he = launch_row_norm(h_mid, d.R, d.D, nullptr, d.eps, ln2, xn, st);
    if (he != hipSuccess) return hip_status(he);
    return hip_status(run_ffn(d, L, xn, h_mid, rec_rows, rec_count, src_slot, w_gate_up, w_down, H_out, ws, st,
                              nullptr));
}

int specfold_verify_layer(const specfold_shape* shape, const int32_t* parent_host,
                          const specfold_layer_weights* w, const specfold_prefix_kv* prefix,
                          const specfold_bf16* H_in, float delta, specfold_bf16* H_out,
                          specfold_layer_stats* stats, const specfold_trace* trace, void* ws,
                          size_t ws_bytes, void* stream) {
    int e = check_layer_shape(shape);
    if (e) return e;
    const Dims d = dims_of(*shape);
    const Layout L = layout_of(d);
    ParentMap par;
    if ((e = check_layer_args(d, parent_host, w, prefix, H_in, H_out, stats, par))) return e;
    if ((e = check_ws(ws, ws_bytes, L))) return e;
    const size_t nh = static_cast<size_t>(d.R) * d.D * 2;
    if (overlaps(H_out, nh, ws, ws_bytes) || overlaps(H_in, nh, ws, ws_bytes)) return SPECFOLD_ERR_ALIAS;
    return launch_layer(d, L, par, w, prefix, H_in, delta, H_out, stats, trace, ws, static_cast<hipStream_t>(stream));
}

int specfold_verify_layer_noalloc(const specfold_shape* shape, const int32_t* parent_host,
                                  const specfold_layer_weights* w, const specfold_prefix_kv* prefix,
                                  const specfold_bf16* H_in, float delta, specfold_bf16* H_out,
                                  specfold_layer_stats* stats, const specfold_trace* trace, void* stream) {
    int e = check_layer_shape(shape);
    if (e) return e;
    const Dims d = dims_of(*shape);
    const Layout L = layout_of(d);
    ParentMap par;
    if ((e = check_layer_args(d, parent_host, w, prefix, H_in, H_out, stats, par))) return e;
    if (L.total > SPECFOLD_NOALLOC_SCRATCH_BYTES) return SPECFOLD_ERR_WORKSPACE;
    void* ws = nullptr;
    if ((e = device_scratch(&ws))) return e;
    return launch_layer(d, L, par, w, prefix, H_in, delta, H_out, stats, trace, ws, static_cast<hipStream_t>(stream));
}

size_t specfold_head_workspace_bytes(const specfold_shape* shape, int32_t vocab) {
    if (check_head_shape(shape, vocab)) return 0;
    return head_layout(*shape, vocab).total;
}

int specfold_embed(const specfold_shape* shape, const int32_t* tokens, const specfold_bf16* E, int32_t vocab,
                   specfold_bf16* H, void* stream) {
    int e = check_rows_shape(shape, SPECFOLD_MAX_BLOCK);
    if (e) return e;
    if (vocab < 1) return SPECFOLD_ERR_SHAPE;
    if ((e = dev(tokens)) || (e = dev(E)) || (e = dev(H))) return e;
    const int R = shape->n_branch * shape->block, D = shape->hidden;
    if (overlaps(H, static_cast<size_t>(R) * D * 2, E, static_cast<size_t>(vocab) * D * 2) ||
        overlaps(H, static_cast<size_t>(R) * D * 2, tokens, static_cast<size_t>(R) * 4))
        return SPECFOLD_ERR_ALIAS;
    return hip_status(launch_embed(tokens, R, E, vocab, D, H, static_cast<hipStream_t>(stream)));
}

int specfold_lm_head(const specfold_shape* shape, const specfold_bf16* H, const specfold_bf16* ln_f,
                     const specfold_bf16* w_lm, int32_t vocab, int32_t* token, float* logit, void* ws,
                     size_t ws_bytes, void* stream) {
    int e = check_head_shape(shape, vocab);
    if (e) return e;
    if ((e = dev(H)) || (e = dev(ln_f)) || (e = dev(w_lm)) || (e = dev(token)) || (e = dev(logit))) return e;
    const HeadLayout L = head_layout(*shape, vocab);
    if (!ws) return SPECFOLD_ERR_NULL;
    if (ws_bytes < L.total) return SPECFOLD_ERR_WORKSPACE;
    if ((e = dev(ws))) return e;
    const int R = shape->n_branch * shape->block, D = shape->hidden;
    if (overlaps(ws, ws_bytes, H, static_cast<size_t>(R) * D * 2) || overlaps(token, static_cast<size_t>(R) * 4, logit,
                                                                              static_cast<size_t>(R) * 4))
        return SPECFOLD_ERR_ALIAS;
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint16_t* xn = at<uint16_t>(ws, L.xn);
    float* val = at<float>(ws, L.val);
    int32_t* idx = at<int32_t>(ws, L.idx);
    hipError_t he = launch_rmsnorm_rows(H, R, D, ln_f, shape->rms_eps, xn, st);
    if (he != hipSuccess) return hip_status(he);
    const int cap = gemm_group_cols(L.cfg);
    int gbase = 0;
    for (int v0 = 0; v0 < vocab; v0 += L.piece) {
        const int n = vocab - v0 < L.piece ? vocab - v0 : L.piece;
        GemmCfg c = L.cfg;
        c.groups = (n + cap - 1) / cap;
        GemmArgs g{};
        g.A = xn; g.lda = D; g.a_rows = nullptr; g.a_row_limit = R; g.m_count = nullptr; g.m_fixed = R;
        g.m_cap = R; g.W = w_lm + static_cast<size_t>(v0) * D; g.K = D; g.Nout = n;
        g.arg_val = val; g.arg_idx = idx; g.col_base = v0; g.group_base = gbase;
        if ((he = launch_gemm(g, c, st)) != hipSuccess) return hip_status(he);
        gbase += c.groups;
    }
    return hip_status(launch_argmax_merge(val, idx, L.groups, R, token, logit, st));
}
}  // extern "C"
