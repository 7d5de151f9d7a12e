// The pages' attention-state correction for folded rows [SpecFold summary, App. B, §A.1,
// §A.3], built as a comparison variant (see correction.h).  One 64-lane wave owns one
// (row, query head) and a workgroup the query heads of one KV head; lane l owns dimensions l
// and l + 64 of the head's numerator (head_dim <= 128), scores are one key per lane.  Scores
// are kept in base-2 units (score * log2(e) / sqrt(d)); the state of a (row, head) is
// (m, l, acc[d]) in fp32.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "correction.h"

namespace {

constexpr int kWave = 64;
constexpr int kMaxDim = 2 * kWave;

struct Args {
    int nb, N, Hq, Hkv, hd, P;
    float scale_log2;
    const uint16_t* q_c;
    const uint16_t* k_c;
    const uint16_t* v_c;
    const int32_t* rec_rows;
    const int32_t* rec_count;
    const int32_t* src_slot;
    const uint8_t* fold;
    const uint16_t* pk;
    const uint16_t* pv;
    int64_t pk_st, pk_sh, pv_st, pv_sh;
    float* state;
    const float* cstate;
    float* out;
    uint64_t mask;
    int32_t par[SPECFOLD_MAX_BRANCHES];
};

__device__ __forceinline__ float bf(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// the lane's two elements of a head_dim vector (zero past head_dim)
__device__ __forceinline__ void load2(const uint16_t* p, int hd, int lane, float& x0, float& x1) {
    x0 = lane < hd ? bf(p[lane]) : 0.f;
    x1 = lane + kWave < hd ? bf(p[lane + kWave]) : 0.f;
}

__device__ __forceinline__ float* state_of(float* s, const Args& a, int row, int h) {
    return s + (static_cast<size_t>(row) * a.Hq + h) * (a.hd + 2);
}

__device__ __forceinline__ const uint16_t* kv_row(const uint16_t* base, const Args& a, int slot, int g) {
    return base + (static_cast<size_t>(slot) * a.Hkv + g) * a.hd;
}

constexpr int kChunk = 64;                  // keys staged in LDS per step of the fresh pass
constexpr int kMaxGroup = 8;                // query heads per KV head (one wave each)

// lane's head_dim-long dot product of the query held in qv (d/2 packed bf16 pairs, the same in
// every lane) with row `row` of a K tile in LDS whose 16-byte chunks are rotated by the row
// (chunk c of row r sits at position (c + r) % (d / 8)), so the 64 lanes of a wave read 64
// different rows without bank conflicts
template <int D>
__device__ __forceinline__ float dot_tile(const uint32_t* qv, const uint4* tile, int row) {
    constexpr int nc = D >> 3;
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < nc; ++c) {
        const uint4 kv = tile[row * nc + ((c + row) % nc)];
        const uint32_t w[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t qq = qv[4 * c + t];
            acc += __uint_as_float(qq << 16) * __uint_as_float(w[t] << 16);
            acc += __uint_as_float(qq & 0xffff0000u) * __uint_as_float(w[t] & 0xffff0000u);
        }
    }
    return acc;
}

// lane's dot product of the packed query with a key row in global memory (16-byte loads)
template <int D>
__device__ __forceinline__ float dot_global(const uint32_t* qv, const uint16_t* k) {
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < (D >> 3); ++c) {
        const uint4 kv = *reinterpret_cast<const uint4*>(k + 8 * c);
        const uint32_t w[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t qq = qv[4 * c + t];
            acc += __uint_as_float(qq << 16) * __uint_as_float(w[t] << 16);
            acc += __uint_as_float(qq & 0xffff0000u) * __uint_as_float(w[t] & 0xffff0000u);
        }
    }
    return acc;
}

template <int D>
__device__ __forceinline__ void load_query(uint32_t* qv, const uint16_t* q) {
#pragma unroll
    for (int t = 0; t < (D >> 1); ++t) qv[t] = *reinterpret_cast<const uint32_t*>(q + 2 * t);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// grid (R, Hkv): blockIdx.x = slot, blockIdx.y = KV head g; wave w = query head g * G + w.
// Keys [prefix ; block] move through LDS in chunks of 64 shared by the group's G heads; lane j
// scores key j of the chunk, the wave folds the chunk into its running state, and lane l
// accumulates dimensions l and l + 64 over the chunk's keys.
template <int D>
__global__ __launch_bounds__(kWave * kMaxGroup) void fresh_kernel(const Args a) {
    __shared__ uint4 sK[kChunk * kMaxDim / 8];
    __shared__ uint16_t sV[kChunk * kMaxDim];
    __shared__ float sP[kMaxGroup][kChunk];
    __shared__ int sBad;
    constexpr int d = D, nc = D >> 3;
    const int R = a.nb * a.N, G = a.Hq / a.Hkv;
    const int slot = blockIdx.x, g = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
    int M = a.rec_count[0];
    M = M < 0 ? 0 : (M > R ? R : M);
    if (slot >= M) return;
    const int row = a.rec_rows[slot];
    if (row < 0 || row >= R) return;
    const int i = row / a.N, h = g * G + w;
    if (tid == 0) sBad = 0;
    uint32_t qv[D / 2];
    load_query<D>(qv, a.q_c + (static_cast<size_t>(slot) * a.Hq + h) * d);
    float m = -INFINITY, l = 0.f, c0 = 0.f, c1 = 0.f;
    const int nkeys = a.P + a.N;
    for (int k0 = 0; k0 < nkeys; k0 += kChunk) {
        const int nk = min(kChunk, nkeys - k0);
        __syncthreads();                          // the previous chunk is consumed
        for (int e = tid; e < nk * nc; e += kWave * G) {
            const int r = e / nc, c = e - r * nc, t = k0 + r;
            const uint16_t *kp, *vp;
            if (t < a.P) {
                kp = a.pk + t * a.pk_st + g * a.pk_sh;
                vp = a.pv + t * a.pv_st + g * a.pv_sh;
            } else {
                const int s = a.src_slot[i * a.N + (t - a.P)];
                if (s < 0 || s >= M) { sBad = 1; continue; }
                kp = kv_row(a.k_c, a, s, g);
                vp = kv_row(a.v_c, a, s, g);
            }
            sK[r * nc + ((c + r) % nc)] = *reinterpret_cast<const uint4*>(kp + 8 * c);
            *reinterpret_cast<uint4*>(sV + r * d + 8 * c) = *reinterpret_cast<const uint4*>(vp + 8 * c);
        }
        __syncthreads();
        const float s = lane < nk ? dot_tile<D>(qv, sK, lane) * a.scale_log2 : -INFINITY;
        const float mn = fmaxf(m, wave_max(s));
        const float r = m == -INFINITY ? 0.f : exp2f(m - mn);
        const float p = lane < nk ? exp2f(s - mn) : 0.f;
        l = l * r + wave_sum(p);
        c0 *= r;
        c1 *= r;
        m = mn;
        sP[w][lane] = p;
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        for (int j = 0; j < nk; ++j) {
            const float pj = sP[w][j];
            if (lane < d) c0 += pj * bf(sV[j * d + lane]);
            if (lane + kWave < d) c1 += pj * bf(sV[j * d + kWave + lane]);
        }
    }
    __syncthreads();
    if (sBad) m = l = c0 = c1 = __builtin_nanf("");
    float* st = state_of(a.state, a, row, h);
    if (lane == 0) { st[0] = m; st[1] = l; }
    if (lane < d) st[2 + lane] = c0;
    if (lane + kWave < d) st[2 + kWave + lane] = c1;
}

// grid (R, Hkv): blockIdx.x = row; wave w = query head g * G + w.  Folded rows of the branches
// in a.mask.  Lane m scores block position m when the child recomputed it (old: the parent's
// key there, new: the child's); the wave reduces, and lane l accumulates dimensions l and
// l + 64 over the changed positions.
template <int D>
__global__ __launch_bounds__(kWave * kMaxGroup) void level_kernel(const Args a) {
    const int row = blockIdx.x, g = blockIdx.y;
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    const int i = row / a.N, n = row - i * a.N;
    if (i == 0 || !((a.mask >> i) & 1ull) || a.fold[row] == 0) return;
    constexpr int d = D;
    const int R = a.nb * a.N, G = a.Hq / a.Hkv, h = g * G + w;
    const int p = a.par[i];
    float* st = state_of(a.state, a, row, h);
    const int sq = a.src_slot[row];
    const bool changed = lane < a.N && a.fold[i * a.N + lane] == 0;
    const int s_old = changed ? a.src_slot[p * a.N + lane] : 0, s_new = changed ? a.src_slot[i * a.N + lane] : 0;
    const bool bad_lane = changed && (s_old < 0 || s_old >= R || s_new < 0 || s_new >= R);
    if (sq < 0 || sq >= R || __ballot(bad_lane) != 0) {
        if (lane == 0) st[0] = st[1] = __builtin_nanf("");
        return;
    }
    // the folded query is its source's: the parent's at this position
    uint32_t qv[D / 2];
    load_query<D>(qv, a.q_c + (static_cast<size_t>(sq) * a.Hq + h) * d);
    const float* ps = state_of(a.state, a, p * a.N + n, h);
    const float mp = ps[0], lp = ps[1];
    const float so_l = changed ? dot_global<D>(qv, kv_row(a.k_c, a, s_old, g)) * a.scale_log2 : -INFINITY;
    const float sn_l = changed ? dot_global<D>(qv, kv_row(a.k_c, a, s_new, g)) * a.scale_log2 : -INFINITY;
    // the running maximum over the parent's keys and the child's new terms
    const float mx = fmaxf(mp, wave_max(sn_l));
    const float eo = changed ? exp2f(so_l - mx) : 0.f, en = changed ? exp2f(sn_l - mx) : 0.f;
    const float so = wave_sum(eo), sn = wave_sum(en);
    float o0 = 0.f, o1 = 0.f, n0 = 0.f, n1 = 0.f;
    uint64_t todo = __ballot(changed);
    while (todo) {
        const int m = __builtin_ctzll(todo);
        todo &= todo - 1;
        const float eom = __shfl(eo, m, kWave), enm = __shfl(en, m, kWave);
        const int som = __shfl(s_old, m, kWave), snm = __shfl(s_new, m, kWave);
        float v0, v1;
        load2(kv_row(a.v_c, a, som, g), d, lane, v0, v1);
        o0 += eom * v0;
        o1 += eom * v1;
        load2(kv_row(a.v_c, a, snm, g), d, lane, v0, v1);
        n0 += enm * v0;
        n1 += enm * v1;
    }
    const float r = mp == -INFINITY ? 0.f : exp2f(mp - mx);
    const float ap0 = lane < d ? ps[2 + lane] : 0.f;
    const float ap1 = lane + kWave < d ? ps[2 + kWave + lane] : 0.f;
    if (lane == 0) { st[0] = mx; st[1] = lp * r - so + sn; }
    if (lane < d) st[2 + lane] = ap0 * r - o0 + n0;
    if (lane + kWave < d) st[2 + kWave + lane] = ap1 * r - o1 + n1;
}

// grid (R): one workgroup per row divides every head's numerator by its denominator
__global__ __launch_bounds__(256) void finalize_kernel(const Args a) {
    const int row = blockIdx.x, hd = a.hd;
    for (int e = threadIdx.x; e < a.Hq * hd; e += blockDim.x) {
        const int h = e / hd, j = e - h * hd;
        const float* st = a.cstate + (static_cast<size_t>(row) * a.Hq + h) * (hd + 2);
        a.out[(static_cast<size_t>(row) * a.Hq + h) * hd + j] = st[2 + j] / st[1];
    }
}

int check_shape(const specfold_shape* s) {
    if (!s) return SPECFOLD_ERR_NULL;
    if (s->n_branch < 1 || s->n_branch > SPECFOLD_MAX_BRANCHES || s->block < 1 || s->block > SPECFOLD_MAX_BLOCK ||
        s->n_q_heads < 1 || s->n_kv_heads < 1 || s->n_q_heads % s->n_kv_heads != 0 || s->head_dim < 1 ||
        (s->head_dim != 16 && s->head_dim != 32 && s->head_dim != 64 && s->head_dim != 128) ||
        s->n_q_heads / s->n_kv_heads > kMaxGroup ||
        s->prefix_len < 0)
        return SPECFOLD_ERR_SHAPE;
    return SPECFOLD_OK;
}

int check_tree(const specfold_shape* s, const int32_t* par) {
    if (!par) return SPECFOLD_ERR_NULL;
    if (par[0] != -1) return SPECFOLD_ERR_TREE;
    for (int i = 1; i < s->n_branch; ++i)
        if (par[i] < 0 || par[i] >= i) return SPECFOLD_ERR_TREE;
    return SPECFOLD_OK;
}

Args base_args(const specfold_shape* s) {
    Args a{};
    a.nb = s->n_branch;
    a.N = s->block;
    a.Hq = s->n_q_heads;
    a.Hkv = s->n_kv_heads;
    a.hd = s->head_dim;
    a.P = s->prefix_len;
    a.scale_log2 = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(s->head_dim)));
    return a;
}

int launch(void (*k)(Args), dim3 grid, dim3 block, const Args& a, void* stream) {
    hipLaunchKernelGGL(k, grid, block, 0, static_cast<hipStream_t>(stream), a);
    return hipGetLastError() == hipSuccess ? SPECFOLD_OK : SPECFOLD_ERR_HIP;
}

int launch_group(void (*k)(Args), const Args& a, void* stream) {
    return launch(k, dim3(a.nb * a.N, a.Hkv), dim3(kWave * (a.Hq / a.Hkv)), a, stream);
}

int launch_fresh(const Args& a, void* stream) {
    switch (a.hd) {
        case 16: return launch_group(fresh_kernel<16>, a, stream);
        case 32: return launch_group(fresh_kernel<32>, a, stream);
        case 64: return launch_group(fresh_kernel<64>, a, stream);
        case 128: return launch_group(fresh_kernel<128>, a, stream);
        default: return SPECFOLD_ERR_SHAPE;
    }
}

int launch_level(const Args& a, void* stream) {
    switch (a.hd) {
        case 16: return launch_group(level_kernel<16>, a, stream);
        case 32: return launch_group(level_kernel<32>, a, stream);
        case 64: return launch_group(level_kernel<64>, a, stream);
        case 128: return launch_group(level_kernel<128>, a, stream);
        default: return SPECFOLD_ERR_SHAPE;
    }
}

}  // namespace

extern "C" int specfold_variant_correction_levels(const specfold_shape* shape, const int32_t* parent_host,
                                                  uint64_t* masks, int32_t* n_levels) {
    int e = check_shape(shape);
    if (e == SPECFOLD_OK) e = check_tree(shape, parent_host);
    if (e != SPECFOLD_OK) return e;
    if (!masks || !n_levels) return SPECFOLD_ERR_NULL;
    int depth[SPECFOLD_MAX_BRANCHES];
    int top = 0;
    depth[0] = 0;
    for (int i = 0; i < shape->n_branch; ++i) masks[i] = 0;
    for (int i = 1; i < shape->n_branch; ++i) {
        depth[i] = depth[parent_host[i]] + 1;
        masks[depth[i] - 1] |= 1ull << i;
        if (depth[i] > top) top = depth[i];
    }
    *n_levels = top;
    return SPECFOLD_OK;
}

extern "C" int specfold_variant_correction_fresh(const specfold_shape* shape, const specfold_bf16* q_c,
                                                 const specfold_bf16* k_c, const specfold_bf16* v_c,
                                                 const int32_t* rec_rows, const int32_t* rec_count,
                                                 const int32_t* src_slot, const specfold_prefix_kv* prefix,
                                                 float* state, void* stream) {
    const int e = check_shape(shape);
    if (e != SPECFOLD_OK) return e;
    if (!q_c || !k_c || !v_c || !rec_rows || !rec_count || !src_slot || !state) return SPECFOLD_ERR_NULL;
    if (shape->prefix_len > 0 && (!prefix || !prefix->k || !prefix->v)) return SPECFOLD_ERR_NULL;
    Args a = base_args(shape);
    a.q_c = q_c;
    a.k_c = k_c;
    a.v_c = v_c;
    a.rec_rows = rec_rows;
    a.rec_count = rec_count;
    a.src_slot = src_slot;
    if (shape->prefix_len > 0) {
        a.pk = prefix->k;
        a.pv = prefix->v;
        a.pk_st = prefix->k_stride_tok;
        a.pk_sh = prefix->k_stride_head;
        a.pv_st = prefix->v_stride_tok;
        a.pv_sh = prefix->v_stride_head;
    }
    a.state = state;
    return launch_fresh(a, stream);
}

extern "C" int specfold_variant_correction_level(const specfold_shape* shape, const int32_t* parent_host,
                                                 uint64_t branch_mask, const specfold_bf16* q_c,
                                                 const specfold_bf16* k_c, const specfold_bf16* v_c,
                                                 const int32_t* src_slot, const uint8_t* fold, float* state,
                                                 void* stream) {
    int e = check_shape(shape);
    if (e == SPECFOLD_OK) e = check_tree(shape, parent_host);
    if (e != SPECFOLD_OK) return e;
    if (!q_c || !k_c || !v_c || !src_slot || !fold || !state) return SPECFOLD_ERR_NULL;
    if (shape->n_branch < 64 && (branch_mask >> shape->n_branch) != 0) return SPECFOLD_ERR_SHAPE;
    Args a = base_args(shape);
    a.q_c = q_c;
    a.k_c = k_c;
    a.v_c = v_c;
    a.src_slot = src_slot;
    a.fold = fold;
    a.state = state;
    a.mask = branch_mask & ~1ull;
    for (int i = 0; i < shape->n_branch; ++i) a.par[i] = parent_host[i];
    return launch_level(a, stream);
}

extern "C" int specfold_variant_correction_finalize(const specfold_shape* shape, const float* state, float* out,
                                                    void* stream) {
    const int e = check_shape(shape);
    if (e != SPECFOLD_OK) return e;
    if (!state || !out) return SPECFOLD_ERR_NULL;
    Args a = base_args(shape);
    a.cstate = state;
    a.out = out;
    return launch(finalize_kernel, dim3(a.nb * a.N), dim3(256), a, stream);
}
