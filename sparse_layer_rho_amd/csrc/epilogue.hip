// Epilogues of the split-K projections.  Each sums its K-split partials in ascending split
// order (deterministic), then:
//   qkv:   applies the rotate-half rotary embedding to the Q and K heads at absolute position
//          P + n and scatters bf16 q_c / k_c / v_c [SpecFold summary, App. B: recomputed
//          positions get RMSNorm and packed QKV projections with rotary embeddings];
//   oproj: adds the residual stream, h_mid = H + attn W_o^T (every row), and writes the
//          RMSNorm'd row the FFN consumes;
//   down:  one workgroup per recompute slot reduces that slot's FFN output once and adds it to
//          the residual stream of every row whose fold source is that slot,
//          H_out[r] = h_mid[r] + f[src_slot[r]] [SpecFold summary, App. B: every position adds
//          its own residual stream, which is never folded; §A.2: folded positions reuse the
//          source's FFN output].
// Every thread owns 4 consecutive columns of one row and issues all its loads (SPL split
// partials, rounded up; splits past the last read zeros) before it adds anything, so a kernel
// costs one memory round trip instead of one per split.
#include "kernels.h"
#include "lanes.h"

namespace specfold {

namespace {

__device__ __forceinline__ int clamp_m(const int32_t* m_count, int cap) {
    int M = m_count[0];
    return M < 0 ? 0 : (M > cap ? cap : M);
}

// the float4s at byte offset base + s * stride for splits s < S (zeros past S) ...
template <int SPL>
__device__ __forceinline__ void load_splits(f32x4 (&v)[SPL], __amdgpu_buffer_rsrc_t r, uint32_t base, uint32_t stride,
                                            int S) {
#pragma unroll
    for (int s = 0; s < SPL; ++s) v[s] = buf_loadf4(r, s < S ? base + s * stride : kOob);
}

// ... and their sum in ascending split order
template <int SPL>
__device__ __forceinline__ f32x4 add_splits(const f32x4 (&v)[SPL]) {
    f32x4 acc = v[0];
#pragma unroll
    for (int s = 1; s < SPL; ++s) acc += v[s];
    return acc;
}

template <int SPL>
__device__ __forceinline__ f32x4 sum_splits(__amdgpu_buffer_rsrc_t r, uint32_t base, uint32_t stride, int S) {
    f32x4 v[SPL];
    load_splits<SPL>(v, r, base, stride, S);
    return add_splits<SPL>(v);
}

__device__ __forceinline__ void unpack4(const uint2 v, float* f) {
    f[0] = __uint_as_float(v.x << 16);
    f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16);
    f[3] = __uint_as_float(v.y & 0xffff0000u);
}

__device__ __forceinline__ uint2 pack4(const float* f) {
    return make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
}

// workgroup m = recompute slot m; thread u = (head, 4 consecutive rotary pairs j0 .. j0+3)
template <int SPL>
__global__ __launch_bounds__(1024) void qkv_epilogue_kernel(const QkvEpiArgs a) {
    const int m = blockIdx.x;
    const int heads = a.Hq + 2 * a.Hkv, half = a.hd >> 1, q4 = a.hd >> 3;
    const int u = threadIdx.x;
    if (m >= clamp_m(a.m_count, a.m_cap) || u >= heads * q4) return;
    const int nq = heads * a.hd;
    const int hh = u / q4, j0 = (u - hh * q4) * 4;
    const int c1 = hh * a.hd + j0;
    const __amdgpu_buffer_rsrc_t rP =
        make_rsrc(a.part, static_cast<uint32_t>(static_cast<size_t>(a.splits) * a.m_cap * nq * 4));
    const uint32_t stride = static_cast<uint32_t>(a.m_cap) * nq * 4;
    const uint32_t base = (static_cast<uint32_t>(m) * nq + c1) * 4;
    // one round trip: the slot's row, the frequency table and the partials are all requested
    // before any of them is used (the scheduling barrier keeps the compiler from waiting for
    // the row before it issues the rest)
    const int row = a.rec_rows[m];
    double inv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) inv[e] = a.inv_freq[j0 + e];
    f32x4 p1[SPL], p2[SPL];
    load_splits<SPL>(p1, rP, base, stride, a.splits);
    load_splits<SPL>(p2, rP, base + half * 4, stride, a.splits);
    __builtin_amdgcn_sched_barrier(0);
    const bool ok = row >= 0 && row < a.R;
    // the rotation angles (P + n) theta^(-2j/d), formed in double
    const double pos = static_cast<double>(a.P + (ok ? row % a.N : 0));
    double ang[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) ang[e] = pos * inv[e];
    f32x4 x1 = add_splits<SPL>(p1);
    f32x4 x2 = add_splits<SPL>(p2);
    if (!ok) x1 = x2 = f32x4{1.f, 1.f, 1.f, 1.f} * __builtin_nanf("");
    float y1[4], y2[4];
    if (hh < a.Hq + a.Hkv) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // the angle in revolutions, reduced to [-1/2, 1/2] in double, then the hardware
            // sine and cosine, which take revolutions (absolute error near 2^-20, far below the
            // bf16 rounding of the rotated values)
            const double rev = ang[e] * 0.15915494309189533577;     // 1 / (2 pi)
            const float red = static_cast<float>(rev - rint(rev));
            const float sn = __builtin_amdgcn_sinf(red), cs = __builtin_amdgcn_cosf(red);
            y1[e] = x1[e] * cs - x2[e] * sn;
            y2[e] = x2[e] * cs + x1[e] * sn;
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) { y1[e] = x1[e]; y2[e] = x2[e]; }
    }
    uint16_t* dst;
    if (hh < a.Hq) dst = a.q_c + (static_cast<size_t>(m) * a.Hq + hh) * a.hd;
    else if (hh < a.Hq + a.Hkv) dst = a.k_c + (static_cast<size_t>(m) * a.Hkv + (hh - a.Hq)) * a.hd;
    else dst = a.v_c + (static_cast<size_t>(m) * a.Hkv + (hh - a.Hq - a.Hkv)) * a.hd;
    *reinterpret_cast<uint2*>(dst + j0) = pack4(y1);
    *reinterpret_cast<uint2*>(dst + j0 + half) = pack4(y2);
}

// workgroup r = row r; thread t owns column quads t, t + blockDim.x, ... (MAXU of them)
template <int SPL, int MAXU>
__global__ __launch_bounds__(1024) void oproj_epilogue_kernel(const float* __restrict__ part, int splits, int R,
                                                              int D, const uint16_t* __restrict__ H,
                                                              uint16_t* __restrict__ h_mid,
                                                              const uint16_t* __restrict__ ln, float eps,
                                                              uint16_t* __restrict__ xn) {
    __shared__ float s_ss[16];
    const int r = blockIdx.x, tid = threadIdx.x, B = blockDim.x;
    const int D4 = D >> 2;
    const __amdgpu_buffer_rsrc_t rP = make_rsrc(part, static_cast<uint32_t>(static_cast<size_t>(splits) * R * D * 4));
    const __amdgpu_buffer_rsrc_t rH = make_rsrc(H, static_cast<uint32_t>(static_cast<size_t>(R) * D * 2));
    const uint32_t stride = static_cast<uint32_t>(R) * D * 4;
    f32x4 acc[MAXU];
    uint2 hv[MAXU], wv[MAXU];
    // the norm weights come with the partials and the residual (one round trip, not a second
    // one after the row's reduction)
    const __amdgpu_buffer_rsrc_t rL = make_rsrc(ln, static_cast<uint32_t>(D) * 2);
#pragma unroll
    for (int k = 0; k < MAXU; ++k) {
        const int u = tid + k * B;
        const bool valid = u < D4;
        const uint32_t e = static_cast<uint32_t>(r) * D + 4 * u;
        acc[k] = sum_splits<SPL>(rP, valid ? e * 4 : kOob, stride, splits);
        hv[k] = buf_load8(rH, valid ? e * 2 : kOob);
        wv[k] = xn && ln ? buf_load8(rL, valid ? 8 * u : kOob) : make_uint2(0, 0);
    }
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < MAXU; ++k) {
        const int u = tid + k * B;
        float h[4];
        unpack4(hv[k], h);
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] += acc[k][e];
        hv[k] = pack4(h);
        if (u < D4) {
            *reinterpret_cast<uint2*>(h_mid + static_cast<size_t>(r) * D + 4 * u) = hv[k];
            unpack4(hv[k], h);                     // RMSNorm reads the bf16-rounded residual
#pragma unroll
            for (int e = 0; e < 4; ++e) ss += h[e] * h[e];
        }
    }
    if (!xn) return;
    ss = wave_sum_dpp(ss);
    if ((tid & 63) == 0) s_ss[tid >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < 16; ++w) tot += w < (B >> 6) ? s_ss[w] : 0.f;   // one LDS round trip
    const float inv = 1.0f / sqrtf(tot / static_cast<float>(D) + eps);
#pragma unroll
    for (int k = 0; k < MAXU; ++k) {
        const int u = tid + k * B;
        if (u >= D4) continue;
        float h[4], w[4] = {1.f, 1.f, 1.f, 1.f};
        unpack4(hv[k], h);
        if (ln) unpack4(wv[k], w);
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = h[e] * inv * w[e];
        *reinterpret_cast<uint2*>(xn + static_cast<size_t>(r) * D + 4 * u) = pack4(h);
    }
}

// workgroup (b, part): reduces slot b (when b < M) into every row that inherits from it, over
// the part-th of the gridDim.y ranges of column quads; also writes NaN into those columns of row
// b when row b's source slot is invalid.  The parts spread each slot's split partials (its
// largest input) over several CUs.  The rows that can inherit from slot b are the rows at its
// position n (a fold source is an ancestor's row at the same position), so their residual
// rows are requested with the partials, before it is known which of them inherit: two round
// trips (the slot's row, then everything else) instead of three.
template <int SPL, int MAXU>
__global__ __launch_bounds__(128) void down_epilogue_kernel(const float* __restrict__ part, int splits, int m_cap,
                                                             const int32_t* m_count, const int32_t* rec_rows,
                                                             const int32_t* __restrict__ src_slot, int nb, int N,
                                                             int D, const uint16_t* __restrict__ h_mid,
                                                             uint16_t* __restrict__ H_out) {
    constexpr int kSpec = 12;                      // branches whose residual rows are loaded speculatively
    const int b = blockIdx.x, tid = threadIdx.x, B = blockDim.x;
    const int R = nb * N;
    const int D4 = D >> 2;
    const int QP = (D4 + static_cast<int>(gridDim.y) - 1) / static_cast<int>(gridDim.y);
    const int u0 = static_cast<int>(blockIdx.y) * QP, u1 = min(D4, u0 + QP);   // this part's quads
    // first round trip: the recompute count, this row's source slot and this slot's row
    const int M = clamp_m(m_count, m_cap);
    const int sb = b < R ? src_slot[b] : 0;
    const int row = b < m_cap ? rec_rows[b] : -1;
    if (b < R && (sb < 0 || sb >= M)) {
        const float nan = __builtin_nanf("");
        for (int c4 = u0 + tid; c4 < u1; c4 += B)
            *reinterpret_cast<uint2*>(H_out + static_cast<size_t>(b) * D + 4 * c4) =
                make_uint2(pack_bf16x2(nan, nan), pack_bf16x2(nan, nan));
    }
    if (b >= M || row < 0 || row >= R) return;
    const int n = row % N;
    // second round trip: the slot's partials, the source slots of the rows at position n (the
    // rows that can inherit from slot b) and, speculatively, the residual rows of the first
    // kSpec of them, so the rows that do inherit need no third round trip
    const __amdgpu_buffer_rsrc_t rP = make_rsrc(part, static_cast<uint32_t>(static_cast<size_t>(splits) * m_cap * D * 4));
    const __amdgpu_buffer_rsrc_t rH = make_rsrc(h_mid, static_cast<uint32_t>(static_cast<size_t>(R) * D * 2));
    const uint32_t stride = static_cast<uint32_t>(m_cap) * D * 4;
    // every wave loads the candidates' source slots itself (lane t: branch t), first, so they
    // are waited for alone
    const int lane = tid & (kWave - 1);
    const int cand = lane < nb ? src_slot[lane * N + n] : -1;
    f32x4 pv[MAXU][SPL];
#pragma unroll
    for (int k = 0; k < MAXU; ++k) {
        const int u = u0 + tid + k * B;
        load_splits<SPL>(pv[k], rP, u < u1 ? (static_cast<uint32_t>(b) * D + 4 * u) * 4 : kOob, stride, splits);
    }
    uint2 hv[kSpec][MAXU];
#pragma unroll
    for (int t = 0; t < kSpec; ++t)
#pragma unroll
        for (int k = 0; k < MAXU; ++k) {
            const int u = u0 + tid + k * B;
            hv[t][k] = buf_load8(rH, t < nb && u < u1 ? (static_cast<uint32_t>(t * N + n) * D + 4 * u) * 2 : kOob);
        }
    __builtin_amdgcn_sched_barrier(0);
    const uint64_t hit = __ballot(cand == b);      // uniform: the branches that inherit from b
    f32x4 f[MAXU];
#pragma unroll
    for (int k = 0; k < MAXU; ++k) f[k] = add_splits<SPL>(pv[k]);
#pragma unroll
    for (int t = 0; t < kSpec; ++t) {
        if (!((hit >> t) & 1)) continue;
#pragma unroll
        for (int k = 0; k < MAXU; ++k) {
            const int u = u0 + tid + k * B;
            if (u >= u1) continue;
            float h[4];
            unpack4(hv[t][k], h);
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] += f[k][e];
            *reinterpret_cast<uint2*>(H_out + static_cast<size_t>(t * N + n) * D + 4 * u) = pack4(h);
        }
    }
    // the speculative loads are needed on every path (else the compiler sinks a row's load
    // into the branch that stores it, behind a round trip of its own)
    uint32_t keep = 0;
#pragma unroll
    for (int t = 0; t < kSpec; ++t)
#pragma unroll
        for (int k = 0; k < MAXU; ++k) keep ^= hv[t][k].x ^ hv[t][k].y;
    asm volatile("" ::"v"(keep));
    // branches past the first kSpec: one round trip per branch
    for (int t = kSpec; t < nb; ++t) {
        if (!((hit >> t) & 1)) continue;
#pragma unroll
        for (int k = 0; k < MAXU; ++k) {
            const int u = u0 + tid + k * B;
            if (u >= u1) continue;
            float h[4];
            unpack4(buf_load8(rH, (static_cast<uint32_t>(t * N + n) * D + 4 * u) * 2), h);
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] += f[k][e];
            *reinterpret_cast<uint2*>(H_out + static_cast<size_t>(t * N + n) * D + 4 * u) = pack4(h);
        }
    }
}

// split count rounded up to the compiled load batch
template <typename F>
hipError_t with_spl(int splits, F&& f) {
    if (splits <= 4) return f(std::integral_constant<int, 4>{});
    if (splits <= 8) return f(std::integral_constant<int, 8>{});
    if (splits <= 16) return f(std::integral_constant<int, 16>{});
    if (splits <= 32) return f(std::integral_constant<int, 32>{});
    return hipErrorInvalidValue;
}

// threads per row: the column quads, rounded up to a wave and capped at 1024 (then 2 per thread)
inline int quad_block(int D4) {
    const int b = ((D4 + 63) / 64) * 64;
    return b > 1024 ? 1024 : (b < 64 ? 64 : b);
}

}  // namespace

hipError_t launch_qkv_epilogue(const QkvEpiArgs& a, hipStream_t st) {
    if (a.m_cap <= 0) return hipSuccess;
    const int units = (a.Hq + 2 * a.Hkv) * (a.hd >> 3);
    if (units > 1024) return hipErrorInvalidValue;
    const int block = ((units + 63) / 64) * 64;
    return with_spl(a.splits, [&](auto spl) {
        hipLaunchKernelGGL(qkv_epilogue_kernel<decltype(spl)::value>, dim3(a.m_cap), dim3(block), 0, st, a);
        return hipGetLastError();
    });
}

hipError_t launch_oproj_epilogue(const float* part, int splits, int R, int D, const uint16_t* H,
                                 uint16_t* h_mid, const uint16_t* ln, float eps, uint16_t* xn,
                                 hipStream_t st) {
    if (R <= 0) return hipSuccess;
    const int D4 = D >> 2, block = quad_block(D4);
    const int per = (D4 + block - 1) / block;
    if (per > 2) return hipErrorInvalidValue;
    return with_spl(splits, [&](auto spl) {
        constexpr int SPL = decltype(spl)::value;
        if (per == 1)
            hipLaunchKernelGGL((oproj_epilogue_kernel<SPL, 1>), dim3(R), dim3(block), 0, st, part, splits, R, D, H,
                               h_mid, ln, eps, xn);
        else
            hipLaunchKernelGGL((oproj_epilogue_kernel<SPL, 2>), dim3(R), dim3(block), 0, st, part, splits, R, D, H,
                               h_mid, ln, eps, xn);
        return hipGetLastError();
    });
}

hipError_t launch_down_epilogue(const float* part, int splits, int m_cap, const int32_t* m_count,
                                const int32_t* rec_rows, const int32_t* src_slot, int nb, int N, int D,
                                const uint16_t* h_mid, uint16_t* H_out, hipStream_t st) {
    const int R = nb * N;
    if (R <= 0) return hipSuccess;
    // column parts of at most 128 quads (512 columns): three at D = 1536, seven at 3584
    const int D4 = D >> 2, parts = (D4 + 127) / 128;
    const int qp = (D4 + parts - 1) / parts, block = quad_block(qp);
    const int per = (qp + block - 1) / block;
    if (per > 1 || block > 128) return hipErrorInvalidValue;     // the kernel's launch bounds
    const dim3 grid(R > m_cap ? R : m_cap, parts);
    return with_spl(splits, [&](auto spl) {
        constexpr int SPL = decltype(spl)::value;
        hipLaunchKernelGGL((down_epilogue_kernel<SPL, 1>), grid, dim3(block), 0, st, part, splits, m_cap, m_count,
                           rec_rows, src_slot, nb, N, D, h_mid, H_out);
        return hipGetLastError();
    });
}

}  // namespace specfold
