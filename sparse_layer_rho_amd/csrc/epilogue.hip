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
#include "kernels.h"

namespace specfold {

namespace {

__device__ __forceinline__ int clamp_m(const int32_t* m_count, int cap) {
    int M = m_count[0];
    return M < 0 ? 0 : (M > cap ? cap : M);
}

__global__ __launch_bounds__(256) void qkv_epilogue_kernel(const QkvEpiArgs a) {
    const int m = blockIdx.x;
    if (m >= clamp_m(a.m_count, a.m_cap)) return;
    const int row = a.rec_rows[m];
    const bool ok = row >= 0 && row < a.R;
    const double pos = static_cast<double>(a.P + (ok ? row % a.N : 0));
    const int heads = a.Hq + 2 * a.Hkv;
    const int half = a.hd >> 1;
    const int nq = heads * a.hd;
    const float bad = ok ? 0.f : __builtin_nanf("");
    for (int idx = threadIdx.x; idx < heads * half; idx += blockDim.x) {
        const int hh = idx / half, j = idx - hh * half;
        const int c1 = hh * a.hd + j, c2 = c1 + half;
        float x1 = bad, x2 = bad;
        for (int s = 0; s < a.splits; ++s) {
            const float* pr = a.part + (static_cast<size_t>(s) * a.m_cap + m) * nq;
            x1 += pr[c1];
            x2 += pr[c2];
        }
        float y1 = x1, y2 = x2;
        if (hh < a.Hq + a.Hkv) {
            // angle (P + n) theta^(-2j/d) formed in double and reduced to [-pi, pi]
            const double ang = pos * a.inv_freq[j];
            const double twopi = 6.283185307179586476925286766559;
            const float red = static_cast<float>(ang - twopi * rint(ang / twopi));
            float sn, cs;
            sincosf(red, &sn, &cs);
            y1 = x1 * cs - x2 * sn;
            y2 = x2 * cs + x1 * sn;
        }
        uint16_t* dst;
        if (hh < a.Hq) dst = a.q_c + (static_cast<size_t>(m) * a.Hq + hh) * a.hd;
        else if (hh < a.Hq + a.Hkv) dst = a.k_c + (static_cast<size_t>(m) * a.Hkv + (hh - a.Hq)) * a.hd;
        else dst = a.v_c + (static_cast<size_t>(m) * a.Hkv + (hh - a.Hq - a.Hkv)) * a.hd;
        dst[j] = f32_to_bf16(y1);
        dst[j + half] = f32_to_bf16(y2);
    }
}

__device__ __forceinline__ void load_bf16x4(const uint16_t* p, float* f) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    f[0] = __uint_as_float(v.x << 16);
    f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16);
    f[3] = __uint_as_float(v.y & 0xffff0000u);
}

// one wave per row
__global__ __launch_bounds__(256) void oproj_epilogue_kernel(const float* __restrict__ part, int splits, int R,
                                                             int D, const uint16_t* __restrict__ H,
                                                             uint16_t* __restrict__ h_mid,
                                                             const uint16_t* __restrict__ ln, float eps,
                                                             uint16_t* __restrict__ xn) {
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (r >= R) return;
    const int D4 = D >> 2;
    float ss = 0.f;
    for (int c4 = lane; c4 < D4; c4 += 64) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < splits; ++s)
            acc += *reinterpret_cast<const f32x4*>(part + (static_cast<size_t>(s) * R + r) * D + 4 * c4);
        float h[4];
        load_bf16x4(H + static_cast<size_t>(r) * D + 4 * c4, h);
        const uint2 hv = make_uint2(pack_bf16x2(h[0] + acc[0], h[1] + acc[1]), pack_bf16x2(h[2] + acc[2], h[3] + acc[3]));
        *reinterpret_cast<uint2*>(h_mid + static_cast<size_t>(r) * D + 4 * c4) = hv;
        const float q0 = __uint_as_float(hv.x << 16), q1 = __uint_as_float(hv.x & 0xffff0000u);
        const float q2 = __uint_as_float(hv.y << 16), q3 = __uint_as_float(hv.y & 0xffff0000u);
        ss += q0 * q0 + q1 * q1 + q2 * q2 + q3 * q3;
    }
    if (!xn) return;
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / static_cast<float>(D) + eps);
    for (int c4 = lane; c4 < D4; c4 += 64) {
        float h[4], w[4] = {1.f, 1.f, 1.f, 1.f};
        load_bf16x4(h_mid + static_cast<size_t>(r) * D + 4 * c4, h);
        if (ln) load_bf16x4(ln + 4 * c4, w);
        *reinterpret_cast<uint2*>(xn + static_cast<size_t>(r) * D + 4 * c4) =
            make_uint2(pack_bf16x2(h[0] * inv * w[0], h[1] * inv * w[1]), pack_bf16x2(h[2] * inv * w[2], h[3] * inv * w[3]));
    }
}

// workgroup b: reduces slot b (when b < M) into every row that inherits from it; also writes
// NaN into row b when row b's source slot is invalid
__global__ __launch_bounds__(256) void down_epilogue_kernel(const float* __restrict__ part, int splits, int m_cap,
                                                            const int32_t* m_count, const int32_t* rec_rows,
                                                            const int32_t* __restrict__ src_slot, int nb, int N,
                                                            int D, const uint16_t* __restrict__ h_mid,
                                                            uint16_t* __restrict__ H_out) {
    __shared__ int s_rows[kMaxBranches];
    __shared__ int s_cnt;
    const int b = blockIdx.x;
    const int M = clamp_m(m_count, m_cap);
    const int R = nb * N;
    const int D4 = D >> 2;
    if (b < R) {
        const int sb = src_slot[b];
        if (sb < 0 || sb >= M) {
            const float nan = __builtin_nanf("");
            for (int c4 = threadIdx.x; c4 < D4; c4 += blockDim.x)
                *reinterpret_cast<uint2*>(H_out + static_cast<size_t>(b) * D + 4 * c4) =
                    make_uint2(pack_bf16x2(nan, nan), pack_bf16x2(nan, nan));
        }
    }
    if (b >= M) return;
    const int row = rec_rows[b];
    if (row < 0 || row >= R) return;
    const int n = row % N;
    if (threadIdx.x == 0) s_cnt = 0;
    __syncthreads();
    if (threadIdx.x < nb) {
        const int r = threadIdx.x * N + n;
        if (src_slot[r] == b) s_rows[atomicAdd(&s_cnt, 1)] = r;
    }
    __syncthreads();
    const int cnt = s_cnt;
    for (int c4 = threadIdx.x; c4 < D4; c4 += blockDim.x) {
        f32x4 f = {0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < splits; ++s)
            f += *reinterpret_cast<const f32x4*>(part + (static_cast<size_t>(s) * m_cap + b) * D + 4 * c4);
        for (int t = 0; t < cnt; ++t) {
            const int r = s_rows[t];
            float h[4];
            load_bf16x4(h_mid + static_cast<size_t>(r) * D + 4 * c4, h);
            *reinterpret_cast<uint2*>(H_out + static_cast<size_t>(r) * D + 4 * c4) =
                make_uint2(pack_bf16x2(h[0] + f[0], h[1] + f[1]), pack_bf16x2(h[2] + f[2], h[3] + f[3]));
        }
    }
}

}  // namespace

hipError_t launch_qkv_epilogue(const QkvEpiArgs& a, hipStream_t st) {
    if (a.m_cap <= 0) return hipSuccess;
    hipLaunchKernelGGL(qkv_epilogue_kernel, dim3(a.m_cap), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_oproj_epilogue(const float* part, int splits, int R, int D, const uint16_t* H,
                                 uint16_t* h_mid, const uint16_t* ln, float eps, uint16_t* xn,
                                 hipStream_t st) {
    if (R <= 0) return hipSuccess;
    hipLaunchKernelGGL(oproj_epilogue_kernel, dim3((R + 3) / 4), dim3(256), 0, st, part, splits, R, D, H, h_mid,
                       ln, eps, xn);
    return hipGetLastError();
}

hipError_t launch_down_epilogue(const float* part, int splits, int m_cap, const int32_t* m_count,
                                const int32_t* rec_rows, const int32_t* src_slot, int nb, int N, int D,
                                const uint16_t* h_mid, uint16_t* H_out, hipStream_t st) {
    const int R = nb * N;
    if (R <= 0) return hipSuccess;
    hipLaunchKernelGGL(down_epilogue_kernel, dim3(R > m_cap ? R : m_cap), dim3(256), 0, st, part, splits, m_cap,
                       m_count, rec_rows, src_slot, nb, N, D, h_mid, H_out);
    return hipGetLastError();
}

}  // namespace specfold
