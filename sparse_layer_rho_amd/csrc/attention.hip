// Folded attention, exact per branch [SpecFold review, "무엇과 다른가": exact with respect to
// the branch's own KV; SpecFold summary, §A.1: the folded query ends with the child's exact
// state].  For row (i, n), head h, group g = h / (Hq/Hkv), the keys are the shared prefix
// [P][Hkv][d] (a strided zero-copy view, [SpecFold review, "어떻게 쓰나"]) followed by the N
// block keys of branch i, k_c[src_slot(i, m)], and the query is q_c[src_slot(i, n)].
//
// A folded row's query and the prefix equal its source's, so the prefix part of its softmax
// state is its source's: kernel 1 computes the prefix state (running max m, denominator l,
// unnormalised output o -- the retained per-head statistics of [SpecFold summary, App. B])
// once per recompute slot, split over chunks of the prefix (flash-decoding style).  Kernel 2
// computes the N-key block part for every row of every branch and merges it with the chunk
// states of the row's source slot by log-sum-exp, in a fixed order (deterministic).
//
// Both kernels are FlashAttention-style on bf16 MFMA with the transposed product S^T = K Q^T:
// keys are the MFMA rows, the 16 queries of a wave are its columns, so each lane owns one
// query's statistics and the P V product O^T = V^T P^T takes P straight from registers
// (the key order inside a 32-key step is permuted identically on both operands).
#include "kernels.h"

namespace specfold {

namespace {

constexpr float kNegInf = -__builtin_inff();

template <int HD>
struct AttnTile {
    static constexpr int KS = (HD + 31) / 32;   // 32-wide k-steps over head_dim
    static constexpr int DT = HD / 16;          // 16-row output tiles over head_dim
    static constexpr int KROW = HD * 2 + 16;    // LDS bytes per key row (padded)
    static constexpr int VROW = 64 * 2 + 8;     // LDS bytes per transposed value row (64 keys)
};

// Load up to 64 keys/values (rows given by key_ptr) into LDS: K row-major, V transposed.
template <int HD, typename KeyPtr>
__device__ __forceinline__ void stage_kv(uint8_t* sK, uint8_t* sV, int nk, KeyPtr key_ptr) {
    using T = AttnTile<HD>;
    constexpr int CH = HD / 8;
    uint16_t* vt = reinterpret_cast<uint16_t*>(sV);
    for (int idx = threadIdx.x; idx < 64 * CH; idx += blockDim.x) {
        const int key = idx / CH, cc = idx - key * CH;
        uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
        const uint16_t* kp = nullptr;
        const uint16_t* vp = nullptr;
        if (key < nk) key_ptr(key, kp, vp);
        if (kp) {
            kv = *reinterpret_cast<const uint4*>(kp + cc * 8);
            vv = *reinterpret_cast<const uint4*>(vp + cc * 8);
        }
        *reinterpret_cast<uint4*>(sK + key * T::KROW + cc * 16) = kv;
        const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            vt[(cc * 8 + 2 * e) * (T::VROW / 2) + key] = static_cast<uint16_t>(w[e] & 0xffffu);
            vt[(cc * 8 + 2 * e + 1) * (T::VROW / 2) + key] = static_cast<uint16_t>(w[e] >> 16);
        }
    }
}

// One 64-key block of online softmax for the wave's 16 queries.
// qf: B operand (query lane&15, d = 32s + 8*(lane>>4)); nk valid keys.
template <int HD>
__device__ __forceinline__ void attend_block(const uint8_t* sK, const uint8_t* sV, int nk,
                                             const uint4 (&qf)[AttnTile<HD>::KS], float scale_log2,
                                             float& run_m, float& run_l, f32x4 (&o)[AttnTile<HD>::DT]) {
    using T = AttnTile<HD>;
    const int lane = threadIdx.x & 63;
    const int g4 = lane >> 4, l16 = lane & 15;
    const int ntiles = (nk + 15) >> 4;
    f32x4 sc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
        sc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (kt < ntiles) {
#pragma unroll
            for (int s = 0; s < T::KS; ++s) {
                const int d0 = 32 * s + 8 * g4;
                const uint4 kf = (d0 < HD) ? *reinterpret_cast<const uint4*>(sK + (kt * 16 + l16) * T::KROW + d0 * 2)
                                           : make_uint4(0, 0, 0, 0);
                sc[kt] = mfma16x16x32(kf, qf[s], sc[kt]);
            }
        }
    }
    // lane holds S^T[key = 16kt + 4*g4 + i][query l16]
    float bmax = kNegInf;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = kt * 16 + 4 * g4 + i;
            const float v = (key < nk) ? sc[kt][i] * scale_log2 : kNegInf;
            sc[kt][i] = v;
            bmax = fmaxf(bmax, v);
        }
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16, kWave));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32, kWave));
    const float new_m = fmaxf(run_m, bmax);
    const float alpha = (run_m == kNegInf) ? 0.f : exp2f(run_m - new_m);
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float e = (sc[kt][i] == kNegInf) ? 0.f : exp2f(sc[kt][i] - new_m);
            sc[kt][i] = e;
            psum += e;
        }
    run_l = run_l * alpha + psum;
    run_m = new_m;
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) o[dt] *= alpha;
    // O^T += V^T P^T over two 32-key steps; slot 8*g4 + i <-> key 32u + 4*g4 + i and
    // slot 8*g4 + 4 + i <-> key 32u + 16 + 4*g4 + i on both operands
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        if (32 * u < nk) {
            const float pf[8] = {sc[2 * u][0], sc[2 * u][1], sc[2 * u][2], sc[2 * u][3],
                                 sc[2 * u + 1][0], sc[2 * u + 1][1], sc[2 * u + 1][2], sc[2 * u + 1][3]};
            const uint4 pb = pack8(pf);
#pragma unroll
            for (int dt = 0; dt < T::DT; ++dt) {
                const uint16_t* vrow = reinterpret_cast<const uint16_t*>(sV + (dt * 16 + l16) * T::VROW);
                const uint2 lo = *reinterpret_cast<const uint2*>(vrow + 32 * u + 4 * g4);
                const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 32 * u + 16 + 4 * g4);
                o[dt] = mfma16x16x32(make_uint4(lo.x, lo.y, hi.x, hi.y), pb, o[dt]);
            }
        }
    }
}

template <int HD>
__device__ __forceinline__ void load_query(const uint16_t* qrow, bool valid, uint4 (&qf)[AttnTile<HD>::KS]) {
    const int g4 = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int s = 0; s < AttnTile<HD>::KS; ++s) {
        const int d0 = 32 * s + 8 * g4;
        qf[s] = (valid && d0 < HD) ? *reinterpret_cast<const uint4*>(qrow + d0) : make_uint4(0, 0, 0, 0);
    }
}

__device__ __forceinline__ int clamp_count(const int32_t* m_count, int cap) {
    int M = m_count[0];
    return M < 0 ? 0 : (M > cap ? cap : M);
}

// grid: x = tiles of 64 (slot, head-in-group) queries, y = prefix chunk, z = KV group
template <int HD>
__global__ __launch_bounds__(256) void attn_prefix_kernel(const AttnArgs a) {
    using T = AttnTile<HD>;
    __shared__ __align__(16) uint8_t sK[64 * T::KROW];
    __shared__ __align__(16) uint8_t sV[HD * T::VROW];
    const int G = a.Hq / a.Hkv;
    const int g = blockIdx.z, chunk = blockIdx.y;
    const int M = clamp_count(a.m_count, a.m_cap);
    const int nq = M * G;
    const int q0 = blockIdx.x * 64;
    if (q0 >= nq) return;
    const int key0 = chunk * a.chunk_len;
    const int key1 = min(a.P, key0 + a.chunk_len);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int qi = q0 + wave * 16 + (lane & 15);
    const bool qvalid = qi < nq;
    const int m = qvalid ? qi / G : 0, h = g * G + (qvalid ? qi % G : 0);
    uint4 qf[T::KS];
    load_query<HD>(a.q_c + (static_cast<size_t>(m) * a.Hq + h) * HD, qvalid, qf);

    float run_m = kNegInf, run_l = 0.f;
    f32x4 o[T::DT];
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int kb = key0; kb < key1; kb += 64) {
        const int nk = min(64, key1 - kb);
        __syncthreads();
        stage_kv<HD>(sK, sV, nk, [&](int key, const uint16_t*& kp, const uint16_t*& vp) {
            kp = a.pk + (kb + key) * a.pk_st + g * a.pk_sh;
            vp = a.pv + (kb + key) * a.pv_st + g * a.pv_sh;
        });
        __syncthreads();
        attend_block<HD>(sK, sV, nk, qf, a.scale_log2, run_m, run_l, o);
    }
    run_l += __shfl_xor(run_l, 16, kWave);
    run_l += __shfl_xor(run_l, 32, kWave);
    if (!qvalid) return;
    const size_t base = (static_cast<size_t>(chunk) * a.m_cap + m) * a.Hq + h;
    if ((lane >> 4) == 0) {
        a.part_ml[2 * base] = run_m;
        a.part_ml[2 * base + 1] = run_l;
    }
    float* po = a.part_o + base * HD + 4 * (lane >> 4);
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) *reinterpret_cast<f32x4*>(po + dt * 16) = o[dt];
}

// grid: x = branch, y = KV group, z = group of 4 query tiles (16 positions x 1 head each)
template <int HD>
__global__ __launch_bounds__(256) void attn_block_kernel(const AttnArgs a) {
    using T = AttnTile<HD>;
    __shared__ __align__(16) uint8_t sK[64 * T::KROW];
    __shared__ __align__(16) uint8_t sV[HD * T::VROW];
    __shared__ int sSlot[64];
    __shared__ int sBad;
    const int G = a.Hq / a.Hkv, N = a.N;
    const int i = blockIdx.x, g = blockIdx.y;
    const int M = clamp_count(a.m_count, a.m_cap);
    const int nt16 = (N + 15) >> 4;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int qt = blockIdx.z * 4 + wave;

    if (threadIdx.x == 0) sBad = 0;
    __syncthreads();
    if (threadIdx.x < 64) {
        int s = -1;
        if (threadIdx.x < N) {
            s = a.src_slot[i * N + threadIdx.x];
            if (s < 0 || s >= M) {
                s = -1;
                atomicOr(&sBad, 1);
            }
        }
        sSlot[threadIdx.x] = s;
    }
    __syncthreads();
    stage_kv<HD>(sK, sV, N, [&](int key, const uint16_t*& kp, const uint16_t*& vp) {
        const int s = sSlot[key];
        if (s >= 0) {
            kp = a.k_c + (static_cast<size_t>(s) * a.Hkv + g) * HD;
            vp = a.v_c + (static_cast<size_t>(s) * a.Hkv + g) * HD;
        }
    });
    __syncthreads();
    if (qt >= G * nt16) return;

    const int j = qt / nt16, nt = qt - j * nt16;
    const int h = g * G + j;
    const int n = nt * 16 + (lane & 15);
    const bool nvalid = n < N;
    const int qslot = nvalid ? sSlot[n] : -1;
    uint4 qf[T::KS];
    load_query<HD>(a.q_c + (static_cast<size_t>(qslot < 0 ? 0 : qslot) * a.Hq + h) * HD, qslot >= 0, qf);

    float run_m = kNegInf, run_l = 0.f;
    f32x4 o[T::DT];
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    attend_block<HD>(sK, sV, N, qf, a.scale_log2, run_m, run_l, o);
    run_l += __shfl_xor(run_l, 16, kWave);
    run_l += __shfl_xor(run_l, 32, kWave);
    if (!nvalid) return;

    // merge with the prefix chunk states of the source slot, chunks in ascending order
    const int ps = qslot < 0 ? 0 : qslot;
    float mx = run_m;
    for (int c = 0; c < a.n_chunks; ++c)
        mx = fmaxf(mx, a.part_ml[2 * ((static_cast<size_t>(c) * a.m_cap + ps) * a.Hq + h)]);
    const float wb = exp2f(run_m - mx);
    float L = run_l * wb;
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) o[dt] *= wb;
    for (int c = 0; c < a.n_chunks; ++c) {
        const size_t base = (static_cast<size_t>(c) * a.m_cap + ps) * a.Hq + h;
        const float wc = exp2f(a.part_ml[2 * base] - mx);
        L += a.part_ml[2 * base + 1] * wc;
        const float* po = a.part_o + base * HD + 4 * (lane >> 4);
#pragma unroll
        for (int dt = 0; dt < T::DT; ++dt) o[dt] += *reinterpret_cast<const f32x4*>(po + dt * 16) * wc;
    }
    const bool bad = (qslot < 0) || (sBad != 0);
    const float invL = bad ? __builtin_nanf("") : 1.0f / L;
    const int row = i * N + n;
    uint16_t* dst = a.attn + (static_cast<size_t>(row) * a.Hq + h) * HD + 4 * (lane >> 4);
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) {
        const f32x4 v = o[dt] * invL;
        *reinterpret_cast<uint2*>(dst + dt * 16) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    }
    if (a.lse && (lane >> 4) == 0)
        a.lse[static_cast<size_t>(row) * a.Hq + h] = bad ? __builtin_nanf("") : (mx + log2f(L)) * 0.69314718055994531f;
}

}  // namespace

hipError_t launch_attn_prefix(const AttnArgs& a, hipStream_t st) {
    if (a.n_chunks <= 0) return hipSuccess;
    const int G = a.Hq / a.Hkv;
    const dim3 grid((a.m_cap * G + 63) / 64, a.n_chunks, a.Hkv);
    switch (a.hd) {
        case 16: hipLaunchKernelGGL(attn_prefix_kernel<16>, grid, dim3(256), 0, st, a); break;
        case 32: hipLaunchKernelGGL(attn_prefix_kernel<32>, grid, dim3(256), 0, st, a); break;
        case 64: hipLaunchKernelGGL(attn_prefix_kernel<64>, grid, dim3(256), 0, st, a); break;
        case 128: hipLaunchKernelGGL(attn_prefix_kernel<128>, grid, dim3(256), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_attn_block(const AttnArgs& a, hipStream_t st) {
    const int G = a.Hq / a.Hkv;
    const int tiles = G * ((a.N + 15) / 16);
    const dim3 grid(a.nb, a.Hkv, (tiles + 3) / 4);
    switch (a.hd) {
        case 16: hipLaunchKernelGGL(attn_block_kernel<16>, grid, dim3(256), 0, st, a); break;
        case 32: hipLaunchKernelGGL(attn_block_kernel<32>, grid, dim3(256), 0, st, a); break;
        case 64: hipLaunchKernelGGL(attn_block_kernel<64>, grid, dim3(256), 0, st, a); break;
        case 128: hipLaunchKernelGGL(attn_block_kernel<128>, grid, dim3(256), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace specfold
