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
// Keys and values move through LDS in blocks of 64: K row-major, V transposed (the PV product
// needs 8 consecutive keys of one dimension per lane).  Every load is a bounded buffer load
// (keys past the end and invalid slots read as zeros), so a block costs one round trip, and the
// prefix kernel fetches block b+1 into registers while it multiplies block b.
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
    static constexpr int CH = HD / 8;           // 16-byte chunks per key row
    static constexpr int U = (64 * CH + 255) / 256;   // staging units per thread (256 threads)
};

// Registers of one 64-key block: unit u of thread t is chunk cc of key `key`, with
// idx = t + 256 u = cc * 64 + key (consecutive threads take consecutive keys, so the transposed
// V stores of a wave cover 128 contiguous bytes).  off(key, cc) gives the byte offsets of the
// K and V chunk, or kOob.
template <int HD>
struct KVRegs {
    uint4 k[AttnTile<HD>::U], v[AttnTile<HD>::U];

    template <typename Off>
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, Off off) {
        using T = AttnTile<HD>;
#pragma unroll
        for (int u = 0; u < T::U; ++u) {
            const int idx = threadIdx.x + 256 * u;
            const int cc = idx >> 6, key = idx & 63;
            uint32_t ok_ = kOob, ov = kOob;
            if (idx < 64 * T::CH) off(key, cc, ok_, ov);
            k[u] = buf_load16(rk, ok_);
            v[u] = buf_load16(rv, ov);
        }
    }

    __device__ __forceinline__ void store(uint8_t* sK, uint8_t* sV) const {
        using T = AttnTile<HD>;
        uint16_t* vt = reinterpret_cast<uint16_t*>(sV);
#pragma unroll
        for (int u = 0; u < T::U; ++u) {
            const int idx = threadIdx.x + 256 * u;
            if (idx >= 64 * T::CH) continue;
            const int cc = idx >> 6, key = idx & 63;
            *reinterpret_cast<uint4*>(sK + key * T::KROW + cc * 16) = k[u];
            const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                vt[(cc * 8 + 2 * e) * (T::VROW / 2) + key] = static_cast<uint16_t>(w[e] & 0xffffu);
                vt[(cc * 8 + 2 * e + 1) * (T::VROW / 2) + key] = static_cast<uint16_t>(w[e] >> 16);
            }
        }
    }
};

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

// query fragments of one head row (byte offset qoff in q_c, or kOob)
template <int HD>
__device__ __forceinline__ void load_query(__amdgpu_buffer_rsrc_t rq, uint32_t qoff, uint4 (&qf)[AttnTile<HD>::KS]) {
    const int g4 = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int s = 0; s < AttnTile<HD>::KS; ++s) {
        const int d0 = 32 * s + 8 * g4;
        qf[s] = buf_load16(rq, d0 < HD ? qoff + d0 * 2 : kOob);
    }
}

__device__ __forceinline__ int clamp_count(const int32_t* m_count, int cap) {
    int M = m_count[0];
    return M < 0 ? 0 : (M > cap ? cap : M);
}

// bytes spanned by a strided prefix view [P][Hkv][HD]
__device__ __forceinline__ uint32_t view_bytes(int P, int Hkv, int64_t st, int64_t sh, int HD) {
    return static_cast<uint32_t>(((P - 1) * st + (Hkv - 1) * sh + HD) * 2);
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

    const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q_c, static_cast<uint32_t>(static_cast<size_t>(a.m_cap) * a.Hq * HD * 2));
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.pk, view_bytes(a.P, a.Hkv, a.pk_st, a.pk_sh, HD));
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.pv, view_bytes(a.P, a.Hkv, a.pv_st, a.pv_sh, HD));
    auto block_off = [&](int kb) {
        const int nk = min(64, key1 - kb);
        return [=](int key, int cc, uint32_t& ok_, uint32_t& ov) {
            if (key < nk) {
                ok_ = static_cast<uint32_t>(((kb + key) * a.pk_st + g * a.pk_sh + cc * 8) * 2);
                ov = static_cast<uint32_t>(((kb + key) * a.pv_st + g * a.pv_sh + cc * 8) * 2);
            }
        };
    };
    KVRegs<HD> kv;
    kv.load(rk, rv, block_off(key0));
    uint4 qf[T::KS];
    load_query<HD>(rq, qvalid ? static_cast<uint32_t>((m * a.Hq + h) * HD * 2) : kOob, qf);

    float run_m = kNegInf, run_l = 0.f;
    f32x4 o[T::DT];
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int kb = key0; kb < key1; kb += 64) {
        __syncthreads();                           // the previous block is consumed
        kv.store(sK, sV);
        __syncthreads();
        if (kb + 64 < key1) kv.load(rk, rv, block_off(kb + 64));   // in flight during the block
        attend_block<HD>(sK, sV, min(64, key1 - kb), qf, a.scale_log2, run_m, run_l, o);
    }
    run_l += __shfl_xor(run_l, 16, kWave);
    run_l += __shfl_xor(run_l, 32, kWave);
    if (!qvalid) return;
    const size_t base = (static_cast<size_t>(chunk) * a.m_cap + m) * a.Hq + h;
    if ((lane >> 4) == 0)
        *reinterpret_cast<float2*>(a.part_ml + 2 * base) = make_float2(run_m, run_l);
    float* po = a.part_o + base * HD + 4 * (lane >> 4);
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) *reinterpret_cast<f32x4*>(po + dt * 16) = o[dt];
}

// grid: x = branch, y = KV group, z = group of 4 query tiles (16 positions x 1 head each)
template <int HD>
__global__ __launch_bounds__(256) void attn_block_kernel(const AttnArgs a) {
    using T = AttnTile<HD>;
    constexpr int kBatch = 4;                      // prefix chunk states loaded per round trip
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
    const uint32_t rows_bytes = static_cast<uint32_t>(static_cast<size_t>(a.m_cap) * a.Hkv * HD * 2);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k_c, rows_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v_c, rows_bytes);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q_c, static_cast<uint32_t>(static_cast<size_t>(a.m_cap) * a.Hq * HD * 2));
    KVRegs<HD> kv;
    kv.load(rk, rv, [&](int key, int cc, uint32_t& ok_, uint32_t& ov) {
        const int s = key < N ? sSlot[key] : -1;
        if (s >= 0) ok_ = ov = static_cast<uint32_t>(((s * a.Hkv + g) * HD + cc * 8) * 2);
    });

    const bool active = qt < G * nt16;             // wave-uniform
    const int j = active ? qt / nt16 : 0, nt = active ? qt - j * nt16 : 0;
    const int h = g * G + j;
    const int n = nt * 16 + (lane & 15);
    const bool nvalid = active && n < N;
    const int qslot = nvalid ? sSlot[n] : -1;
    uint4 qf[T::KS];
    load_query<HD>(rq, qslot >= 0 ? static_cast<uint32_t>((qslot * a.Hq + h) * HD * 2) : kOob, qf);

    // prefix chunk states of the source slot: the first batch is requested now, so it arrives
    // while the block part is computed
    const int ps = qslot < 0 ? 0 : qslot;
    const __amdgpu_buffer_rsrc_t rml =
        make_rsrc(a.part_ml, static_cast<uint32_t>(static_cast<size_t>(a.n_chunks) * a.m_cap * a.Hq * 8));
    const __amdgpu_buffer_rsrc_t ro =
        make_rsrc(a.part_o, static_cast<uint32_t>(static_cast<size_t>(a.n_chunks) * a.m_cap * a.Hq * HD * 4));
    float2 ml[kBatch];
    f32x4 co[kBatch][T::DT];
    auto load_states = [&](int c0) {
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const bool ok = active && c0 + b < a.n_chunks;
            const uint32_t base = static_cast<uint32_t>(((c0 + b) * a.m_cap + ps) * a.Hq + h);
            ml[b] = __builtin_bit_cast(float2, buf_load8(rml, ok ? base * 8 : kOob));
#pragma unroll
            for (int dt = 0; dt < T::DT; ++dt)
                co[b][dt] = buf_loadf4(ro, ok ? (base * HD + dt * 16 + 4 * (lane >> 4)) * 4 : kOob);
        }
    };
    load_states(0);
    kv.store(sK, sV);
    __syncthreads();
    if (!active) return;

    float run_m = kNegInf, run_l = 0.f;
    f32x4 o[T::DT];
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    attend_block<HD>(sK, sV, N, qf, a.scale_log2, run_m, run_l, o);
    run_l += __shfl_xor(run_l, 16, kWave);
    run_l += __shfl_xor(run_l, 32, kWave);

    // merge the prefix chunk states in ascending chunk order by online log-sum-exp rescaling
    for (int c0 = 0; c0 < a.n_chunks; c0 += kBatch) {
        if (c0 > 0) load_states(c0);
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            if (c0 + b >= a.n_chunks) break;
            const float nm = fmaxf(run_m, ml[b].x);
            const float wa = exp2f(run_m - nm), wc = exp2f(ml[b].x - nm);
            run_l = run_l * wa + ml[b].y * wc;
#pragma unroll
            for (int dt = 0; dt < T::DT; ++dt) o[dt] = o[dt] * wa + co[b][dt] * wc;
            run_m = nm;
        }
    }
    if (!nvalid) return;
    const bool bad = (qslot < 0) || (sBad != 0);
    const float invL = bad ? __builtin_nanf("") : 1.0f / run_l;
    const int row = i * N + n;
    uint16_t* dst = a.attn + (static_cast<size_t>(row) * a.Hq + h) * HD + 4 * (lane >> 4);
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) {
        const f32x4 v = o[dt] * invL;
        *reinterpret_cast<uint2*>(dst + dt * 16) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    }
    if (a.lse && (lane >> 4) == 0)
        a.lse[static_cast<size_t>(row) * a.Hq + h] = bad ? __builtin_nanf("") : (run_m + log2f(run_l)) * 0.69314718055994531f;
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
