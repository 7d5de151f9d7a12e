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
// Keys and values move HBM -> LDS with buffer_load ... lds (no register staging), both
// row-major: one such load fills 1 KB of LDS, i.e. whole key rows, so every 4-lane quad reads
// one 64-byte segment.  Row r keeps its 16-byte chunk c at position c ^ fk(r) in K and
// c ^ fv(r) in V, which makes the K fragment reads (16 rows x one chunk) and the transposed V
// reads conflict-free.  The P V product needs 8 keys of one dimension per lane; gfx950's
// ds_read_b64_tr_b16 delivers them from the row-major layout: in each 16-lane group, lane p
// names the 4 elements at (row p/4, columns 4(p%4)..+3) of a 4 x 16 tile, and lane L receives
// column L of that tile (one element per row).  Every load is bounded (keys past the end and
// invalid slots read as zeros).  The prefix kernel requests a whole stage of 128 keys at once,
// so a stage costs one round trip, and the next stage is in flight while one is multiplied;
// two waves share each query tile, one per 64-key half of the stage.
//
// Both kernels are FlashAttention-style on bf16 MFMA with the transposed product S^T = K Q^T:
// keys are the MFMA rows, the 16 queries of a wave are its columns, so each lane owns one
// query's statistics and the P V product O^T = V^T P^T takes P straight from registers
// (the key order inside a 32-key step is permuted identically on both operands).
#include "kernels.h"
#include "lanes.h"

namespace specfold {

namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr int kStageKeys = 128;                 // prefix keys per LDS stage
constexpr float kLazy = 8.f;                    // softmax reference slack, log2 units

typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int HD>
struct AttnTile {
    static constexpr int KS = (HD + 31) / 32;   // 32-wide k-steps over head_dim
    static constexpr int DT = HD / 16;          // 16-row output tiles over head_dim
    static constexpr int CH = HD / 8;           // 16-byte chunks per key row
    static constexpr int RB = HD * 2;           // LDS bytes per key row
    static __device__ __forceinline__ int fk(int r) { return r & (CH - 1); }
    static __device__ __forceinline__ int fv(int r) { return (2 * r) & (CH - 1); }
};

// 16 bytes per lane, global -> LDS: lane l's bytes land at lds + 16 l (lds is wave-uniform);
// the address is voff (per lane) + soff (wave-uniform)
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff, uint32_t soff = 0) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(lds), 16, voff, soff, 0, 0);
}

// this wave's buffer loads (register and LDS) are complete
__device__ __forceinline__ void vm_drain() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// at most N of this wave's vector-memory operations are outstanding (gfx9 s_waitcnt: vmcnt
// bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima)
template <int N>
__device__ __forceinline__ void vm_wait_le_states() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// 2^x with the hardware instruction (no rescaling of results below 2^-126: softmax weights
// that small are below the fp32 resolution of the running sum anyway)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// two floats -> two bf16, round to nearest even, with gfx950's v_cvt_pk_bf16_f32
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2_t));
}

__device__ __forceinline__ uint4 cvt_bf16x8(const float* f) {
    return make_uint4(cvt_bf16x2(f[0], f[1]), cvt_bf16x2(f[2], f[3]), cvt_bf16x2(f[4], f[5]),
                      cvt_bf16x2(f[6], f[7]));
}

// ds_read_b128 as inline asm: the compiler can neither hoist a wait above the rest of a batch
// nor reuse a batch's registers before it lands, so all of a block's key fragments are in
// flight together (left to itself it keeps two in flight); kf_wait<N> supplies the wait
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_u8*)(p)));
}

template <int OFF>
__device__ __forceinline__ u32x4 lds_read16(uint32_t addr) {
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}

// at most N of this wave's LDS reads outstanding; the fragments of `v` are used only after it
template <int N, int C>
__device__ __forceinline__ void kf_wait(u32x4 (&v)[C]) {
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(N) : "memory");
#pragma unroll
    for (int i = 0; i < C; ++i) asm volatile("" : "+v"(v[i]));
}

// Request NKEYS rows of K and V into sK / sV (swizzled as above).  row_off(row, k_or_v) gives
// the element offset of a key row's first dimension, or -1 for a missing key (the host keeps
// every view under 1 GB, so offsets fit in 32 bits).  Load i of the NKEYS*CH/64 per tensor is
// issued by wave i % NW (NW waves in the workgroup).  Every offset is formed before the first
// load: for a row_off that reads LDS, the compiler would otherwise re-read it after each load
// into LDS (one round trip per load).
template <int HD, int NKEYS, int NW, typename RowOff>
__device__ __forceinline__ void request_rows(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                             uint8_t* sK, uint8_t* sV, RowOff row_off) {
    using T = AttnTile<HD>;
    constexpr int kLoads = NKEYS * T::CH / 64;
    constexpr int kPer = (kLoads + NW - 1) / NW;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    uint32_t ok_[kPer], ov[kPer];
#pragma unroll
    for (int t = 0; t < kPer; ++t) {
        const int i = wave + NW * t;
        const int q = i * 64 + lane;
        const int row = q / T::CH, pos = q % T::CH;
        const int ek = i < kLoads ? row_off(row, 0) : -1, ev = i < kLoads ? row_off(row, 1) : -1;
        ok_[t] = ek < 0 ? kOob : static_cast<uint32_t>((ek + 8 * (pos ^ T::fk(row))) * 2);
        ov[t] = ev < 0 ? kOob : static_cast<uint32_t>((ev + 8 * (pos ^ T::fv(row))) * 2);
    }
#pragma unroll
    for (int t = 0; t < kPer; ++t) {
        const int i = wave + NW * t;
        if (i >= kLoads) break;                    // wave-uniform
        dma16(rk, sK + i * 1024, ok_[t]);
        dma16(rv, sV + i * 1024, ov[t]);
    }
}

// One block of 16 * NKT keys (NKT = 2 or 4) of online softmax for the wave's NQ tiles of 16
// queries; sK / sV point at the block's first row (a multiple of 16 rows into the stage, so
// the swizzles line up).  Every key and value fragment read from LDS serves all NQ tiles.
// qf[q]: B operand of query tile q (query lane&15, d = 32s + 8*(lane>>4)); nk valid keys.
template <int HD, int NKT, int NQ>
__device__ __forceinline__ void attend_block(const uint8_t* sK, const uint8_t* sV, int nk,
                                             const uint4 (&qf)[NQ][AttnTile<HD>::KS], float scale_log2,
                                             float (&run_m)[NQ], float (&run_l)[NQ],
                                             f32x4 (&o)[NQ][AttnTile<HD>::DT]) {
    using T = AttnTile<HD>;
    static_assert(NKT == 2 || NKT == 4, "blocks of 32 or 64 keys");
    const int lane = threadIdx.x & 63;
    const int g4 = lane >> 4, l16 = lane & 15;
    // Branch-free: rows past nk hold zeros (their loads were out of range), their scores are
    // masked below and their P entries are zero, so all fragment reads can be issued at once.
    f32x4 sc[NQ][NKT];
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) sc[q][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (HD % 32 == 0) {
        // every 32-wide k-step lies inside the row: the NKT reads of one k-step differ in
        // their key tile only (fk depends on the row's low bits, the same in every tile), so
        // they take immediate offsets; k-step s is waited for with the later ones in flight
        u32x4 kf[T::KS][NKT];
#pragma unroll
        for (int s = 0; s < T::KS; ++s) {
            const int c = 4 * s + g4;
            const uint32_t a = lds_addr(sK) + l16 * T::RB + ((c ^ T::fk(l16)) << 4);
            kf[s][0] = lds_read16<0>(a);
            kf[s][1] = lds_read16<16 * T::RB>(a);
            if constexpr (NKT == 4) {
                kf[s][2] = lds_read16<32 * T::RB>(a);
                kf[s][3] = lds_read16<48 * T::RB>(a);
            }
        }
        auto step = [&](int s) {
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int q = 0; q < NQ; ++q)
                    sc[q][kt] = mfma16x16x32(__builtin_bit_cast(uint4, kf[s][kt]), qf[q][s], sc[q][kt]);
            __builtin_amdgcn_sched_barrier(0);    // k-step s's MFMAs stay ahead of the next wait
        };
        if constexpr (T::KS == 4) {
            kf_wait<3 * NKT>(kf[0]); step(0);
            kf_wait<2 * NKT>(kf[1]); step(1);
            kf_wait<NKT>(kf[2]); step(2);
            kf_wait<0>(kf[3]); step(3);
        } else if constexpr (T::KS == 2) {
            kf_wait<NKT>(kf[0]); step(0);
            kf_wait<0>(kf[1]); step(1);
        } else {
            kf_wait<0>(kf[0]); step(0);
        }
    } else {
        uint4 kf[NKT][T::KS];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
            const int r = kt * 16 + l16;
#pragma unroll
            for (int s = 0; s < T::KS; ++s) {
                const int c = 4 * s + g4;
                kf[kt][s] = (8 * c < HD) ? *reinterpret_cast<const uint4*>(sK + r * T::RB + ((c ^ T::fk(r)) << 4))
                                         : make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int s = 0; s < T::KS; ++s)
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int q = 0; q < NQ; ++q) sc[q][kt] = mfma16x16x32(kf[kt][s], qf[q][s], sc[q][kt]);
    }
    // lane holds S^T[key = 16kt + 4*g4 + i][query l16] of each query tile.  The reference
    // maximum run_m moves only when a score passes it by more than kLazy (log2 units).  The
    // state (run_m, run_l, o) is exact for any reference, and below that margin every weight
    // exp2(s - run_m) <= 2^kLazy stays far inside fp32 and bf16, so most blocks skip rescaling
    // o; the rescale runs when any query of the wave moves its reference.
    float alpha[NQ];
    bool rescale_any = false;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        float bmax = kNegInf;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = kt * 16 + 4 * g4 + i;
                const float v = (key < nk) ? sc[q][kt][i] * scale_log2 : kNegInf;
                sc[q][kt][i] = v;
                bmax = fmaxf(bmax, v);
            }
        bmax = max_rows4(bmax);                    // over the query's four lanes
        const bool grow = bmax > run_m[q] + kLazy;
        const float new_m = grow ? bmax : run_m[q];
        float psum = 0.f;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e = (sc[q][kt][i] == kNegInf) ? 0.f : fast_exp2(sc[q][kt][i] - new_m);
                sc[q][kt][i] = e;
                psum += e;
            }
        const bool rescale = grow && run_m[q] != kNegInf;   // a state of zeros needs no rescale
        alpha[q] = rescale ? fast_exp2(run_m[q] - new_m) : 1.f;
        rescale_any = rescale_any || rescale;
        run_l[q] = run_l[q] * alpha[q] + psum;
        run_m[q] = new_m;
    }
    if (__ballot(rescale_any) != 0) {              // wave-uniform
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int dt = 0; dt < T::DT; ++dt) o[q][dt] *= alpha[q];
    }
    // O^T += V^T P^T over 32-key steps; slot 8*g4 + i <-> key 32u + 4*g4 + i and
    // slot 8*g4 + 4 + i <-> key 32u + 16 + 4*g4 + i on both operands.  The A operand (V^T,
    // rows = dimensions) comes from two transposed reads of 4 keys each: lane p of the group
    // names key row 4*g4 + p/4 (+16), dimensions 16dt + 4(p%4)..+3.
    const int pr = l16 >> 2, pc = l16 & 3;
#pragma unroll
    for (int u = 0; u < NKT / 2; ++u) {
        uint4 pb[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const float pf[8] = {sc[q][2 * u][0], sc[q][2 * u][1], sc[q][2 * u][2], sc[q][2 * u][3],
                                 sc[q][2 * u + 1][0], sc[q][2 * u + 1][1], sc[q][2 * u + 1][2], sc[q][2 * u + 1][3]};
            pb[q] = cvt_bf16x8(pf);
        }
        const int r0 = 32 * u + 4 * g4 + pr, r1 = r0 + 16;
        uint2 lo[T::DT], hi[T::DT];
#pragma unroll
        for (int dt = 0; dt < T::DT; ++dt) {
            const int c = 2 * dt + (pc >> 1);
            const uint8_t* a0 = sV + r0 * T::RB + ((c ^ T::fv(r0)) << 4) + 8 * (pc & 1);
            const uint8_t* a1 = sV + r1 * T::RB + ((c ^ T::fv(r1)) << 4) + 8 * (pc & 1);
            lo[dt] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0)));
            hi[dt] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a1)));
        }
#pragma unroll
        for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                o[q][dt] = mfma16x16x32(make_uint4(lo[dt].x, lo[dt].y, hi[dt].x, hi[dt].y), pb[q], o[q][dt]);
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

// grid: x = prefix chunk * Hkv + KV group, y = group of QT 16-query tiles of (slot,
// head-in-group) queries, so the groups below the recompute count are dispatched first.
// 2 QT compute waves: wave w takes query tile w % QT and, of every stage, the 64-key half w / QT;
// the two halves' states are merged through LDS at the end.  (Every wave reads a whole 64-key
// block from LDS, so few waves per CU keep the LDS port from saturating.)  LW = 0: the compute
// waves also request the stages; LW = 4 (chunks of several stages): four more waves request
// them, so the next stage's loads are issued while the current one is multiplied rather than
// before.  Dynamic LDS: one stage of kStageKeys rows of K and V, or two when a chunk spans
// several stages.
template <int HD, int QT, int LW>
__global__ __launch_bounds__(128 * QT + 64 * LW) void attn_prefix_kernel(const AttnArgs a) {
    using T = AttnTile<HD>;
    constexpr int kStageBytes = kStageKeys * T::RB;
    extern __shared__ __align__(16) uint8_t smem[];
    const int G = a.Hq / a.Hkv;
    const int g = blockIdx.x % a.Hkv, chunk = blockIdx.x / a.Hkv;
    const int M = clamp_count(a.m_count, a.m_cap);
    const int nq = M * G;
    const int q0 = blockIdx.y * 16 * QT;
    if (q0 >= nq) return;
    const int key0 = chunk * a.chunk_len;
    const int key1 = min(a.P, key0 + a.chunk_len);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const bool loader = LW > 0 && wave >= 2 * QT;  // wave-uniform
    const int qw = wave % QT, half = wave / QT;
    const int qi = q0 + qw * 16 + (lane & 15);
    const bool qvalid = qi < nq;
    const int m = qvalid ? qi / G : 0, h = g * G + (qvalid ? qi % G : 0);

    const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q_c, static_cast<uint32_t>(static_cast<size_t>(a.m_cap) * a.Hq * HD * 2));
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.pk, view_bytes(a.P, a.Hkv, a.pk_st, a.pk_sh, HD));
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.pv, view_bytes(a.P, a.Hkv, a.pv_st, a.pv_sh, HD));
    const int kst = static_cast<int>(a.pk_st), kbase = g * static_cast<int>(a.pk_sh);
    const int vst = static_cast<int>(a.pv_st), vbase = g * static_cast<int>(a.pv_sh);
    // Stage requests: load i (1 KB, kRpl key rows) of a stage is issued by wave i % NW.  A
    // wave's loads are kRpl * NW rows apart, a multiple of the swizzle period, so the lane's
    // row within its load and its swizzled chunk are the same in every load: the lane offsets
    // are formed once and each load adds a wave-uniform key offset (no per-load arithmetic).
    // Only a stage that runs past the chunk's end masks rows, per lane.
    constexpr int NW = LW > 0 ? LW : 2 * QT, kRpl = 64 / T::CH, kLoads = kStageKeys / kRpl;
    constexpr int kPer = (kLoads + NW - 1) / NW;
    static_assert((NW * kRpl) % T::CH == 0, "a wave's loads keep the lane's swizzle");
    const int rw = LW > 0 ? wave - 2 * QT : wave;  // requesting wave index (load waves: >= 0)
    const int lrow = rw * kRpl + lane / T::CH, pos = lane % T::CH;
    const uint32_t koff = static_cast<uint32_t>((lrow * kst + kbase + 8 * (pos ^ T::fk(lrow))) * 2);
    const uint32_t voff = static_cast<uint32_t>((lrow * vst + vbase + 8 * (pos ^ T::fv(lrow))) * 2);
    auto request_stage = [&](int kb, int buf) {
        uint8_t* sK = smem + buf * 2 * kStageBytes;
        uint8_t* sV = sK + kStageBytes;
        if (kb + kStageKeys <= key1) {             // wave-uniform: every row of the stage is a key
#pragma unroll
            for (int t = 0; t < kPer; ++t) {
                const int i = rw + NW * t;
                if (kLoads % NW != 0 && i >= kLoads) break;
                const int r0 = kb + NW * kRpl * t;
                dma16(rk, sK + i * 1024, koff, static_cast<uint32_t>(r0 * kst * 2));
                dma16(rv, sV + i * 1024, voff, static_cast<uint32_t>(r0 * vst * 2));
            }
        } else {
#pragma unroll
            for (int t = 0; t < kPer; ++t) {
                const int i = rw + NW * t;
                if (kLoads % NW != 0 && i >= kLoads) break;
                const int r0 = kb + NW * kRpl * t;
                const bool ok = r0 + lrow < key1;
                dma16(rk, sK + i * 1024, ok ? koff + static_cast<uint32_t>(r0 * kst * 2) : kOob);
                dma16(rv, sV + i * 1024, ok ? voff + static_cast<uint32_t>(r0 * vst * 2) : kOob);
            }
        }
    };
    const bool requester = LW == 0 || loader;
    if (requester) request_stage(key0, 0);
    uint4 qf[1][T::KS];
    if (!loader) load_query<HD>(rq, qvalid ? static_cast<uint32_t>((m * a.Hq + h) * HD * 2) : kOob, qf[0]);

    float run_m[1] = {kNegInf}, run_l[1] = {0.f};
    f32x4 o[1][T::DT];
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) o[0][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    int buf = 0;
    for (int kb = key0; kb < key1; kb += kStageKeys) {
        if (requester) vm_drain();
        __syncthreads();                           // stage kb is in LDS; the other buffer is free
        if (requester && kb + kStageKeys < key1) request_stage(kb + kStageKeys, buf ^ 1);
        const uint8_t* sK = smem + buf * 2 * kStageBytes;
        const int sb = 64 * half, nst = min(kStageKeys, key1 - kb);
        if (!loader && sb < nst)                   // wave-uniform
            attend_block<HD, 4, 1>(sK + sb * T::RB, sK + kStageBytes + sb * T::RB, min(64, nst - sb), qf,
                                   a.scale_log2, run_m, run_l, o);
        __syncthreads();                           // this buffer is consumed
        buf ^= 1;
    }
    // merge the second half's state into the first (per-lane partial denominators are
    // rescaled like the outputs; the rescale factor is uniform over a query's four lanes)
    float* xs = reinterpret_cast<float*>(smem) + qw * (T::DT * 4 + 2) * 64 + lane;
    if (!loader && half == 1) {
#pragma unroll
        for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
            for (int e = 0; e < 4; ++e) xs[(dt * 4 + e) * 64] = o[0][dt][e];
        xs[T::DT * 4 * 64] = run_m[0];
        xs[(T::DT * 4 + 1) * 64] = run_l[0];
    }
    __syncthreads();
    if (loader || half == 1) return;
    float rm = run_m[0], rl = run_l[0];
    {
        const float m1 = xs[T::DT * 4 * 64], l1 = xs[(T::DT * 4 + 1) * 64];
        const float nm = fmaxf(rm, m1);
        const float w0 = rm == kNegInf ? 0.f : exp2f(rm - nm);
        const float w1 = m1 == kNegInf ? 0.f : exp2f(m1 - nm);
        rl = rl * w0 + l1 * w1;
#pragma unroll
        for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
            for (int e = 0; e < 4; ++e) o[0][dt][e] = o[0][dt][e] * w0 + xs[(dt * 4 + e) * 64] * w1;
        rm = nm;
    }
    rl = sum_rows4(rl);
    if (!qvalid) return;
    const size_t base = (static_cast<size_t>(chunk) * a.m_cap + m) * a.Hq + h;
    if ((lane >> 4) == 0)
        *reinterpret_cast<float2*>(a.part_ml + 2 * base) = make_float2(rm, rl);
    float* po = a.part_o + base * HD + 4 * (lane >> 4);
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) *reinterpret_cast<f32x4*>(po + dt * 16) = o[0][dt];
}

// grid: x = branch, y = KV group, z = query tile (16 positions x 1 head).  One wave per
// workgroup: the chunk states a tile merges are its largest input, and single-wave workgroups
// spread them over as many CUs as there are tiles.
template <int HD, int NKT>
__global__ __launch_bounds__(64) void attn_block_kernel(const AttnArgs a) {
    using T = AttnTile<HD>;
    constexpr int kBatch = 4;                      // prefix chunk states loaded per round trip
    __shared__ __align__(16) uint8_t sK[16 * NKT * T::RB];
    __shared__ __align__(16) uint8_t sV[16 * NKT * T::RB];
    __shared__ int sSlot[64];
    const int G = a.Hq / a.Hkv, N = a.N;
    const int i = blockIdx.x, g = blockIdx.y;
    const int M = clamp_count(a.m_count, a.m_cap);
    const int nt16 = (N + 15) >> 4;
    const int lane = threadIdx.x;
    const int qt = blockIdx.z;

    int s_own = -1;
    if (lane < N) {
        s_own = a.src_slot[i * N + lane];
        if (s_own < 0 || s_own >= M) s_own = -2;
    }
    const bool any_bad = __ballot(s_own == -2) != 0;   // some position has no valid source
    sSlot[lane] = s_own < 0 ? -1 : s_own;
    __syncthreads();
    const uint32_t rows_bytes = static_cast<uint32_t>(static_cast<size_t>(a.m_cap) * a.Hkv * HD * 2);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k_c, rows_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v_c, rows_bytes);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q_c, static_cast<uint32_t>(static_cast<size_t>(a.m_cap) * a.Hq * HD * 2));
    request_rows<HD, 16 * NKT, 1>(rk, rv, sK, sV, [&](int row, int) -> int {
        const int s = row < N ? sSlot[row] : -1;
        return s < 0 ? -1 : (s * a.Hkv + g) * HD;
    });

    const bool active = qt < G * nt16;             // wave-uniform
    const int j = active ? qt / nt16 : 0, nt = active ? qt - j * nt16 : 0;
    const int h = g * G + j;
    const int n = nt * 16 + (lane & 15);
    const bool nvalid = active && n < N;
    const int qslot = nvalid ? sSlot[n] : -1;
    uint4 qf[1][T::KS];
    load_query<HD>(rq, qslot >= 0 ? static_cast<uint32_t>((qslot * a.Hq + h) * HD * 2) : kOob, qf[0]);

    // prefix chunk states of the source slot: the first batch is requested now, so it arrives
    // with the block's keys
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
    // the states are requested last, so waiting until only they are outstanding means the
    // keys (in LDS) and the query have landed; the block part runs while the states arrive
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    load_states(0);
    __builtin_amdgcn_sched_barrier(0);
    vm_wait_le_states<kBatch * (1 + T::DT)>();
    __syncthreads();
    if (!active) return;

    float bm[1] = {kNegInf}, bl[1] = {0.f};
    f32x4 bo[1][T::DT];
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) bo[0][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    attend_block<HD, NKT, 1>(sK, sV, N, qf, a.scale_log2, bm, bl, bo);
    float run_m = bm[0], run_l = sum_rows4(bl[0]);
    f32x4 o[T::DT];
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) o[dt] = bo[0][dt];

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
    const bool bad = (qslot < 0) || any_bad;
    const float invL = bad ? __builtin_nanf("") : 1.0f / run_l;
    const int row = i * N + n;
    uint16_t* dst = a.attn + (static_cast<size_t>(row) * a.Hq + h) * HD + 4 * (lane >> 4);
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) {
        const f32x4 v = o[dt] * invL;
        *reinterpret_cast<uint2*>(dst + dt * 16) = make_uint2(cvt_bf16x2(v[0], v[1]), cvt_bf16x2(v[2], v[3]));
    }
    if (a.lse && (lane >> 4) == 0)
        a.lse[static_cast<size_t>(row) * a.Hq + h] = bad ? __builtin_nanf("") : (run_m + log2f(run_l)) * 0.69314718055994531f;
}

template <int HD, int QT, int LW>
hipError_t launch_prefix_qt(const AttnArgs& a, hipStream_t st) {
    // one LDS stage holds the whole chunk, else two alternate
    const size_t stage = static_cast<size_t>(2) * kStageKeys * AttnTile<HD>::RB;
    const size_t lds = (a.chunk_len > kStageKeys ? 2 : 1) * stage;
    static_assert(QT * (AttnTile<HD>::DT * 4 + 2) * 64 * 4 <= 2 * kStageKeys * AttnTile<HD>::RB,
                  "the merge exchange fits in one stage");
    const int G = a.Hq / a.Hkv;
    const dim3 grid(a.n_chunks * a.Hkv, (a.m_cap * G + 16 * QT - 1) / (16 * QT));
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_prefix_kernel<HD, QT, LW>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_prefix_kernel<HD, QT, LW>), grid, dim3(128 * QT + 64 * LW), lds, st, a);
    return hipGetLastError();
}

// Two query tiles per workgroup while their workgroups fit on the CUs at once (fewer waves per
// CU read each block from LDS); four once two would need a second round, where sharing each
// K/V stage over more queries pays.  A chunk of one stage leaves room for two workgroups per
// CU, a longer one (two stage buffers) for one.  The recompute count is known on the device
// only; the tiles are planned for plan_rows recompute rows (the layer passes all rows when its
// threshold folds nothing but exact copies, else half of them, the pages' fold ratios being
// 0.5-0.7).  Measured: the 7B layer at P = 2048
// (M = 100, 352 busy two-tile workgroups) 28.3 against 18.9 us with four; the 1.5B layer at
// P = 2048 (M = 108, 168 busy) 14.0 against 15.5.
template <int HD>
hipError_t launch_prefix_hd(const AttnArgs& a, hipStream_t st) {
    const int G = a.Hq / a.Hkv;
    const long slots = a.chunk_len > kStageKeys ? 256 : 512;
    const int rows = a.plan_rows > 0 ? (a.plan_rows < a.m_cap ? a.plan_rows : a.m_cap) : (a.m_cap + 1) / 2;
    const long busy2 = static_cast<long>(a.n_chunks) * a.Hkv * ((rows * G + 31) / 32);
    const bool multi = a.chunk_len > kStageKeys;
    if (busy2 <= slots) return multi ? launch_prefix_qt<HD, 2, 4>(a, st) : launch_prefix_qt<HD, 2, 0>(a, st);
    return multi ? launch_prefix_qt<HD, 4, 4>(a, st) : launch_prefix_qt<HD, 4, 0>(a, st);
}

template <int HD>
void launch_block_hd(const AttnArgs& a, dim3 grid, hipStream_t st) {
    // blocks of up to 32 positions take the 32-key form (no MFMAs or fragment reads on padding)
    if (a.N <= 32) hipLaunchKernelGGL((attn_block_kernel<HD, 2>), grid, dim3(64), 0, st, a);
    else hipLaunchKernelGGL((attn_block_kernel<HD, 4>), grid, dim3(64), 0, st, a);
}

}  // namespace

hipError_t launch_attn_prefix(const AttnArgs& a, hipStream_t st) {
    if (a.n_chunks <= 0) return hipSuccess;
    if (a.chunk_len <= 0 || a.chunk_len % 64 != 0) return hipErrorInvalidValue;
    switch (a.hd) {
        case 16: return launch_prefix_hd<16>(a, st);
        case 32: return launch_prefix_hd<32>(a, st);
        case 64: return launch_prefix_hd<64>(a, st);
        case 128: return launch_prefix_hd<128>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_attn_block(const AttnArgs& a, hipStream_t st) {
    if (a.N > 64) return hipErrorInvalidValue;
    const int G = a.Hq / a.Hkv;
    const dim3 grid(a.nb, a.Hkv, G * ((a.N + 15) / 16));
    switch (a.hd) {
        case 16: launch_block_hd<16>(a, grid, st); break;
        case 32: launch_block_hd<32>(a, grid, st); break;
        case 64: launch_block_hd<64>(a, grid, st); break;
        case 128: launch_block_hd<128>(a, grid, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace specfold
