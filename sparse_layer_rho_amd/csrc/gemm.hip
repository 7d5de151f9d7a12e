// Gathered-row bf16 GEMM on gfx950 MFMA: C[m][n] = sum_k A[row(m)][k] * W[n][k].
//
// The layer's projections are skinny: M (recompute rows, <= R = 288 at B = 8, N = 32) is small
// and W [Nout][K] is large, so the kernel is built to stream W once from HBM at full rate:
//   * a 256-thread workgroup (4 waves) owns NT 16-column tiles over all M rows and a range of K
//     (grid.y splits K when the column tiles alone cannot fill the 256 CUs);
//   * both operands move HBM/L2 -> LDS by buffer_load ... lds (no register staging) into a ring
//     of ST stages, each stage holding KS 32-wide k-steps in MFMA fragment order (lane l's
//     16 bytes at lane*16, so every LDS read is a conflict-free ds_read_b128);
//   * addresses are branch-free: rows past M, column tiles past Nout and k-steps past the split
//     use out-of-range buffer offsets, which read as zeros without touching memory -- so the
//     number of loads in flight is static and the waits are exact vmcnt counts;
//   * the 4 waves split the M tiles and share the weight fragments; v_mfma_f32_16x16x32_bf16
//     with a weight fragment as the A operand and 16 activation rows as the B operand leaves
//     each lane 4 consecutive output columns of one row.
// Rows come from an identity map, a device list, or -- fused -- from the fold flags: every
// workgroup compacts them in LDS (ascending row order) and workgroup (0,0) also publishes the
// recompute list, per-branch offsets, row -> slot map and fold sources
// [SpecFold summary, App. B: compaction and source resolution feed the projection].
// Epilogues: fp32 partial sums (reduced in a fixed order by the next kernel, so results are
// deterministic), or SwiGLU for the FFN's gate/up projection, where gate tile t and up tile
// t + NT/2 meet in the same lane.
#include <type_traits>

#include "kernels.h"

namespace specfold {

namespace {

constexpr uint32_t kOobRow = 0x40000000u;   // offset of a missing row / column tile (>= any buffer)
constexpr uint32_t kOobK = 0x80000000u;     // added to every offset of a k-step past the split
constexpr uint32_t kRsrcWord3 = 0x00020000u;

enum { EPI_PARTIAL = 0, EPI_SWIGLU = 1 };

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kRsrcWord3);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
    typedef __attribute__((address_space(3))) void lds_void;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(lds), 16, voff, 0, 0, 0);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// ds_read_b128 issued as inline asm: the compiler cannot prove these reads miss the LDS bytes
// that in-flight DMA is writing and would otherwise wait for all DMA before every read; the
// ring-buffer protocol (exact vmcnt + barrier) already orders them.  Results are only valid
// after lds_wait().
__device__ __forceinline__ u32x4 lds_read16(const uint8_t* p) {
    u32x4 v;
    const uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_u8*)(p)));
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(a));
    return v;
}

// wait for every issued LDS read and pin the fragments after the wait
template <int N>
__device__ __forceinline__ void lds_wait(u32x4 (&v)[N]) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(v[i]));
}

__device__ __forceinline__ uint4 as_uint4(const u32x4& v) { return make_uint4(v.x, v.y, v.z, v.w); }

// call f(std::integral_constant<int, n>) for a runtime n in [0, MAX]
template <int MAX, int N = 0, typename F>
__device__ __forceinline__ void dispatch_count(int n, F&& f) {
    if constexpr (N < MAX) {
        if (n == N) f(std::integral_constant<int, N>{});
        else dispatch_count<MAX, N + 1>(n, f);
    } else {
        f(std::integral_constant<int, MAX>{});
    }
}

__device__ __forceinline__ void block_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Compact the recompute rows (fold == 0) of R rows into s_rows (ascending), 256 threads.
// Returns M.  When publish, also writes the global list, offsets, row_slot and fold sources.
__device__ int compact_in_lds(const GemmArgs& p, int32_t* s_rows, int* s_tot, bool publish) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int R = p.fc_R, N = p.fc_N;
    int base = 0;
    for (int r0 = 0; r0 < R; r0 += 256) {
        const int r = r0 + tid;
        const bool rec = (r < R) && (p.fc_fold[r] == 0);
        const uint64_t m = __ballot(rec);
        const int excl = __popcll(m & ((1ull << lane) - 1ull));
        if (lane == 0) s_tot[wave] = __popcll(m);
        __syncthreads();
        const int t0 = s_tot[0], t1 = s_tot[1], t2 = s_tot[2], t3 = s_tot[3];
        const int woff = (wave > 0 ? t0 : 0) + (wave > 1 ? t1 : 0) + (wave > 2 ? t2 : 0);
        const int slot = base + woff + excl;
        if (rec) s_rows[slot] = r;
        if (publish && r < R) {
            p.fc_row_slot[r] = rec ? slot : -1;
            if (rec) p.fc_rec_rows[slot] = r;
            if (r % N == 0) p.fc_branch_off[r / N] = slot;
        }
        base += t0 + t1 + t2 + t3;
        __syncthreads();
    }
    if (publish) {
        if (tid == 0) {
            p.fc_rec_count[0] = base;
            p.fc_branch_off[p.fc_nb] = base;
            if (p.fc_count_copy) p.fc_count_copy[0] = base;
        }
        // fold sources: walk each row's chain up the parent map (branch 0 terminates);
        // slots come from the LDS list by binary search
        for (int r = tid; r < R; r += 256) {
            const int i = r / N, n = r - i * N;
            int j = i;
            for (int s = 0; s < p.fc_nb && j > 0 && p.fc_fold[j * N + n] != 0; ++s) j = p.fc_par.p[j];
            const int src_row = j * N + n;
            int lo = 0, hi = base;                   // first slot with s_rows[slot] >= src_row
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (s_rows[mid] < src_row) lo = mid + 1; else hi = mid;
            }
            const int slot = (lo < base && s_rows[lo] == src_row) ? lo : -1;
            p.fc_src_branch[r] = j;
            p.fc_src_slot[r] = slot;
            if (p.fc_src_slot_copy) p.fc_src_slot_copy[r] = slot;
        }
    }
    __syncthreads();
    return base;
}

template <int NT, int MTW, int KS, int ST, int EPI>
__global__ __launch_bounds__(256, 1) void gemm_kernel(const GemmArgs p) {
    constexpr int MP = 4 * MTW * 16;                       // rows per pass
    constexpr int W_FR = KS * NT;                          // weight fragments per stage
    constexpr int A_FR = 4 * MTW * KS;                     // activation fragments per stage
    constexpr int STAGE = (W_FR + A_FR) * 1024;            // bytes per stage
    constexpr int WLOADS = W_FR / 4;                       // weight DMA per wave per stage
    constexpr int LPS = WLOADS + MTW * KS;                 // DMA per wave per stage
    static_assert(NT % 4 == 0, "weight fragments must split over 4 waves");
    static_assert((ST - 2) * LPS < 64, "vmcnt range");
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ int s_tot[4];
    int32_t* s_rows = reinterpret_cast<int32_t*>(smem + ST * STAGE);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar branches
    const int y = blockIdx.y, S = gridDim.y;
    // blockIdx.x -> (column tile, row chunk).  Consecutive workgroup ids go round-robin over the
    // 8 XCDs, so the chunks of one tile get ids that share id % 8 and sit within 8*C of each
    // other: they run on one XCD at about the same time and the tile's weights come from that
    // XCD's L2 after the first chunk fetched them.
    const int C = p.m_chunks;
    const int id = blockIdx.x, grp = id / (8 * C), rem = id - grp * 8 * C;
    const int chunk = rem >> 3, tile = grp * 8 + (rem & 7);

    int M;
    const bool fused = p.fc_fold != nullptr;
    if (fused) {
        M = compact_in_lds(p, s_rows, s_tot, blockIdx.x == 0 && blockIdx.y == 0);   // (tile 0, chunk 0)
    } else {
        M = p.m_count ? p.m_count[0] : p.m_fixed;
    }
    M = M < 0 ? 0 : (M > p.m_cap ? p.m_cap : M);
    M = __builtin_amdgcn_readfirstlane(M);
    const int m0 = chunk * MP;
    if (tile >= p.n_tiles || m0 >= M) return;     // uniform: nothing for this workgroup

    // k-steps (32 wide) of this split, grouped in stages of KS
    const int nks = p.K / 32;
    const int ks0 = static_cast<int>(static_cast<int64_t>(y) * nks / S);
    const int ks1 = static_cast<int>(static_cast<int64_t>(y + 1) * nks / S);
    const int nstages = (ks1 - ks0 + KS - 1) / KS;

    // weight fragment rows: fragment f = s*NT + nt, loaded by wave f % 4
    const __amdgpu_buffer_rsrc_t rW = make_rsrc(p.W, static_cast<uint32_t>(static_cast<size_t>(p.Nout) * p.K * 2));
    const int bx = tile;
    auto col_of = [&](int nt) -> int {
        if (EPI == EPI_SWIGLU) {
            const int j0 = bx * (NT / 2) * 16;
            return nt < NT / 2 ? j0 + nt * 16 : p.F + j0 + (nt - NT / 2) * 16;
        }
        return (bx * NT + nt) * 16;
    };
    auto col_ok = [&](int nt) -> bool {
        return EPI == EPI_SWIGLU ? (bx * (NT / 2) + (nt % (NT / 2))) * 16 < p.F : col_of(nt) < p.Nout;
    };
    // wave w loads fragments f = 4q + w; with NT % 4 == 0 its k-step (4q)/NT is static
    uint32_t woff[WLOADS];
#pragma unroll
    for (int q = 0; q < WLOADS; ++q) {
        const int nt = (4 * q) % NT + wave;   // its k-step is added per stage (kadd)
        woff[q] = col_ok(nt) ? static_cast<uint32_t>(((static_cast<size_t>(col_of(nt)) + (lane & 15)) * p.K +
                                                     8 * (lane >> 4)) * 2)
                             : kOobRow;
    }
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A, static_cast<uint32_t>(static_cast<size_t>(p.a_row_limit) * p.lda * 2));

    {
        const int mrows = min(MP, M - m0);
        const int mtiles = __builtin_amdgcn_readfirstlane((mrows + 15) >> 4);
        uint32_t aoff[MTW];
#pragma unroll
        for (int i = 0; i < MTW; ++i) {
            const int m = (wave + 4 * i) * 16 + (lane & 15);
            uint32_t o = kOobRow;
            if (m < mrows) {
                const int src = fused ? s_rows[m0 + m] : (p.a_rows ? p.a_rows[m0 + m] : m0 + m);
                if (src >= 0 && src < p.a_row_limit)
                    o = static_cast<uint32_t>((static_cast<size_t>(src) * p.lda + 8 * (lane >> 4)) * 2);
            }
            aoff[i] = o;
        }

        auto issue = [&](int stage, int kstage) {
            uint8_t* sb = smem + stage * STAGE;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const int ks = ks0 + kstage * KS + s;
                const uint32_t kadd = ks < ks1 ? static_cast<uint32_t>(ks * 64) : kOobK;
#pragma unroll
                for (int q = 0; q < WLOADS; ++q)
                    if ((4 * q) / NT == s) lds_dma16(rW, sb + (4 * q + wave) * 1024, woff[q] + kadd);
#pragma unroll
                for (int i = 0; i < MTW; ++i)
                    lds_dma16(rA, sb + (W_FR + (wave * MTW + i) * KS + s) * 1024, aoff[i] + kadd);
            }
        };

#pragma unroll
        for (int st = 0; st < ST - 1; ++st) issue(st, st);

        // the k-loop, specialised on this wave's number of active row tiles so no branch sits
        // between the MFMAs and the accumulators stay in place across iterations
        auto kloop = [&](auto nact_c) {
            constexpr int NACT = decltype(nact_c)::value;
            constexpr int NA = NACT > 0 ? NACT : 1;
            f32x4 acc[NA][NT];
#pragma unroll
            for (int i = 0; i < NA; ++i)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) acc[i][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int it = 0; it < nstages; ++it) {
                wait_vmcnt<(ST - 2) * LPS>();
                block_barrier();
                const int nxt = it + ST - 1;
                issue(nxt % ST, nxt);
                const uint8_t* sb = smem + (it % ST) * STAGE;
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    u32x4 fr[NT + (NACT > 0 ? NACT : 1)];
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) fr[nt] = lds_read16(sb + (s * NT + nt) * 1024 + lane * 16);
#pragma unroll
                    for (int i = 0; i < NACT; ++i)
                        fr[NT + i] = lds_read16(sb + (W_FR + (wave * MTW + i) * KS + s) * 1024 + lane * 16);
                    if (NACT == 0) fr[NT] = u32x4{0u, 0u, 0u, 0u};
                    lds_wait(fr);
#pragma unroll
                    for (int i = 0; i < NACT; ++i) {
                        const uint4 a = as_uint4(fr[NT + i]);
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt)
                            acc[i][nt] = mfma16x16x32(as_uint4(fr[nt]), a, acc[i][nt]);
                    }
                }
            }
            wait_vmcnt<0>();
            block_barrier();

            // epilogue: lane holds C[row m][cols col + 4*(lane>>4) + q]
#pragma unroll
            for (int i = 0; i < NACT; ++i) {
                const int m = (wave + 4 * i) * 16 + (lane & 15);
                if (m >= mrows) continue;
                if (EPI == EPI_SWIGLU) {
#pragma unroll
                    for (int nt = 0; nt < NT / 2; ++nt) {
                        if (!col_ok(nt)) continue;
                        float o[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float g = acc[i][nt][q], u = acc[i][nt + NT / 2][q];
                            o[q] = g / (1.0f + expf(-g)) * u;
                        }
                        *reinterpret_cast<uint2*>(p.act + static_cast<size_t>(m0 + m) * p.F + col_of(nt) + 4 * (lane >> 4)) =
                            make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
                    }
                } else {
                    float* dst = p.partial + (static_cast<size_t>(y) * p.m_cap + m0 + m) * p.Nout + 4 * (lane >> 4);
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        if (col_ok(nt)) *reinterpret_cast<f32x4*>(dst + col_of(nt)) = acc[i][nt];
                }
            }
        };
        // active tiles of this wave: i with wave + 4 i < mtiles
        const int nact = mtiles > wave ? min(MTW, (mtiles - wave + 3) >> 2) : 0;
        dispatch_count<MTW>(nact, kloop);
    }
}

// Kernel shapes: NT column tiles per workgroup, MTW row tiles per wave (64*MTW rows per
// workgroup), KS k-steps per stage, ST stages.  LDS = ST*(KS*NT + 4*MTW*KS) KB + the row list.
template <int NT, int MTW, int KS, int ST, int EPI>
hipError_t launch_shape(GemmArgs a, int n_tiles, int splits, hipStream_t st) {
    constexpr int STAGE = (KS * NT + 4 * MTW * KS) * 1024;
    constexpr int MP = 64 * MTW;
    a.n_tiles = n_tiles;
    a.m_chunks = (a.m_cap + MP - 1) / MP;
    if (a.m_chunks < 1) a.m_chunks = 1;
    const size_t lds = static_cast<size_t>(ST) * STAGE + (a.fc_fold ? static_cast<size_t>(a.fc_R) * 4 : 0);
    auto kern = gemm_kernel<NT, MTW, KS, ST, EPI>;
    static size_t configured = 0;   // dynamic-LDS cap raised so far for this kernel
    if (lds > configured) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (e != hipSuccess) return e;
        configured = lds;
    }
    const dim3 grid(((n_tiles + 7) / 8) * 8 * a.m_chunks, splits);
    hipLaunchKernelGGL(kern, grid, dim3(256), lds, st, a);
    return hipGetLastError();
}

template <int EPI>
hipError_t launch_cfg(const GemmArgs& a, int nt, int n_cols, int splits, int max_rows, hipStream_t st) {
    // n_cols: output columns one tile of 16*NT weight rows stands for (SwiGLU pairs gate + up)
    if (nt == 8) {
        const int tiles = (n_cols + (EPI == EPI_SWIGLU ? 64 : 128) - 1) / (EPI == EPI_SWIGLU ? 64 : 128);
        if (max_rows <= 64) return launch_shape<8, 1, 2, 6, EPI>(a, tiles, splits, st);    // 6 x 24 KB
        return launch_shape<8, 2, 2, 4, EPI>(a, tiles, splits, st);                        // 4 x 32 KB
    }
    const int tiles = (n_cols + (EPI == EPI_SWIGLU ? 32 : 64) - 1) / (EPI == EPI_SWIGLU ? 32 : 64);
    if (max_rows <= 64) return launch_shape<4, 1, 2, 8, EPI>(a, tiles, splits, st);        // 8 x 16 KB
    return launch_shape<4, 2, 2, 5, EPI>(a, tiles, splits, st);                            // 5 x 24 KB
}

}  // namespace

hipError_t launch_gemm_partial(const GemmArgs& a, int splits, int max_rows, int nt, hipStream_t st) {
    return launch_cfg<EPI_PARTIAL>(a, nt, a.Nout, splits, max_rows, st);
}

hipError_t launch_gemm_swiglu(const GemmArgs& a, int max_rows, int nt, hipStream_t st) {
    return launch_cfg<EPI_SWIGLU>(a, nt, a.F, 1, max_rows, st);
}

}  // namespace specfold
