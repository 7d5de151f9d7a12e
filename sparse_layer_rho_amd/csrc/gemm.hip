// Gathered-row bf16 GEMM on gfx950 MFMA: C[m][n] = sum_k A[row(m)][k] * W[n][k].
//
// The layer's projections are skinny: M (recompute rows, <= R = 288 at B = 8, N = 32) is small
// and W [Nout][K] is large, so the kernel is built to stream W from HBM at full rate:
//   * a 256-thread workgroup (4 waves) owns NT 16-row weight tiles (16*NT output columns), a
//     chunk of 64*MTW activation rows and a range of K (grid.y splits K when the column tiles
//     alone cannot fill the 256 CUs);
//   * K advances in stages of 256: for its stage every wave loads 2 weight rows x 512 contiguous
//     bytes per instruction (the access pattern HBM serves fastest), one stage ahead into
//     registers, and writes them into LDS in an XOR-swizzled row-major layout, so the MFMA
//     fragment reads (16 rows x 16 bytes per lane group) are conflict-free ds_read_b128;
//   * each wave loads its own activation row tiles straight into registers in MFMA operand
//     layout (they are L2-resident), double-buffered, so activations never touch LDS;
//   * loads are branch-free: rows past M, column tiles past Nout and K past the split use
//     out-of-range buffer offsets, which read as zeros without touching memory, and every wait
//     is the compiler's own exact vmcnt;
//   * v_mfma_f32_16x16x32_bf16 with a weight fragment as the A operand and 16 activation rows
//     as the B operand leaves each lane 4 consecutive output columns of one row.
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

// Out-of-range offsets: a missing row / column tile adds kOobRow, K past the split adds kOobK.
// Buffers are < 1 GB (checked by the host), so any sum involving either is out of range and the
// two never wrap back into range together.
constexpr uint32_t kOobRow = 0x40000000u;
constexpr uint32_t kOobK = 0x80000000u;
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr int kStageK = 256;                // K elements per stage (512 bytes of a bf16 row)

enum { EPI_PARTIAL = 0, EPI_SWIGLU = 1 };

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kRsrcWord3);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ void block_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

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

template <int NT, int MTW, int EPI>
__global__ __launch_bounds__(256, 1) void gemm_kernel(const GemmArgs p) {
    constexpr int WROWS = 16 * NT;                 // weight rows per workgroup
    constexpr int WBUF = WROWS * 512;              // LDS bytes of one weight stage
    constexpr int WLD = WROWS / 8;                 // 16-byte weight loads per lane per stage
    constexpr int MP = 64 * MTW;                   // activation rows per workgroup
    static_assert(NT % 2 == 0 && WLD >= 1, "tile shape");
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ int s_tot[4];
    int32_t* s_rows = reinterpret_cast<int32_t*>(smem + 2 * WBUF);

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
    const int mrows = min(MP, M - m0);
    const int mtiles = __builtin_amdgcn_readfirstlane((mrows + 15) >> 4);

    // K range of this split (in 32-wide k-steps) and its stages of 256
    const int nks = p.K / 32;
    const int k_begin = static_cast<int>(static_cast<int64_t>(y) * nks / S) * 32;
    const int k_end = static_cast<int>(static_cast<int64_t>(y + 1) * nks / S) * 32;
    const int nstages = (k_end - k_begin + kStageK - 1) / kStageK;

    auto col_of = [&](int nt) -> int {             // first output column of N-tile nt
        if (EPI == EPI_SWIGLU) {
            const int j0 = tile * (NT / 2) * 16;
            return nt < NT / 2 ? j0 + nt * 16 : p.F + j0 + (nt - NT / 2) * 16;
        }
        return (tile * NT + nt) * 16;
    };
    auto col_ok = [&](int nt) -> bool {
        return EPI == EPI_SWIGLU ? (tile * (NT / 2) + (nt % (NT / 2))) * 16 < p.F : col_of(nt) < p.Nout;
    };

    // ---- weight loads: load q of this lane covers weight row r = (q*4 + wave)*2 + lane/32
    // (of the tile's WROWS rows) and 16-byte chunk lane%32 of the stage's 512 bytes
    const __amdgpu_buffer_rsrc_t rW = make_rsrc(p.W, static_cast<uint32_t>(static_cast<size_t>(p.Nout) * p.K * 2));
    const int wchunk = lane & 31;
    uint32_t wrow_off[WLD];
    uint32_t wlds[WLD];
#pragma unroll
    for (int q = 0; q < WLD; ++q) {
        const int r = (q * 4 + wave) * 2 + (lane >> 5);
        const int nt = r >> 4, rr = r & 15;
        wrow_off[q] = col_ok(nt) ? static_cast<uint32_t>((static_cast<size_t>(col_of(nt)) + rr) * p.K * 2) : kOobRow;
        wlds[q] = static_cast<uint32_t>(r * 512 + ((wchunk ^ rr) << 4));   // swizzled LDS slot
    }
    auto load_w = [&](int st, uint4 (&w)[WLD]) {
        const int k = k_begin + st * kStageK + wchunk * 8;
        const uint32_t kb = k < k_end ? static_cast<uint32_t>(k * 2) : kOobK;
#pragma unroll
        for (int q = 0; q < WLD; ++q) w[q] = buf_load16(rW, wrow_off[q] + kb);
    };
    auto store_w = [&](int buf, const uint4 (&w)[WLD]) {
        uint8_t* b = smem + buf * WBUF;
#pragma unroll
        for (int q = 0; q < WLD; ++q) *reinterpret_cast<uint4*>(b + wlds[q]) = w[q];
    };

    // ---- activation loads: tile i of this wave = rows m0 + (wave + 4i)*16 + lane%16; k-step s of
    // a stage reads logical chunk 4s + lane/16 (8 bf16) -- the MFMA B operand
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A, static_cast<uint32_t>(static_cast<size_t>(p.a_row_limit) * p.lda * 2));
    uint32_t arow_off[MTW];
#pragma unroll
    for (int i = 0; i < MTW; ++i) {
        const int m = (wave + 4 * i) * 16 + (lane & 15);
        uint32_t o = kOobRow;
        if (m < mrows) {
            const int src = fused ? s_rows[m0 + m] : (p.a_rows ? p.a_rows[m0 + m] : m0 + m);
            if (src >= 0 && src < p.a_row_limit) o = static_cast<uint32_t>(static_cast<size_t>(src) * p.lda * 2);
        }
        arow_off[i] = o;
    }

    // the stage loop, specialised on this wave's number of active row tiles (no branch sits
    // between the MFMAs) and unrolled by two for the register double buffers
    auto run = [&](auto nact_c) {
        constexpr int NACT = decltype(nact_c)::value;
        constexpr int NA = NACT > 0 ? NACT : 1;
        f32x4 acc[NA][NT];
#pragma unroll
        for (int i = 0; i < NA; ++i)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[i][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        uint4 w0[WLD], w1[WLD];
        uint4 a0[NA][8], a1[NA][8];

        auto load_a = [&](int st, uint4 (&a)[NA][8]) {
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const int k = k_begin + st * kStageK + (4 * s + (lane >> 4)) * 8;
                const uint32_t kb = k < k_end ? static_cast<uint32_t>(k * 2) : kOobK;
#pragma unroll
                for (int i = 0; i < NACT; ++i) a[i][s] = buf_load16(rA, arow_off[i] + kb);
            }
        };
        auto compute = [&](int buf, const uint4 (&a)[NA][8]) {
            const uint8_t* b = smem + buf * WBUF;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                uint4 wf[NT];
                const int c = 4 * s + (lane >> 4);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const int r = nt * 16 + (lane & 15);
                    wf[nt] = *reinterpret_cast<const uint4*>(b + r * 512 + ((c ^ (lane & 15)) << 4));
                }
#pragma unroll
                for (int i = 0; i < NACT; ++i)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) acc[i][nt] = mfma16x16x32(wf[nt], a[i][s], acc[i][nt]);
            }
        };

        // stage it: W(it) in registers -> LDS buffer it%2 while W(it+1), A(it+1) are in flight
        load_w(0, w0);
        load_a(0, a0);
        load_w(1, w1);
        for (int it = 0; it < nstages; it += 2) {
            store_w(0, w0);
            block_barrier();
            load_w(it + 2, w0);
            load_a(it + 1, a1);
            compute(0, a0);

            store_w(1, w1);
            block_barrier();
            load_w(it + 3, w1);
            load_a(it + 2, a0);
            compute(1, a1);
        }

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
    dispatch_count<MTW>(nact, run);
}

template <int NT, int MTW, int EPI>
hipError_t launch_shape(GemmArgs a, int n_tiles, int splits, hipStream_t st) {
    constexpr int MP = 64 * MTW;
    a.n_tiles = n_tiles;
    a.m_chunks = (a.m_cap + MP - 1) / MP;
    if (a.m_chunks < 1) a.m_chunks = 1;
    const size_t lds = 2 * static_cast<size_t>(16 * NT * 512) + (a.fc_fold ? static_cast<size_t>(a.fc_R) * 4 : 0);
    auto kern = gemm_kernel<NT, MTW, EPI>;
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
    // a tile of 16*NT weight rows covers 16*NT output columns (SwiGLU: 8*NT gate + 8*NT up rows)
    const int per = (EPI == EPI_SWIGLU ? 8 : 16) * nt;
    const int tiles = (n_cols + per - 1) / per;
    if (nt == 8) {
        if (max_rows <= 64) return launch_shape<8, 1, EPI>(a, tiles, splits, st);
        return launch_shape<8, 2, EPI>(a, tiles, splits, st);
    }
    if (max_rows <= 64) return launch_shape<4, 1, EPI>(a, tiles, splits, st);
    return launch_shape<4, 2, EPI>(a, tiles, splits, st);
}

}  // namespace

hipError_t launch_gemm_partial(const GemmArgs& a, int splits, int max_rows, int nt, hipStream_t st) {
    return launch_cfg<EPI_PARTIAL>(a, nt, a.Nout, splits, max_rows, st);
}

hipError_t launch_gemm_swiglu(const GemmArgs& a, int max_rows, int nt, hipStream_t st) {
    return launch_cfg<EPI_SWIGLU>(a, nt, a.F, 1, max_rows, st);
}

}  // namespace specfold
