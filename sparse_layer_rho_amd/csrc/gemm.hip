// Gathered-row bf16 GEMM on gfx950 MFMA: C[m][n] = sum_k A[row(m)][k] * W[n][k].
//
// The layer's projections are skinny: M (recompute rows, <= R = 288 at B = 8, N = 32) is small
// and W [Nout][K] is large, so the kernel is built to keep many bytes of W in flight:
//   * a 256-thread workgroup owns 16*NT weight rows (output columns), a chunk of MP activation
//     rows and a range of K (grid.y splits K when the column tiles alone cannot fill the CUs);
//   * K advances in stages of 64 elements.  Both operands of a stage move HBM/L2 -> LDS with
//     buffer_load ... lds (no register staging) into a ring of NB stage slots, so NB-1 stages
//     are in flight while one is multiplied.  One such load moves 8 rows x 128 contiguous
//     bytes: every 4-lane quad reads one 64-byte segment, the pattern the texture path serves
//     at full rate (loads straight into MFMA operand layout would touch four rows per quad);
//   * inside a slot, row r keeps its 16-byte chunk c at position c ^ (r & 7), so the MFMA
//     fragment reads (16 rows x one chunk) are conflict-free ds_read_b128;
//   * the four waves form a (NT/2) x (8/NT) grid over (weight tiles, row tiles); each wave
//     multiplies two 16-row weight tiles with TM 16-row activation tiles per 32-wide k-step;
//   * loads are branch-free: rows past M, weight rows past Nout and K past the matrix use
//     out-of-range buffer offsets, which read as zeros without touching memory;
//   * waits are explicit: the ring's loads write no registers and the fragment reads are
//     inline asm, so the compiler inserts no conservative drains; each wave waits on vmcnt for
//     exactly the stage it is about to read and on lgkmcnt for its fragments.
// Rows come from an identity map, a device list, or -- fused -- from the fold flags: every
// workgroup compacts them in LDS (ascending row order) and the grid's last workgroup, one with
// no tile of the product, also publishes the recompute list, per-branch offsets, row -> slot map
// and fold sources
// [SpecFold summary, App. B: compaction and source resolution feed the projection].
// Epilogues: fp32 partial sums (reduced in a fixed order by the next kernel, so results are
// deterministic), or SwiGLU for the FFN's gate/up projection, where a wave's two weight tiles
// are the gate and up rows of the same 16 output columns.
#include <atomic>

#include "kernels.h"

namespace specfold {

namespace {

// Out-of-range offsets: a missing row adds kOobRow, K past the matrix adds kOobK.  Buffers are
// < 1 GB (checked by the host), so any sum involving either is out of range and the two never
// wrap back into range together.
constexpr uint32_t kOobRow = kOob;
constexpr uint32_t kOobK = 0x80000000u;
constexpr int kStageK = 64;                 // K elements per compute stage
constexpr int kSplitUnit = 128;             // K-splits cut K at multiples of this
constexpr int kRowB = 128;                  // bytes of one activation row in one compute stage

enum { EPI_PARTIAL = 0, EPI_SWIGLU = 1, EPI_ARGMAX = 2 };

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// 16 bytes per lane, global -> LDS: lane l's bytes land at lds + 16 l (lds is wave-uniform)
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(lds), 16, voff, 0, 0, 0);
}

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_u8*)(p)));
}

// ds_read_b128 as inline asm: the compiler cannot see these reads, so it neither drains the
// ring's loads before them nor waits for their results; lds_wait<N>() supplies that wait
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int OFF>
__device__ __forceinline__ u32x4 lds_read16(uint32_t addr) {
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}

// wait until at most N of this wave's LDS reads are outstanding, then pin the fragments after
// the wait (the empty asm "modifies" them, so no use can be scheduled above it)
template <int N, int C>
__device__ __forceinline__ void lds_wait(u32x4 (&v)[C]) {
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(N) : "memory");
#pragma unroll
    for (int i = 0; i < C; ++i) asm volatile("" : "+v"(v[i]));
}

// fragments of N consecutive 16-row tiles (rows 16 apart) at addr
template <int N, int ROWB, int I = 0>
__device__ __forceinline__ void read_tiles(u32x4* f, uint32_t addr) {
    if constexpr (I < N) {
        f[I] = lds_read16<I * 16 * ROWB>(addr);
        read_tiles<N, ROWB, I + 1>(f, addr);
    }
}

// wait until at most N of this wave's vector-memory operations are outstanding
template <int N>
__device__ __forceinline__ void vm_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// wait until at most n of this wave's vector-memory operations are outstanding, for a runtime n
// in [0, MAX] (rounded down to a multiple of STEP: waiting for more is always safe)
template <int STEP, int MAX>
__device__ __forceinline__ void vm_wait_le(int n) {
    if constexpr (MAX <= 0) {
        vm_wait<0>();
    } else {
        if (n >= MAX) vm_wait<MAX>();
        else vm_wait_le<STEP, MAX - STEP>(n);
    }
}

__device__ __forceinline__ f32x4 mma(const u32x4& w, const u32x4& a, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w), __builtin_bit_cast(bf16x8, a), c,
                                                   0, 0, 0);
}

__device__ __forceinline__ void block_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Compact the recompute rows (fold == 0) of R rows into s_rows (ascending), on the first 256
// threads of the workgroup (load waves, where a kernel has them, only pass the barriers).
// Returns M.  When publish, also writes the global list, offsets, row_slot and fold sources.
// The flags of the first kPre * 256 rows are requested in one batch (one memory round trip
// instead of one per 256 rows) and kept in LDS (s_fold), with the parent map, so the source
// walks of the publishing workgroup read no global memory.
__device__ int compact_in_lds(const GemmArgs& p, int32_t* s_rows, uint8_t* s_fold, int* s_tot, int* s_par,
                              bool publish) {
    constexpr int kPre = 4;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool act = tid < 256;
    const int R = p.fc_R, N = p.fc_N;
    if (publish && act && tid < p.fc_nb) s_par[tid] = p.fc_par.p[tid];
    uint8_t pre[kPre];
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
        const int r = k * 256 + tid;
        pre[k] = act && r < R ? p.fc_fold[r] : 1;
    }
    int base = 0;
    auto step = [&](int r0, uint8_t f) {
        const int r = r0 + tid;
        const bool in = act && r < R;
        const bool rec = in && (f == 0);
        if (in) s_fold[r] = f;
        const uint64_t m = __ballot(rec);
        const int excl = __popcll(m & ((1ull << lane) - 1ull));
        if (lane == 0 && act) s_tot[wave] = __popcll(m);
        __syncthreads();
        const int t0 = s_tot[0], t1 = s_tot[1], t2 = s_tot[2], t3 = s_tot[3];
        const int woff = (wave > 0 ? t0 : 0) + (wave > 1 ? t1 : 0) + (wave > 2 ? t2 : 0);
        const int slot = base + woff + excl;
        if (rec) s_rows[slot] = r;
        if (publish && in) {
            p.fc_row_slot[r] = rec ? slot : -1;
            if (rec) p.fc_rec_rows[slot] = r;
            if (r % N == 0) p.fc_branch_off[r / N] = slot;
        }
        base += t0 + t1 + t2 + t3;
        __syncthreads();
    };
#pragma unroll
    for (int k = 0; k < kPre; ++k)
        if (k * 256 < R) step(k * 256, pre[k]);
    for (int r0 = kPre * 256; r0 < R; r0 += 256) step(r0, act && r0 + tid < R ? p.fc_fold[r0 + tid] : 1);
    if (publish) {
        if (tid == 0) {
            p.fc_rec_count[0] = base;
            p.fc_branch_off[p.fc_nb] = base;
            if (p.fc_count_copy) p.fc_count_copy[0] = base;
        }
        // fold sources: walk each row's chain up the parent map (branch 0 terminates);
        // slots come from the LDS list by binary search
        for (int r = tid; act && r < R; r += 256) {
            const int i = r / N, n = r - i * N;
            int j = i;
            for (int s = 0; s < p.fc_nb && j > 0 && s_fold[j * N + n] != 0; ++s) j = s_par[j];
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

// Tile shape: WN x WM waves; each wave owns NTW 16-row weight tiles and TM 16-row activation
// tiles.  Weights and activations have rings of their own.  A weight stage spans KSUB compute
// stages (KSUB * 128 contiguous bytes of every weight row: HBM serves runs of 256 bytes and
// more far better than 128-byte pieces of many rows), NBW weight slots keep NBW-1 weight
// stages in flight; activations (L2-resident) move per compute stage through NBA slots.
template <int NTW, int WN, int TM, int KSUB, int NBW, int NBA>
struct Tile {
    static constexpr int WM = 4 / WN;              // waves along the row tiles
    static constexpr int NT = NTW * WN;            // weight tiles per workgroup
    static constexpr int WROWS = 16 * NT;          // weight rows per workgroup
    static constexpr int MP = 16 * TM * WM;        // activation rows per workgroup
    static constexpr int WRB = KSUB * kRowB;       // bytes of a weight row in one weight stage
    static constexpr int WLPR = WRB / 16;          // lanes per weight row in one ring load
    static constexpr int QW = WROWS * WRB / 4096;  // ring loads per wave per weight stage
    static constexpr int QA = MP / 32;             // ring loads per wave per compute stage
    static constexpr int WSLOT = WROWS * WRB;
    static constexpr int ASLOT = MP * kRowB;
    static constexpr int LDS = NBW * WSLOT + NBA * ASLOT;
    static constexpr int LWU = NBW - 1, LA = NBA - 1;
    // most loads issued after an awaited activation stage (see the ring loop)
    static constexpr int MAXN = (LA - 1) * QA + ((LA + KSUB - 1) / KSUB) * QW;
    static_assert(WN == 1 || WN == 2 || WN == 4, "wave grid");
    static_assert(KSUB == 1 || KSUB == 2 || KSUB == 4, "weight stage");
    static_assert(WROWS * WRB % 4096 == 0 && MP % 32 == 0, "ring loads of 1 KB per wave");
    static_assert(TM >= 1 && NTW >= 1 && NTW * TM <= 16, "accumulators per wave");
    static_assert(NBA >= 2 && NBW >= 2 && KSUB * LWU > LA && MAXN < 64, "ring depths");
};

// One workgroup's share of the product for M rows: workgroup `lin` of a launch with S K-splits
// (smem: the rings, s_rows: the fused compaction's row list).
template <int NTW, int WN, int TM, int KSUB, int NBW, int NBA, int EPI, int LW>
__device__ __forceinline__ void gemm_tile(const GemmArgs& p, const int M, const int lin, const int S, uint8_t* smem,
                                          const int32_t* s_rows) {
    using T = Tile<NTW, WN, TM, KSUB, NBW, NBA>;
    constexpr int MP = T::MP, QW = T::QW, QA = T::QA;
    static_assert(EPI != EPI_SWIGLU || NTW % 2 == 0, "SwiGLU tiles come in gate/up pairs");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar branches
    const int C = p.m_chunks;
    const bool fused = p.fc_fold != nullptr;
    // rows [0, M) split evenly over c_use of the C row workgroups of each group: as many as M
    // needs, but at least min_chunks (two workgroups streaming the same weight tile, the
    // second from L2, run faster than one), decided here because M is only known on the device
    const int c_need = (M + MP - 1) / MP;
    const int c_use = max(1, min(C, max(c_need, p.min_chunks)));
    // linear workgroup id -> (split, column group, row workgroup) over the c_use row
    // workgroups in use: the busy workgroups of all splits take the lowest ids (the grid is
    // sized for C), so consecutive ids -- which the dispatcher deals round-robin to the XCDs
    // and, within an XCD, to its CUs -- spread them evenly over the CUs whatever C, c_use and
    // S are (interleaving idle ids with a period that shares a factor with the CU count would
    // load some CUs twice and leave others idle).  The row workgroups of one group share
    // id % 8 and sit within 8 c_use ids of each other: they run on one XCD at about the same
    // time and the group's weights come from that XCD's L2 after the first fetched them.
    // With xcd_split (S a multiple of 8), the K-splits are placed by XCD instead (consecutive ids
    // go round-robin to the 8 XCDs, so id % 8 names the XCD): XCD x takes the splits y = x
    // (mod 8) of every group, and its L2 fetches the activation columns of its own K ranges only,
    // instead of all of them (8 copies of the activations crossing the fabric per launch).
    int y, chunk, g;
    if (p.xcd_split && S % 8 == 0) {
        const int x = lin & 7, j = lin >> 3;
        const int GC = p.n_groups * c_use;
        const int ys = j / GC;
        if (ys >= S / 8) return;
        const int rem = j - ys * GC;
        y = x + 8 * ys;
        g = rem / c_use;
        chunk = rem - g * c_use;
    } else {
        const int A = ((p.n_groups + 7) / 8) * 8 * c_use;      // busy workgroups per split
        if (lin >= S * A) return;
        y = lin / A;
        const int id = lin - y * A;
        const int grp = id / (8 * c_use), rem = id - grp * 8 * c_use;
        chunk = rem >> 3;
        g = grp * 8 + (rem & 7);
    }
    const int per = (M + c_use - 1) / c_use;   // <= MP
    const int m0 = chunk * per;
    if (g >= p.n_groups || m0 >= M) return;    // uniform: nothing to do here
    const int mrows = min(per, M - m0);

    // output columns [c0, c1) of this group: units of 4 columns (a lane holds 4 consecutive
    // columns), the last unit possibly partial, spread evenly over the groups; the last group
    // ends at ncols.  With ceil(ncols / 4) units no group is wider than the group capacity the
    // host sized the grid for (ncols <= groups * capacity, capacity a multiple of 4).
    // (32-bit unsigned products: the launchers keep groups * units below 2^32, so no 64-bit
    // division, a long scalar sequence, sits in every workgroup's prologue)
    const int ncols = EPI == EPI_SWIGLU ? p.F : p.Nout;
    const uint32_t units = static_cast<uint32_t>(ncols + 3) / 4, ng = static_cast<uint32_t>(p.n_groups);
    const int c0 = static_cast<int>(static_cast<uint32_t>(g) * units / ng) * 4;
    const int c1 = min(ncols, static_cast<int>(static_cast<uint32_t>(g + 1) * units / ng) * 4);

    // K range of this split: whole units of kSplitUnit elements (a multiple of every weight
    // stage), so the split boundaries -- and with them the order in which every output's sum
    // is formed -- depend on K and the split count only, not on the tile shape or the rows
    static_assert(kSplitUnit % (KSUB * kStageK) == 0, "weight stages tile the split unit");
    const int nun = (p.K + kSplitUnit - 1) / kSplitUnit;   // K < 2^29, S <= 32: products fit
    const int u0 = static_cast<int>(static_cast<uint32_t>(y * nun) / static_cast<uint32_t>(S));
    const int u1 = static_cast<int>(static_cast<uint32_t>((y + 1) * nun) / static_cast<uint32_t>(S));
    const int k_begin = u0 * kSplitUnit;
    const int k_stop = min(p.K, u1 * kSplitUnit);
    const int nws = k_stop > k_begin ? (k_stop - k_begin + KSUB * kStageK - 1) / (KSUB * kStageK) : 0;
    const int nst = k_stop > k_begin ? (k_stop - k_begin + kStageK - 1) / kStageK : 0;

    // weight row of slot row r (r < WROWS), or -1 past the group.  SwiGLU slots interleave
    // [gate 16 | up 16] pairs, so a wave's tile pair holds the gate and up rows of 16 columns.
    auto w_row = [&](int r) -> int {
        if (EPI == EPI_SWIGLU) {
            const int col = c0 + (r >> 5) * 16 + (r & 15);
            return col < c1 ? (((r >> 4) & 1) ? p.F + col : col) : -1;
        }
        const int col = c0 + r;
        return col < c1 ? col : -1;
    };

    // ---- ring loads (1 KB per wave each), issued by four waves: the compute waves themselves
    // (LW = 0), or four load waves beside them (LW = 4: waves 4-7 only issue loads, so a stage's
    // issue runs beside the multiplication instead of before it).  Issuing wave lw's weight load
    // q fills weight-slot rows (q*4 + lw) * (1024 / WRB) + lane / WLPR; the lane takes physical
    // chunk lane % WLPR of the row, which holds logical chunk (lane % WLPR) ^ (row & 15).
    // Activation load q fills slot rows (q*4 + lw)*8 + lane/8, physical chunk lane & 7 =
    // logical chunk (lane & 7) ^ (row & 7).
    static_assert(LW == 0 || LW == 4, "no load waves, or four");
    const bool issuer = LW == 0 || wave >= 4;      // wave-uniform
    const int lw = LW == 0 ? wave : wave - 4;
    constexpr int WLPR = T::WLPR, RPL = 1024 / T::WRB;     // weight rows per load
    const __amdgpu_buffer_rsrc_t rW = make_rsrc(p.W, static_cast<uint32_t>(static_cast<size_t>(p.Nout) * p.K * 2));
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A, static_cast<uint32_t>(static_cast<size_t>(p.a_row_limit) * p.lda * 2));
    uint32_t woff[QW], aoff[QA];
    int wlk[QW];                                   // logical K offset of the lane's weight chunk
    const int alk = ((lane & 7) ^ ((lane >> 3) & 7)) * 8;
    if (issuer) {
#pragma unroll
        for (int q = 0; q < QW; ++q) {
            const int r = (q * 4 + lw) * RPL + lane / WLPR;
            wlk[q] = ((lane % WLPR) ^ (r & (WLPR - 1) & 15)) * 8;
            const int gr = w_row(r);
            woff[q] = (gr >= 0 ? static_cast<uint32_t>(static_cast<size_t>(gr) * p.K * 2) : kOobRow) +
                      static_cast<uint32_t>(wlk[q] * 2);
        }
        // the rows' sources first, every lookup of the wave issued before any is used (a
        // clamped index keeps them unconditional), then the offsets: one round trip for a row
        // list in memory instead of one per load
        int src[QA];
#pragma unroll
        for (int q = 0; q < QA; ++q) {
            const int m = (q * 4 + lw) * 8 + (lane >> 3);
            const int mc = m0 + (m < mrows ? m : 0);
            src[q] = fused ? s_rows[mc] : (p.a_rows ? p.a_rows[mc] : mc);
        }
#pragma unroll
        for (int q = 0; q < QA; ++q) {
            const int m = (q * 4 + lw) * 8 + (lane >> 3);
            const bool ok = m < mrows && src[q] >= 0 && src[q] < p.a_row_limit;
            aoff[q] = (ok ? static_cast<uint32_t>(static_cast<size_t>(src[q]) * p.lda * 2) : kOobRow) +
                      static_cast<uint32_t>(alk * 2);
        }
    }
    uint8_t* const wring = smem;
    uint8_t* const aring = smem + NBW * T::WSLOT;
    auto issue_w = [&](int u) {                    // weight stage u -> slot u % NBW
        uint8_t* slot = wring + (u % NBW) * T::WSLOT;
        const int k0 = k_begin + u * KSUB * kStageK;
#pragma unroll
        for (int q = 0; q < QW; ++q) {
            const uint32_t kb = k0 + wlk[q] < k_stop ? static_cast<uint32_t>(k0 * 2) : kOobK;
            dma16(rW, slot + (q * 4 + lw) * 1024, woff[q] + kb);
        }
    };
    auto issue_a = [&](int t) {                    // activation stage t -> slot t % NBA
        uint8_t* slot = aring + (t % NBA) * T::ASLOT;
        const int k0 = k_begin + t * kStageK;
        const uint32_t kb = k0 + alk < k_stop ? static_cast<uint32_t>(k0 * 2) : kOobK;
#pragma unroll
        for (int q = 0; q < QA; ++q) dma16(rA, slot + (q * 4 + lw) * 1024, aoff[q] + kb);
    };

    // ---- the rings.  Prologue: weight stages 0 .. LWU-1, then activation stages 0 .. LA-1.
    // Iteration t waits for activation stage t (and with it everything requested earlier),
    // then requests activation stage t + LA and, when t starts weight stage u, weight stage
    // u + LWU.  Weight stage t / KSUB is always requested before activation stage t
    // (KSUB * LWU > LA), so one wait covers both; it leaves out exactly the loads this wave
    // issued after activation stage t: activation stages t+1 .. t+LA-1 and the weight stages
    // requested in iterations max(0, t-LA) .. t-1.  With load waves, they wait and issue and
    // the compute waves pass the same nst barriers (and no other in gemm_tile) and multiply.
    constexpr int LWU = T::LWU, LA = T::LA;
    auto issue_prologue = [&]() {
#pragma unroll
        for (int u = 0; u < LWU; ++u)
            if (u < nws) issue_w(u);
#pragma unroll
        for (int t = 0; t < LA; ++t)
            if (t < nst) issue_a(t);
    };
    auto wait_stage = [&](int t) {
        int n_w = 0;
        for (int i = max(0, t - LA); i < t; ++i)
            if (i % KSUB == 0 && i / KSUB + LWU < nws) ++n_w;
        const int n_a = max(0, min(LA - 1, nst - 1 - t));
        vm_wait_le<(QA < QW ? QA : QW), T::MAXN>(n_a * QA + n_w * QW);
    };
    auto issue_next = [&](int t) {
        if (t + LA < nst) issue_a(t + LA);
        if (t % KSUB == 0 && t / KSUB + LWU < nws) issue_w(t / KSUB + LWU);
    };
    if constexpr (LW > 0) {
        if (issuer) {
            issue_prologue();
            for (int t = 0; t < nst; ++t) {
                wait_stage(t);
                block_barrier();                   // stage t landed; the slots of t-1 are free
                issue_next(t);
            }
            return;
        }
    }

    // ---- fragment reads: lane reads row fr = lane & 15 of a 16-row tile at logical chunk
    // 8j + 4kk + (lane >> 4) of compute stage j of the weight stage, k-step kk (weights: XOR row
    // & 15 over the stage's WLPR chunks; XOR with j << 7 moves to compute stage j), or 4kk +
    // (lane >> 4) (activations: XOR row & 7)
    const int wn = wave % WN, wm = wave / WN;
    const int fr = lane & 15, fc = lane >> 4;
    const uint32_t wl0 = fr * T::WRB + ((fc ^ (fr & (WLPR - 1))) << 4);
    const uint32_t wl1 = fr * T::WRB + (((4 + fc) ^ (fr & (WLPR - 1))) << 4);
    const uint32_t al0 = fr * kRowB + ((fc ^ (fr & 7)) << 4);
    const uint32_t al1 = fr * kRowB + (((4 + fc) ^ (fr & 7)) << 4);
    const uint32_t wbase = lds_addr(wring) + wn * NTW * 16 * T::WRB;
    const uint32_t abase = lds_addr(aring) + wm * TM * 16 * kRowB;
    f32x4 acc[TM][NTW];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int t) {
        const uint32_t j7 = static_cast<uint32_t>((t % KSUB) << 7);
        const uint32_t sw = wbase + static_cast<uint32_t>(((t / KSUB) % NBW) * T::WSLOT);
        const uint32_t sa = abase + static_cast<uint32_t>((t % NBA) * T::ASLOT);
        u32x4 f0[NTW + TM], f1[NTW + TM];
        // k-step 0 fragments, then k-step 1: lgkmcnt(NTW + TM) leaves only the second group pending
        read_tiles<NTW, T::WRB>(f0, (wl0 ^ j7) + sw);
        read_tiles<TM, kRowB>(f0 + NTW, al0 + sa);
        read_tiles<NTW, T::WRB>(f1, (wl1 ^ j7) + sw);
        read_tiles<TM, kRowB>(f1 + NTW, al1 + sa);
        lds_wait<NTW + TM>(f0);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < NTW; ++j) acc[i][j] = mma(f0[j], f0[NTW + i], acc[i][j]);
        __builtin_amdgcn_sched_barrier(0);        // keep k-step 0's MFMAs ahead of the next wait
        lds_wait<0>(f1);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < NTW; ++j) acc[i][j] = mma(f1[j], f1[NTW + i], acc[i][j]);
    };
    if constexpr (LW > 0) {
        for (int t = 0; t < nst; ++t) {
            block_barrier();                       // stage t landed; the slots of t-1 are free
            compute(t);
        }
    } else {
        issue_prologue();
        for (int t = 0; t < nst; ++t) {
            wait_stage(t);
            block_barrier();                       // stage t landed for every wave; slots of t-1 free
            issue_next(t);
            compute(t);
        }
    }

    // ---- epilogue: lane holds C[row m][cols n0 + 4*(lane>>4) + q] of tile (i, j)
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int m = (wm * TM + i) * 16 + (lane & 15);
        if (m >= mrows) continue;
        if (EPI == EPI_SWIGLU) {
#pragma unroll
            for (int j = 0; j < NTW; j += 2) {
                const int col = c0 + (wn * (NTW / 2) + j / 2) * 16 + 4 * (lane >> 4);
                if (col >= c1) continue;
                // silu(g) * up = g * up / (1 + e^-g), with the hardware exp2 and reciprocal
                // (about 1 ulp each in fp32, far below the bf16 rounding of the result)
                float o[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float gt = acc[i][j][q], up = acc[i][j + 1][q];
                    const float e = __builtin_amdgcn_exp2f(gt * -1.4426950408889634f);
                    o[q] = gt * __builtin_amdgcn_rcpf(1.0f + e) * up;
                }
                *reinterpret_cast<uint2*>(p.act + static_cast<size_t>(m0 + m) * p.F + col) =
                    make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
            }
        } else if constexpr (EPI == EPI_ARGMAX && WN == 1) {
            // the wave holds every column of the group for its rows: the lane's best over its
            // columns in ascending order (first maximum kept; NaN never taken), then the best of
            // the 4 lanes sharing the row (ties to the lower column)
            float best = 0.f;
            int bi = -1;
#pragma unroll
            for (int j = 0; j < NTW; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int col = c0 + j * 16 + 4 * (lane >> 4) + q;
                    const float v = acc[i][j][q];
                    if (col < c1 && v == v && (bi < 0 || v > best)) { best = v; bi = col; }
                }
#pragma unroll
            for (int off = 16; off <= 32; off <<= 1) {
                const float ob = __shfl_xor(best, off, kWave);
                const int oi = __shfl_xor(bi, off, kWave);
                if (oi >= 0 && (bi < 0 || ob > best || (ob == best && oi < bi))) { best = ob; bi = oi; }
            }
            if ((lane >> 4) == 0) {
                const size_t o = static_cast<size_t>(p.group_base + g) * p.m_cap + m0 + m;
                p.arg_val[o] = bi < 0 ? __builtin_nanf("") : best;
                p.arg_idx[o] = bi < 0 ? -1 : p.col_base + bi;
            }
        } else {
            float* dst = p.partial + (static_cast<size_t>(y) * p.m_cap + m0 + m) * p.Nout + 4 * (lane >> 4);
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                const int col = c0 + (wn * NTW + j) * 16;
                if (col + 4 * (lane >> 4) < c1) *reinterpret_cast<f32x4*>(dst + col) = acc[i][j];
            }
        }
    }
}

template <int NTW, int WN, int TM, int KSUB, int NBW, int NBA, int EPI, int LW>
__global__ __launch_bounds__(256 + 64 * LW) void gemm_kernel(const GemmArgs p) {
    using T = Tile<NTW, WN, TM, KSUB, NBW, NBA>;
    extern __shared__ __align__(16) uint8_t smem[];
    // the fused compaction's LDS sits behind the rings in the dynamic allocation (fc_lds_bytes),
    // so a launch without it takes the rings' bytes only: static LDS here would push an 80 KB
    // tile just past half of a CU's 160 KB and halve the workgroups a CU holds
    int32_t* s_rows = reinterpret_cast<int32_t*>(smem + T::LDS);
    int M;
    if (p.fc_fold != nullptr) {
        uint8_t* s_fold = reinterpret_cast<uint8_t*>(s_rows + p.fc_R);
        int* s_tot = reinterpret_cast<int*>(smem + T::LDS + ((static_cast<size_t>(p.fc_R) * 5 + 15) & ~size_t(15)));
        int* s_par = s_tot + 4;
        // the grid's last workgroup publishes: busy workgroups take the lowest ids and the launcher
        // adds a row of idle ones, so the publishing work (the list, the row map and every row's
        // fold source) runs beside the projection instead of delaying one of its tiles
        M = compact_in_lds(p, s_rows, s_fold, s_tot, s_par,
                           blockIdx.x == gridDim.x - 1 && blockIdx.y == gridDim.y - 1);
    } else {
        M = p.m_count ? p.m_count[0] : p.m_fixed;
    }
    M = M < 0 ? 0 : (M > p.m_cap ? p.m_cap : M);
    M = __builtin_amdgcn_readfirstlane(M);
    gemm_tile<NTW, WN, TM, KSUB, NBW, NBA, EPI, LW>(p, M, blockIdx.x + gridDim.x * blockIdx.y, gridDim.y, smem, s_rows);
}

// Raise a kernel's dynamic-LDS cap to at least `lds` bytes.  `cap` holds the cap raised so far
// for that kernel (one atomic per launcher instance), so concurrent host threads at worst both
// set the same attribute.
inline hipError_t raise_lds_cap(const void* kern, size_t lds, std::atomic<size_t>& cap) {
    if (lds <= cap.load(std::memory_order_relaxed)) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e == hipSuccess) {
        size_t cur = cap.load(std::memory_order_relaxed);
        while (cur < lds && !cap.compare_exchange_weak(cur, lds, std::memory_order_relaxed)) {
        }
    }
    return e;
}

// A tile shape as a type, for the launch that holds several
template <int NTW, int WN, int TM, int KSUB, int NBW, int NBA, int LW_>
struct Shape {
    using T = Tile<NTW, WN, TM, KSUB, NBW, NBA>;
    static constexpr int LW = LW_;
    static bool is(const GemmCfg& c) {
        return c.ntw == NTW && c.wn == WN && c.tm == TM && c.ksub == KSUB && c.nbw == NBW && c.nba == NBA &&
               c.lw == LW;
    }
    static __device__ __forceinline__ void run(const GemmArgs& p, int M, uint8_t* smem) {
        gemm_tile<NTW, WN, TM, KSUB, NBW, NBA, EPI_SWIGLU, LW>(p, M, blockIdx.x, 1, smem, nullptr);
    }
};

// Three tile shapes of one SwiGLU projection in one launch: shape A for M <= upto_a rows, B for
// M <= upto_b, C above.  M is only known on the device; launches gated by row-count windows
// would cost every idle launch's workgroups a dispatch, a single launch costs only the idle ids
// of its grid (the largest shape's).  The LDS is the largest shape's; p[i] carries shape i's
// groups and chunks.
template <class SA, class SB, class SC>
__global__ __launch_bounds__(256 + 64 * SA::LW) void gemm_shapes_kernel(const GemmArgs pa, const GemmArgs pb, const GemmArgs pc,
                                                          const int upto_a, const int upto_b) {
    extern __shared__ __align__(16) uint8_t smem[];
    int M = pa.m_count ? pa.m_count[0] : pa.m_fixed;
    M = M < 0 ? 0 : (M > pa.m_cap ? pa.m_cap : M);
    M = __builtin_amdgcn_readfirstlane(M);
    if (M <= upto_a) SA::run(pa, M, smem);
    else if (M <= upto_b) SB::run(pb, M, smem);
    else SC::run(pc, M, smem);
}

// the kernels split the 4-column units over the groups with 32-bit products
bool groups_fit(int groups, int ncols) {
    return static_cast<uint64_t>(groups) * static_cast<uint64_t>((ncols + 3) / 4) < (uint64_t(1) << 32);
}

template <int NTW, int WN, int TM, int KSUB, int NBW, int NBA, int EPI, int LW>
hipError_t launch_shape(GemmArgs a, const GemmCfg& c, int splits, hipStream_t st) {
    using T = Tile<NTW, WN, TM, KSUB, NBW, NBA>;
    // the partial-sum and SwiGLU epilogues store whole 4-column units; only the greedy-token
    // epilogue takes a column count that is not a multiple of 4
    if (EPI != EPI_ARGMAX && ((EPI == EPI_SWIGLU ? a.F : a.Nout) % 4) != 0) return hipErrorInvalidValue;
    const int groups = c.groups;
    if (groups < 1 || !groups_fit(groups, EPI == EPI_SWIGLU ? a.F : a.Nout)) return hipErrorInvalidValue;
    a.n_groups = groups;
    a.min_chunks = c.min_chunks;
    a.xcd_split = EPI == EPI_PARTIAL && c.xcd_split ? 1 : 0;
    a.m_chunks = (a.m_cap + T::MP - 1) / T::MP;
    if (a.m_chunks < 1) a.m_chunks = 1;
    // the fused compaction's row list (4 bytes per row), flags (1 byte per row), four wave totals
    // and the parent map
    const size_t fc_lds = a.fc_fold ? ((static_cast<size_t>(a.fc_R) * 5 + 15) & ~size_t(15)) + 4 * (4 + kMaxBranches) : 0;
    const size_t lds = static_cast<size_t>(T::LDS) + fc_lds;
    auto kern = gemm_kernel<NTW, WN, TM, KSUB, NBW, NBA, EPI, LW>;
    static std::atomic<size_t> cap{0};
    hipError_t e = raise_lds_cap(reinterpret_cast<const void*>(kern), lds, cap);
    if (e != hipSuccess) return e;
    // a fused compaction gets eight more (idle) workgroups, the last of which publishes
    const dim3 grid(((groups + 7) / 8) * 8 * a.m_chunks + (a.fc_fold ? 8 : 0), splits);
    hipLaunchKernelGGL(kern, grid, dim3(256 + 64 * LW), lds, st, a);
    return hipGetLastError();
}

template <class SA, class SB, class SC>
hipError_t launch_shapes(GemmArgs a, const GemmCfg* c, const int* upto, hipStream_t st) {
    static_assert(SA::LW == SB::LW && SB::LW == SC::LW, "one launch, one workgroup size");
    a.fc_fold = nullptr;
    GemmArgs p[3] = {a, a, a};
    const int mp[3] = {SA::T::MP, SB::T::MP, SC::T::MP};
    const int rows[3] = {upto[0], upto[1], a.m_cap};   // the most rows each shape ever sees
    int grid = 1;
    for (int i = 0; i < 3; ++i) {
        if (c[i].groups < 1 || !groups_fit(c[i].groups, a.F)) return hipErrorInvalidValue;
        p[i].n_groups = c[i].groups;
        p[i].min_chunks = c[i].min_chunks;
        const int r = rows[i] < a.m_cap ? rows[i] : a.m_cap;
        p[i].m_chunks = (r + mp[i] - 1) / mp[i];
        if (p[i].m_chunks < 1) p[i].m_chunks = 1;
        const int g = ((c[i].groups + 7) / 8) * 8 * p[i].m_chunks;
        if (g > grid) grid = g;
    }
    size_t lds = static_cast<size_t>(SA::T::LDS);
    if (static_cast<size_t>(SB::T::LDS) > lds) lds = SB::T::LDS;
    if (static_cast<size_t>(SC::T::LDS) > lds) lds = SC::T::LDS;
    auto kern = gemm_shapes_kernel<SA, SB, SC>;
    static std::atomic<size_t> cap{0};
    hipError_t e = raise_lds_cap(reinterpret_cast<const void*>(kern), lds, cap);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256 + 64 * SA::LW), lds, st, p[0], p[1], p[2], upto[0], upto[1]);
    return hipGetLastError();
}

}  // namespace

int gemm_chunk_rows(const GemmCfg& c) {
    return 16 * c.tm * (4 / c.wn);
}

int gemm_group_cols(const GemmCfg& c) {
    return (c.swiglu ? 8 : 16) * c.ntw * c.wn;
}

size_t gemm_lds_bytes(const GemmCfg& c) {
    return (static_cast<size_t>(c.nbw) * 16 * c.ntw * c.wn * c.ksub + static_cast<size_t>(c.nba) * gemm_chunk_rows(c)) *
           kRowB;
}

hipError_t launch_gemm(const GemmArgs& a, const GemmCfg& c, hipStream_t st) {
#define SPECFOLD_GEMM_CASE(NTW_, WN_, TM_, KS_, NBW_, NBA_, LW_)                                    \
    if (c.ntw == NTW_ && c.wn == WN_ && c.tm == TM_ && c.ksub == KS_ && c.nbw == NBW_ && c.nba == NBA_ &&  \
        c.lw == LW_)                                                                               \
        return c.argmax ? (WN_ == 1 ? launch_shape<NTW_, WN_, TM_, KS_, NBW_, NBA_, EPI_ARGMAX, LW_>(a, c, 1, st) \
                                    : hipErrorInvalidValue)                                            \
             : c.swiglu ? launch_shape<NTW_, WN_, TM_, KS_, NBW_, NBA_, EPI_SWIGLU, LW_>(a, c, 1, st)     \
                        : launch_shape<NTW_, WN_, TM_, KS_, NBW_, NBA_, EPI_PARTIAL, LW_>(a, c, c.splits, st);
    SPECFOLD_GEMM_CASES(SPECFOLD_GEMM_CASE)
#undef SPECFOLD_GEMM_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_shapes(const GemmArgs& a, const GemmCfg* c, const int* upto, hipStream_t st) {
    if (a.fc_fold != nullptr || upto[0] < 0 || upto[1] < upto[0]) return hipErrorInvalidValue;
    for (int i = 0; i < 3; ++i)
        if (!c[i].swiglu || c[i].argmax) return hipErrorInvalidValue;
#define SPECFOLD_GEMM_TRIPLE(A0, A1, A2, A3, A4, A5, B0, B1, B2, B3, B4, B5, C0, C1, C2, C3, C4, C5, LW_) \
    {                                                                                              \
        using SA = Shape<A0, A1, A2, A3, A4, A5, LW_>;                                             \
        using SB = Shape<B0, B1, B2, B3, B4, B5, LW_>;                                             \
        using SC = Shape<C0, C1, C2, C3, C4, C5, LW_>;                                             \
        if (SA::is(c[0]) && SB::is(c[1]) && SC::is(c[2])) return launch_shapes<SA, SB, SC>(a, c, upto, st); \
    }
    SPECFOLD_GEMM_TRIPLES(SPECFOLD_GEMM_TRIPLE)
#undef SPECFOLD_GEMM_TRIPLE
    return hipErrorInvalidValue;
}

}  // namespace specfold
