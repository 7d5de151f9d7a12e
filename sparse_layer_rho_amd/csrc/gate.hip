// Gate, compaction, fold-source resolution and row RMSNorm.
//
// Gate [SpecFold review, "무엇과 다른가"]: per draft row (i, n) with parent p = par(i),
// rho = |H_i[n] - H_p[n]| / |H_p[n]| and the row folds when rho <= delta; main rows bypass
// the gate [SpecFold summary, App. B].  One 64-lane wave owns one row: the lanes stream the
// child and parent rows in 16-byte chunks (coalesced), accumulate in fp32 and reduce with
// DPP lane moves.  The same loads give the row's sum of squares, i.e. its RMSNorm scale,
// and -- when asked -- the normalised row the QKV projection consumes (RMSNorm weight applied,
// rounded to bf16), so the layer input is read from HBM once.
//
// Compaction [SpecFold summary, App. B]: an exclusive scan of the recompute flags in row order
// (wave ballots + a cross-wave scan in LDS) writes the global list, the per-branch offsets and
// the inverse map row -> slot.  Past 8192 rows one pass over 32768-row tiles with a decoupled
// look-back between them, so large inputs use the whole GPU and read the flags once.
//
// Sources [SpecFold summary, App. B and §A.3]: every row walks its fold chain up the parent map
// (at most n_branch steps; branch 0 always terminates) -- rows are independent, so one
// order-free launch covers all branches.
#include "kernels.h"
#include "lanes.h"

namespace specfold {

namespace {

constexpr int kMaxChunksPerLane = 10;   // 16-byte chunks per lane of one row: D <= 5120

__device__ __forceinline__ float rho_of(float a, float b) {
    if (b > 0.f) return sqrtf(a) / sqrtf(b);
    if (a > 0.f) return __builtin_inff();
    if (a == 0.f) return 0.f;
    return __builtin_nanf("");
}

// xn chunk = bf16(x * s * w) for the 8 elements of a chunk, wv its 8 norm weights
__device__ __forceinline__ uint4 norm_chunk_w(const float* x, float s, const uint4& wv) {
    float w[8], y[8];
    unpack8(wv, w);
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = x[e] * s * w[e];
    return pack8(y);
}

// xn chunk = bf16(x * s * ln) for the 8 elements of chunk k of a row (no ln: bf16(x * s))
__device__ __forceinline__ uint4 norm_chunk(const float* x, float s, const uint16_t* ln, int k) {
    if (ln) return norm_chunk_w(x, s, *reinterpret_cast<const uint4*>(ln + 8 * k));
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = x[e] * s;
    return pack8(y);
}

// the norm weights of the CPL chunks a lane normalises, requested with the row (chunks past the
// row read zeros) so the norm does not wait for a second round trip after the reductions
template <int CPL>
__device__ __forceinline__ void load_norm_weights(const uint16_t* ln, int D, int lane, uint4 (&wv)[CPL]) {
    const __amdgpu_buffer_rsrc_t rL = make_rsrc(ln, static_cast<uint32_t>(D) * 2);
    const int nch = D >> 3;
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
        const int k = lane + t * kWave;
        wv[t] = buf_load16(rL, k < nch ? 16 * k : kOob);
    }
}

// One wave computes rho, fold, inv_rms (and optionally the normalised row) of one row.  Lane l
// holds chunks l, l + 64, ... (CPL of them) of the child and the parent row; all of them are
// requested before any is used (chunks past the row, and the parent of a main row, read zeros
// from an out-of-range offset), so a row costs one memory round trip.  The loads of a row are
// issued by gate_issue and consumed by gate_finish, so a wave can request its next row before it
// reduces the current one.
template <int CPL>
struct GateRow {
    uint4 cv[CPL], pv[CPL];
};

template <int CPL>
__device__ __forceinline__ void gate_issue(const GateParams& p, __amdgpu_buffer_rsrc_t rH, int row, int lane,
                                           GateRow<CPL>& g) {
    const int i = row / p.N, n = row - i * p.N;
    const bool need_pair = (i > 0) && (p.rho_in == nullptr);
    const bool need_rows = need_pair || (p.inv_rms != nullptr) || (p.xn != nullptr);
    const int nch = p.D >> 3;
    const uint32_t cb = need_rows ? static_cast<uint32_t>(row) * p.D * 2 : kOob;
    const uint32_t pb = need_pair ? static_cast<uint32_t>(p.par.p[i] * p.N + n) * p.D * 2 : kOob;
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
        const int k = lane + t * kWave;
        g.cv[t] = buf_load16(rH, k < nch ? cb + 16 * k : kOob);
        g.pv[t] = buf_load16(rH, k < nch ? pb + 16 * k : kOob);
    }
}

template <int CPL>
__device__ __forceinline__ void gate_finish(const GateParams& p, int row, int lane, const GateRow<CPL>& g,
                                            const uint4 (&wv)[CPL]) {
    const int i = row / p.N;
    const int nch = p.D >> 3;
    float a = 0.f, b = 0.f, ss = 0.f;
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
        float x[8], yv[8];
        unpack8(g.cv[t], x);
        unpack8(g.pv[t], yv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float d = x[e] - yv[e];
            ss += x[e] * x[e];
            a += d * d;
            b += yv[e] * yv[e];
        }
    }
    a = wave_sum_dpp(a);
    b = wave_sum_dpp(b);
    ss = wave_sum_dpp(ss);
    const float inv = 1.0f / sqrtf(ss / static_cast<float>(p.D) + p.eps);
    if (lane == 0) {
        float r = 0.f;
        bool f = false;
        if (i > 0) {
            r = p.rho_in ? p.rho_in[row] : rho_of(a, b);
            f = r <= p.delta;                      // NaN compares false: recompute
        }
        p.rho[row] = r;
        p.fold[row] = f ? 1 : 0;
        if (p.fold_copy) p.fold_copy[row] = f ? 1 : 0;
        if (p.inv_rms) p.inv_rms[row] = inv;
    }
    if (p.xn) {
        uint4* o = reinterpret_cast<uint4*>(p.xn + static_cast<size_t>(row) * p.D);
#pragma unroll
        for (int t = 0; t < CPL; ++t) {
            const int k = lane + t * kWave;
            if (k < nch) {
                float x[8];
                unpack8(g.cv[t], x);
                o[k] = p.ln ? norm_chunk_w(x, inv, wv[t]) : norm_chunk(x, inv, nullptr, k);
            }
        }
    }
}

// Grid of one wave per row, 4 waves per workgroup.  Rows are visited in windows of `win`
// positions, branch-major inside a window: consecutive waves read consecutive (contiguous) rows
// of one branch, and a child's parent row -- same positions, an earlier branch -- is read by the
// same window's waves shortly before or after, so the second read is an L2 hit.  With at least 8
// windows, window w's workgroups all sit on XCD w % 8 (the dispatcher deals workgroup ids
// round-robin to the 8 XCDs), so the hit is in that XCD's own L2.  Measured on 9 x 16384 rows of
// 1536 (453 MB): 82 us with 128-position windows on one XCD each, 86-90 us in plain window order,
// 98 us position-major (one workgroup per position), 123 us branch-major over whole branches,
// where every parent row is read again far from its first read.
constexpr int kGateWin = 128;

template <int CPL>
__global__ __launch_bounds__(256) void gate_kernel(const GateParams p, int win, int n_win, int xcd_map) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: scalar index math
    const int wg_per_win = p.nb * win / 4;              // the host keeps win a multiple of 4
    int g = static_cast<int>(blockIdx.x);
    if (xcd_map) {
        const int x = g & 7, k = g >> 3;
        g = ((k / wg_per_win) * 8 + x) * wg_per_win + k % wg_per_win;
    }
    const int w = g * 4 + wave;                         // wave index in (window, branch, position) order
    const int per_win = p.nb * win;                     // (fewer than 2^31 waves: R <= 2^24, win <= 128)
    const int wi = w / per_win, rem = w - wi * per_win;
    const int i = rem / win, n = wi * win + (rem - i * win);
    if (wi >= n_win || n >= p.N) return;
    uint4 wv[CPL];
    if (p.xn && p.ln) load_norm_weights<CPL>(p.ln, p.D, lane, wv);
    const __amdgpu_buffer_rsrc_t rH =
        make_rsrc(p.H, static_cast<uint32_t>(static_cast<size_t>(p.nb) * p.N * p.D * 2));
    GateRow<CPL> r;
    const int row = __builtin_amdgcn_readfirstlane(i * p.N + n);
    gate_issue<CPL>(p, rH, row, lane, r);
    gate_finish<CPL>(p, row, lane, r, wv);
}

// Exclusive scan of the recompute flags of rows [r_begin, r_end) in ascending order, starting
// at slot `base`, by one workgroup (ballots per wave, a cross-wave scan in LDS).  Writes the
// list, row -> slot and the per-branch offsets of the rows it covers; returns the count.
__device__ int scan_rows(const CompactParams& p, int r_begin, int r_end, int base) {
    __shared__ int s_wave_tot[16];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int nw = blockDim.x >> 6;
    const int start = base;
    for (int r0 = r_begin; r0 < r_end; r0 += blockDim.x) {
        const int r = r0 + tid;
        const bool rec = (r < r_end) && (p.fold[r] == 0);
        const uint64_t m = __ballot(rec);
        const int excl = __popcll(m & ((1ull << lane) - 1ull));
        if (lane == 0) s_wave_tot[wave] = __popcll(m);
        __syncthreads();
        int woff = 0, tot = 0;
        for (int w = 0; w < nw; ++w) {
            const int t = s_wave_tot[w];
            woff += (w < wave) ? t : 0;
            tot += t;
        }
        const int slot = base + woff + excl;
        if (r < r_end) {
            p.row_slot[r] = rec ? slot : -1;
            if (rec) p.rec_rows[slot] = r;
            if (r % p.N == 0) p.branch_off[r / p.N] = slot;
        }
        base += tot;
        __syncthreads();
    }
    return base - start;
}

// all rows in one workgroup (R up to a few tiles: the layer's own sizes)
__global__ __launch_bounds__(1024) void compact_kernel(const CompactParams p) {
    const int total = scan_rows(p, 0, p.R, 0);
    if (threadIdx.x == 0) {
        p.rec_count[0] = total;
        p.branch_off[p.nb] = total;
    }
}

// Large inputs: one pass over the flags with a look-back in the manner of Merrill and Garland's
// single-pass scan ("Single-pass Parallel Prefix Scan with Decoupled Look-back", 2016).  Each
// workgroup takes a ticket -- tiles are numbered in the order workgroups start, so a tile only ever
// waits for tiles that are already running -- loads its tile's flags, counts them and publishes the
// count; it then reads every predecessor's published count (at most 512 tiles at 2^24 rows, one
// batch of independent loads rather than a walk that waits for inclusive prefixes to ripple
// down) and scatters its rows from their sum.  The status words and the ticket counter live in
// the caller's workspace and are cleared by a fill kernel just before (a fill kernel, not a memset
// node, so the sequence can be captured in a graph).  Status word: 2 flag bits (0 empty, 1 count
// published) above a 30-bit count (R <= 2^24).
// Measured on 2^24 rows (30 % recomputed): 31.6 us for the clear and scan kernels, against 15.7 us
// for the bare traffic (flags read, row map written, no scan) and 21.7 us for the kernel with
// every store removed: the ticket (3.8 us), the look-back (3.5 us) and the loads run before any
// store can start, and with every tile resident at once nothing overlaps them.  Tiles of 8192 or
// 16384 rows (more rounds) took 82 and 41 us (the ticket and look-back grow with the tile count);
// 65536 rows 31.9 us.
constexpr int kLookbackThreads = 1024;          // threads per workgroup of the look-back scan
constexpr int kLookbackSteps = 4;               // steps of 8 rows per thread in one tile
constexpr int kCompactTile = 8 * kLookbackThreads * kLookbackSteps;   // rows per tile
constexpr int kSmallCompact = 8192;             // up to this many rows one workgroup scans them all
constexpr uint32_t kStAgg = 1u << 30, kStFlags = 3u << 30;
// A predecessor always publishes, so the wait below ends; the bound only guarantees that no
// wave can spin forever whatever happens (about a second of polling); a tile that gives up marks
// the run in its status area (word 1) and takes offset 0.
constexpr int kSpinLimit = 1 << 22;

// Workgroup barrier that orders LDS only: waits for this wave's LDS operations, not for its
// global stores (__syncthreads also drains every outstanding store, so a loop that stores and
// then synchronizes on LDS would wait for its stores' write acknowledgements at every step).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint32_t ld_status(const uint32_t* a) {
    return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_status(uint32_t* a, uint32_t v) {
    __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(1024) void compact_clear_kernel(uint32_t* state, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) state[i] = 0;
}

// The tile is kSteps steps of 8192 rows; in each, thread t owns the 8 consecutive rows 8t .. 8t+7
// of the step.  Every step's flags (one 8-byte load per thread) are requested at once.  One
// workgroup-wide exclusive scan of the per-thread counts of all steps at once (wave scans, the
// wave totals of every step through LDS, one barrier) places every recompute row; the tile's
// count is published and the offset looked back; then every thread writes its 8 row -> slot
// entries of each step as two 16-byte stores, and each step's list is gathered in LDS (two
// buffers, so one barrier per step) and written out in consecutive stores.
template <int THREADS>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(8, 8))) void compact_lookback_kernel(const CompactParams p, uint32_t* state, int ntiles) {
    constexpr int kSub = 8 * THREADS;              // rows of one step
    constexpr int kSteps = kLookbackSteps;
    constexpr int kTile = kSub * kSteps;
    constexpr int kWaves = THREADS / kWave;
    __shared__ int s_wave[kSteps][kWaves];         // each step's per-wave totals
    __shared__ int s_tile, s_base;
    __shared__ int s_list[2][kSub];                // two steps' recompute rows, in slot order
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    if (tid == 0) s_tile = static_cast<int>(atomicAdd(state, 1u));
    __syncthreads();
    const int tile = s_tile;
    if (tile >= ntiles) return;                    // (never: the grid has one workgroup per tile)
    const int r0 = tile * kTile;
    uint32_t bits[kSteps];                         // bit b: row rt + b exists and is recomputed
#pragma unroll
    for (int q = 0; q < kSteps; ++q) {
        const int rt = r0 + q * kSub + 8 * tid;
        bits[q] = 0;
        if (rt + 8 <= p.R) {
            const uint2 v = *reinterpret_cast<const uint2*>(p.fold + rt);
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const uint32_t w = b < 4 ? v.x : v.y;
                bits[q] |= (((w >> (8 * (b & 3))) & 0xffu) == 0 ? 1u : 0u) << b;
            }
        } else {
            for (int b = 0; b < 8 && rt + b < p.R; ++b) bits[q] |= (p.fold[rt + b] == 0 ? 1u : 0u) << b;
        }
    }
    // inclusive scans over the wave, one per step
    int incl[kSteps];
#pragma unroll
    for (int q = 0; q < kSteps; ++q) incl[q] = __popc(bits[q]);
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
#pragma unroll
        for (int q = 0; q < kSteps; ++q) {
            const int t = __shfl_up(incl[q], d, kWave);
            if (lane >= d) incl[q] += t;
        }
    }
    if (lane == kWave - 1) {
#pragma unroll
        for (int q = 0; q < kSteps; ++q) s_wave[q][wave] = incl[q];
    }
    __syncthreads();
    // local[q]: tile-local slot of the thread's first recompute row of step q; step_off[q]: the
    // tile-local slot of step q's first recompute row
    // (each step's wave totals are scanned across the first kWaves lanes of every wave, so a
    // thread holds two values per step instead of all the totals)
    int local[kSteps], step_off[kSteps + 1];
    step_off[0] = 0;
#pragma unroll
    for (int q = 0; q < kSteps; ++q) {
        const int v = lane < kWaves ? s_wave[q][lane] : 0;
        int sc = v;
#pragma unroll
        for (int d = 1; d < kWaves; d <<= 1) {
            const int t = __shfl_up(sc, d, kWave);
            if (lane >= d) sc += t;
        }
        const int before = __shfl(sc - v, wave, kWave), tot = __shfl(sc, kWaves - 1, kWave);
        local[q] = step_off[q] + before + incl[q] - __popc(bits[q]);
        step_off[q + 1] = step_off[q] + tot;
    }
    const int cnt = step_off[kSteps];
    if (tid == 0) st_status(state + 4 + tile, kStAgg | static_cast<uint32_t>(cnt));
    // look-back by wave 0: every predecessor's count is read in one batch of independent loads
    // (lane l reads tiles l, l + 64, ...; at most 64 * kBatch tiles per batch) and summed; a
    // predecessor that has not published yet is read again
    if (wave == 0) {
        constexpr int kBatch = 8;
        const uint32_t* status = state + 4;
        int base = 0, spins = 0;
        for (int j0 = 0; j0 < tile; j0 += kBatch * kWave) {
            uint32_t sw[kBatch];
            while (true) {
                bool missing = false;
#pragma unroll
                for (int b = 0; b < kBatch; ++b) {
                    const int k = j0 + b * kWave + lane;
                    sw[b] = k < tile ? ld_status(status + k) : kStAgg;
                }
#pragma unroll
                for (int b = 0; b < kBatch; ++b) missing |= (sw[b] & kStFlags) == 0;
                if (!__ballot(missing)) break;
                if (++spins > kSpinLimit) {
                    if (lane == 0) st_status(state + 1, 1u);
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
            int v = 0;
#pragma unroll
            for (int b = 0; b < kBatch; ++b) v += static_cast<int>(sw[b] & ~kStFlags);
#pragma unroll
            for (int d = 32; d > 0; d >>= 1) v += __shfl_xor(v, d, kWave);
            base += v;
        }
        if (lane == 0) {
            s_base = base;
            if (tile == ntiles - 1) {
                p.rec_count[0] = base + cnt;
                p.branch_off[p.nb] = base + cnt;
            }
        }
    }
    __syncthreads();
    const int base = s_base;
#pragma unroll
    for (int q = 0; q < kSteps; ++q) {
        const int rt = r0 + q * kSub + 8 * tid;
        const uint32_t bq = bits[q];
        const int lq = local[q] - step_off[q];     // step-local index of the thread's first recompute row
        const int slot = base + local[q];          // slot of the thread's first recompute row
        // branch starts among the thread's rows: one division per step, not one per row
        if (rt < p.R) {
            int br = (rt + p.N - 1) / p.N;
            for (int m = br * p.N; m < rt + 8 && m < p.R; m += p.N, ++br)
                p.branch_off[br] = slot + __popc(bq & ((1u << (m - rt)) - 1u));
        }
        int rs[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const int k = __popc(bq & ((1u << b) - 1u));
            const bool rec = (bq >> b) & 1u;
            rs[b] = rec ? slot + k : -1;
            if (rec) s_list[q & 1][lq + k] = rt + b;
        }
        if (rt + 8 <= p.R) {
            int4* dst = reinterpret_cast<int4*>(p.row_slot + rt);
            dst[0] = make_int4(rs[0], rs[1], rs[2], rs[3]);
            dst[1] = make_int4(rs[4], rs[5], rs[6], rs[7]);
        } else {
            for (int b = 0; b < 8 && rt + b < p.R; ++b) p.row_slot[rt + b] = rs[b];
        }
        // the step's list leaves LDS in consecutive 4-byte stores (coalesced over each wave); the
        // other buffer takes the next step, and this one is refilled only two steps on, after the
        // next step's barrier
        lds_barrier();
        const int tot = step_off[q + 1] - step_off[q];
        for (int e = tid; e < tot; e += THREADS) p.rec_rows[base + step_off[q] + e] = s_list[q & 1][e];
    }
}

__global__ __launch_bounds__(256) void resolve_kernel(const ResolveParams p) {
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= p.R) return;
    const int i = r / p.N, n = r - i * p.N;
    int j = i;
    for (int s = 0; s < p.nb && j > 0 && p.fold[j * p.N + n] != 0; ++s) j = p.par.p[j];
    p.src_branch[r] = j;
    p.src_slot[r] = p.row_slot[j * p.N + n];
}

// one wave per row: xn = bf16(X * s * ln)
__global__ __launch_bounds__(256) void row_norm_kernel(const uint16_t* __restrict__ X, int R, int D,
                                                       const float* inv_rms, float eps,
                                                       const uint16_t* ln, uint16_t* __restrict__ xn) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (row >= R) return;
    const int nch = D >> 3;
    const uint4* c = reinterpret_cast<const uint4*>(X + static_cast<size_t>(row) * D);
    float s;
    if (inv_rms) {
        s = inv_rms[row];
    } else {
        float ss = 0.f;
        for (int k = lane; k < nch; k += kWave) {
            float x[8];
            unpack8(c[k], x);
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
        }
        ss = wave_sum(ss);
        s = 1.0f / sqrtf(ss / static_cast<float>(D) + eps);
    }
    uint4* o = reinterpret_cast<uint4*>(xn + static_cast<size_t>(row) * D);
    for (int k = lane; k < nch; k += kWave) {
        float x[8];
        unpack8(c[k], x);
        o[k] = norm_chunk(x, s, ln, k);
    }
}

}  // namespace

namespace {

// RMSNorm of whole rows (the final norm before the LM head): one wave per row, every chunk of
// the row requested before any is used, as in the gate.
template <int CPL>
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const uint16_t* H, int R, int D, const uint16_t* ln,
                                                           float eps, uint16_t* xn) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & (kWave - 1);
    if (row >= R) return;
    const int nch = D >> 3;
    const __amdgpu_buffer_rsrc_t rH = make_rsrc(H, static_cast<uint32_t>(static_cast<size_t>(R) * D * 2));
    const uint32_t base = static_cast<uint32_t>(row) * D * 2;
    uint4 cv[CPL], wv[CPL];
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
        const int k = lane + t * kWave;
        cv[t] = buf_load16(rH, k < nch ? base + 16 * k : kOob);
    }
    if (ln) load_norm_weights<CPL>(ln, D, lane, wv);
    float ss = 0.f;
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
        float x[8];
        unpack8(cv[t], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
    }
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / static_cast<float>(D) + eps);
    uint4* o = reinterpret_cast<uint4*>(xn + static_cast<size_t>(row) * D);
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
        const int k = lane + t * kWave;
        if (k < nch) {
            float x[8];
            unpack8(cv[t], x);
            o[k] = ln ? norm_chunk_w(x, inv, wv[t]) : norm_chunk(x, inv, nullptr, k);
        }
    }
}

}  // namespace

hipError_t launch_rmsnorm_rows(const uint16_t* H, int R, int D, const uint16_t* ln, float eps, uint16_t* xn,
                               hipStream_t st) {
    if (R <= 0) return hipSuccess;
    const int cpl = ((D >> 3) + kWave - 1) / kWave;
    if (cpl > kMaxChunksPerLane) return hipErrorInvalidValue;
    const dim3 grid((R + 3) / 4), block(256);
    switch (cpl) {
#define SPECFOLD_NORM_CASE(C) \
    case C: hipLaunchKernelGGL(rmsnorm_rows_kernel<C>, grid, block, 0, st, H, R, D, ln, eps, xn); break;
        SPECFOLD_NORM_CASE(1) SPECFOLD_NORM_CASE(2) SPECFOLD_NORM_CASE(3) SPECFOLD_NORM_CASE(4)
        SPECFOLD_NORM_CASE(5) SPECFOLD_NORM_CASE(6) SPECFOLD_NORM_CASE(7) SPECFOLD_NORM_CASE(8)
        SPECFOLD_NORM_CASE(9) SPECFOLD_NORM_CASE(10)
#undef SPECFOLD_NORM_CASE
    }
    return hipGetLastError();
}

hipError_t launch_gate(const GateParams& p, hipStream_t st) {
    const int R = p.nb * p.N;
    if (R <= 0) return hipSuccess;
    const int cpl = ((p.D >> 3) + kWave - 1) / kWave;
    if (cpl > kMaxChunksPerLane) return hipErrorInvalidValue;
    const int win = p.N >= kGateWin ? kGateWin : (p.N + 3) / 4 * 4;
    const int n_win = (p.N + win - 1) / win;
    const int xcd_map = n_win >= 8 ? 1 : 0;
    const long windows = xcd_map ? (n_win + 7) / 8 * 8 : n_win;
    const long waves = windows * p.nb * win;
    const dim3 grid(static_cast<unsigned>(waves / 4)), block(256);
    switch (cpl) {
#define SPECFOLD_GATE_CASE(C) \
    case C: hipLaunchKernelGGL(gate_kernel<C>, grid, block, 0, st, p, win, n_win, xcd_map); break;
        SPECFOLD_GATE_CASE(1) SPECFOLD_GATE_CASE(2) SPECFOLD_GATE_CASE(3) SPECFOLD_GATE_CASE(4)
        SPECFOLD_GATE_CASE(5) SPECFOLD_GATE_CASE(6) SPECFOLD_GATE_CASE(7) SPECFOLD_GATE_CASE(8)
        SPECFOLD_GATE_CASE(9) SPECFOLD_GATE_CASE(10)
#undef SPECFOLD_GATE_CASE
    }
    return hipGetLastError();
}

size_t compact_workspace_bytes(int R) {
    if (R <= kSmallCompact) return 0;
    const size_t ntiles = (static_cast<size_t>(R) + kCompactTile - 1) / kCompactTile;
    return (4 + ntiles) * 4;
}

hipError_t launch_compact(const CompactParams& p, void* ws, hipStream_t st) {
    if (p.R <= kSmallCompact) {
        hipLaunchKernelGGL(compact_kernel, dim3(1), dim3(1024), 0, st, p);
        return hipGetLastError();
    }
    const int ntiles = (p.R + kCompactTile - 1) / kCompactTile;
    if (!ws) return hipErrorInvalidValue;
    uint32_t* state = static_cast<uint32_t*>(ws);
    hipLaunchKernelGGL(compact_clear_kernel, dim3(1), dim3(1024), 0, st, state, 4 + ntiles);
    hipLaunchKernelGGL(compact_lookback_kernel<kLookbackThreads>, dim3(ntiles), dim3(kLookbackThreads), 0, st, p, state,
                       ntiles);
    return hipGetLastError();
}

hipError_t launch_resolve(const ResolveParams& p, hipStream_t st) {
    if (p.R <= 0) return hipSuccess;
    hipLaunchKernelGGL(resolve_kernel, dim3((p.R + 255) / 256), dim3(256), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_row_norm(const uint16_t* X, int R, int D, const float* inv_rms, float eps, const uint16_t* ln,
                           uint16_t* xn, hipStream_t st) {
    if (R <= 0) return hipSuccess;
    hipLaunchKernelGGL(row_norm_kernel, dim3((R + 3) / 4), dim3(256), 0, st, X, R, D, inv_rms, eps, ln, xn);
    return hipGetLastError();
}

}  // namespace specfold
