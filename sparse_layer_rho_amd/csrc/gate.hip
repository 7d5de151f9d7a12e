// Gate, compaction, fold-source resolution and row RMSNorm.
//
// Gate [SpecFold review, "무엇과 다른가"]: per draft row (i, n) with parent p = par(i),
// rho = |H_i[n] - H_p[n]| / |H_p[n]| and the row folds when rho <= delta; main rows bypass
// the gate [SpecFold summary, App. B].  One 64-lane wave owns one row: the lanes stream the
// child and parent rows in 16-byte chunks (coalesced), accumulate in fp32 and reduce with
// cross-lane shuffles.  The same loads give the row's sum of squares, i.e. its RMSNorm scale,
// and -- when asked -- the normalised row the QKV projection consumes (RMSNorm weight applied,
// rounded to bf16), so the layer input is read from HBM once.
//
// Compaction [SpecFold summary, App. B]: an exclusive scan of the recompute flags in row order
// (wave ballots + a cross-wave scan in LDS) writes the global list, the per-branch offsets and
// the inverse map row -> slot.  Past 8192 rows the scan runs over tiles in three passes (count,
// tile offsets, scan from the offset), so large inputs use the whole GPU.
//
// Sources [SpecFold summary, App. B and §A.3]: every row walks its fold chain up the parent map
// (at most n_branch steps; branch 0 always terminates) -- rows are independent, so one
// order-free launch covers all branches.
#include "kernels.h"

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
// holds chunks l, l + 64, ... (CPL of them) of the child and the parent row and of the norm
// weights; all of them are requested before any is used (chunks past the row, and the parent of
// a main row, read zeros from an out-of-range offset), so a row costs one memory round trip.
template <int CPL>
__device__ __forceinline__ void gate_row(const GateParams& p, int row, int lane) {
    const int i = row / p.N, n = row - i * p.N;
    const bool need_pair = (i > 0) && (p.rho_in == nullptr);
    const bool need_rows = need_pair || (p.inv_rms != nullptr) || (p.xn != nullptr);
    const int nch = p.D >> 3;
    float a = 0.f, b = 0.f, ss = 0.f;
    uint4 cv[CPL], wv[CPL];
    if (p.xn && p.ln) load_norm_weights<CPL>(p.ln, p.D, lane, wv);
    if (need_rows) {
        const __amdgpu_buffer_rsrc_t rH =
            make_rsrc(p.H, static_cast<uint32_t>(static_cast<size_t>(p.nb) * p.N * p.D * 2));
        const uint32_t cb = static_cast<uint32_t>(row) * p.D * 2;
        const uint32_t pb = need_pair ? static_cast<uint32_t>(p.par.p[i] * p.N + n) * p.D * 2 : kOob;
        uint4 pv[CPL];
#pragma unroll
        for (int t = 0; t < CPL; ++t) {
            const int k = lane + t * kWave;
            cv[t] = buf_load16(rH, k < nch ? cb + 16 * k : kOob);
            pv[t] = buf_load16(rH, k < nch ? pb + 16 * k : kOob);
        }
#pragma unroll
        for (int t = 0; t < CPL; ++t) {
            float x[8], yv[8];
            unpack8(cv[t], x);
            unpack8(pv[t], yv);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float d = x[e] - yv[e];
                ss += x[e] * x[e];
                a += d * d;
                b += yv[e] * yv[e];
            }
        }
        a = wave_sum(a);
        b = wave_sum(b);
        ss = wave_sum(ss);
    }
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
                unpack8(cv[t], x);
                o[k] = p.ln ? norm_chunk_w(x, inv, wv[t]) : norm_chunk(x, inv, nullptr, k);
            }
        }
    }
}

template <int CPL>
__global__ __launch_bounds__(256) void gate_kernel(const GateParams p) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row < p.nb * p.N) gate_row<CPL>(p, row, threadIdx.x & (kWave - 1));
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

// Large inputs: tiles of kCompactTile rows.  Pass 1 counts each tile's recompute rows into the
// first row_slot entry of the tile (scratch that pass 3 overwrites), pass 2 turns the counts
// into exclusive offsets, pass 3 scans every tile from its offset.  A tile is 32768 rows, so a
// 2^24-row input is 512 tiles: one workgroup per tile stays resident on the CUs at once.
constexpr int kCompactTile = 32768;
constexpr int kScatterSub = 8192;               // rows of one scan step of pass 3 (8 per thread)
constexpr int kSmallCompact = 8192;             // up to this many rows one workgroup scans them all

__global__ __launch_bounds__(1024) void compact_count_kernel(const CompactParams p) {
    __shared__ int s_tot[16];
    const int tile = blockIdx.x, tid = threadIdx.x;
    const int r0 = tile * kCompactTile;
    // thread t counts the kRowsPerThread rows from r0 + kRowsPerThread t: 16-byte loads, or byte
    // loads where the array ends inside them (the flags are bytes; nothing past R is read)
    constexpr int kRowsPerThread = kCompactTile / 1024;
    static_assert(kRowsPerThread % 16 == 0, "whole 16-byte loads");
    const int rt = r0 + kRowsPerThread * tid;
    int cnt = 0;
    if (rt + kRowsPerThread <= p.R) {
        uint4 v[kRowsPerThread / 16];
#pragma unroll
        for (int c = 0; c < kRowsPerThread / 16; ++c) v[c] = *reinterpret_cast<const uint4*>(p.fold + rt + 16 * c);
#pragma unroll
        for (int c = 0; c < kRowsPerThread / 16; ++c) {
            const uint32_t w[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int b = 0; b < 4; ++b) cnt += ((w[q] >> (8 * b)) & 0xffu) == 0 ? 1 : 0;
        }
    } else {
        for (int r = rt; r < p.R && r < rt + kRowsPerThread; ++r) cnt += p.fold[r] == 0 ? 1 : 0;
    }
    cnt = static_cast<int>(wave_sum(static_cast<float>(cnt)));
    if ((tid & 63) == 0) s_tot[tid >> 6] = cnt;
    __syncthreads();
    if (tid == 0) {
        int tot = 0;
        for (int w = 0; w < 16; ++w) tot += s_tot[w];
        p.row_slot[r0] = tot;
    }
}

__global__ __launch_bounds__(1024) void compact_offsets_kernel(const CompactParams p, int ntiles) {
    __shared__ int s_wave[16];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    // thread t owns tiles 2t, 2t+1 (ntiles <= 2048); a wave scan with shuffles, then the waves'
    // totals from LDS
    const int a = 2 * tid < ntiles ? p.row_slot[2 * tid * kCompactTile] : 0;
    const int b = 2 * tid + 1 < ntiles ? p.row_slot[(2 * tid + 1) * kCompactTile] : 0;
    int incl = a + b;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int t = __shfl_up(incl, d, kWave);
        if (lane >= d) incl += t;
    }
    if (lane == kWave - 1) s_wave[wave] = incl;
    __syncthreads();
    int woff = 0, total = 0;
    for (int w = 0; w < 16; ++w) {
        const int t = s_wave[w];
        woff += w < wave ? t : 0;
        total += t;
    }
    const int excl = woff + incl - (a + b);
    if (2 * tid < ntiles) p.row_slot[2 * tid * kCompactTile] = excl;
    if (2 * tid + 1 < ntiles) p.row_slot[(2 * tid + 1) * kCompactTile] = excl + a;
    if (tid == 0) {
        p.rec_count[0] = total;
        p.branch_off[p.nb] = total;
    }
}

// Pass 3: the tile is four steps of 8192 rows; in each, thread t owns the 8 consecutive rows
// 8t .. 8t+7 of the step.  Every step's flags (one 8-byte load per thread) and the tile's offset
// are requested at once (one memory round trip per tile); then, step by step, a
// workgroup-wide exclusive scan of the per-thread counts places the thread's recompute rows,
// the thread writes its 8 row -> slot entries as two 16-byte stores, and the step's list is
// gathered in LDS and written out in consecutive stores.
__global__ __launch_bounds__(1024) void compact_scatter_kernel(const CompactParams p) {
    static_assert(kScatterSub == 8 * 1024 && kCompactTile % kScatterSub == 0, "8 rows per thread and step");
    constexpr int kSteps = kCompactTile / kScatterSub;
    __shared__ int s_wave[2][16];
    __shared__ int s_base;
    __shared__ int s_list[kScatterSub];            // one step's recompute rows, in slot order
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int r0 = blockIdx.x * kCompactTile;
    uint32_t bits[kSteps];                         // bit b: row rt + b exists and is recomputed
#pragma unroll
    for (int q = 0; q < kSteps; ++q) {
        const int rt = r0 + q * kScatterSub + 8 * tid;
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
    if (tid == 0) s_base = p.row_slot[r0];         // the tile's offset (pass 2)
    __syncthreads();
    int base = s_base;
#pragma unroll
    for (int q = 0; q < kSteps; ++q) {
        const int rt = r0 + q * kScatterSub + 8 * tid;
        const int cnt = __popc(bits[q]);
        int incl = cnt;                            // inclusive scan over the wave
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int t = __shfl_up(incl, d, kWave);
            if (lane >= d) incl += t;
        }
        if (lane == kWave - 1) s_wave[q & 1][wave] = incl;
        __syncthreads();                           // (two buffers: step q+1 writes the other)
        int local = 0, tot = 0;
        for (int w = 0; w < 16; ++w) {
            const int t = s_wave[q & 1][w];
            local += w < wave ? t : 0;
            tot += t;
        }
        local += incl - cnt;                       // step-local index of the thread's first recompute row
        const int step_base = base;
        int slot = base + local;                   // slot of the thread's first recompute row
        base += tot;
        const uint32_t bq = bits[q];
        // branch starts among the thread's rows: one division per step, not one per row
        if (rt < p.R) {
            int br = (rt + p.N - 1) / p.N;
            for (int m = br * p.N; m < rt + 8 && m < p.R; m += p.N, ++br)
                p.branch_off[br] = slot + __popc(bq & ((1u << (m - rt)) - 1u));
        }
        int rs[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const int lb = local + __popc(bq & ((1u << b) - 1u));
            const bool rec = (bq >> b) & 1u;
            rs[b] = rec ? slot - local + lb : -1;
            if (rec) s_list[lb] = rt + b;
        }
        if (rt + 8 <= p.R) {
            int4* dst = reinterpret_cast<int4*>(p.row_slot + rt);
            dst[0] = make_int4(rs[0], rs[1], rs[2], rs[3]);
            dst[1] = make_int4(rs[4], rs[5], rs[6], rs[7]);
        } else {
            for (int b = 0; b < 8 && rt + b < p.R; ++b) p.row_slot[rt + b] = rs[b];
        }
        // the step's list leaves LDS in consecutive 4-byte stores (coalesced over each wave)
        __syncthreads();
        for (int e = tid; e < tot; e += 1024) p.rec_rows[step_base + e] = s_list[e];
        __syncthreads();                           // the list is read before the next step refills it
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
    const dim3 grid((R + 3) / 4), block(256);
    switch (cpl) {
#define SPECFOLD_GATE_CASE(C) \
    case C: hipLaunchKernelGGL(gate_kernel<C>, grid, block, 0, st, p); break;
        SPECFOLD_GATE_CASE(1) SPECFOLD_GATE_CASE(2) SPECFOLD_GATE_CASE(3) SPECFOLD_GATE_CASE(4)
        SPECFOLD_GATE_CASE(5) SPECFOLD_GATE_CASE(6) SPECFOLD_GATE_CASE(7) SPECFOLD_GATE_CASE(8)
        SPECFOLD_GATE_CASE(9) SPECFOLD_GATE_CASE(10)
#undef SPECFOLD_GATE_CASE
    }
    return hipGetLastError();
}

hipError_t launch_compact(const CompactParams& p, hipStream_t st) {
    if (p.R <= kSmallCompact) {
        hipLaunchKernelGGL(compact_kernel, dim3(1), dim3(1024), 0, st, p);
        return hipGetLastError();
    }
    const int ntiles = (p.R + kCompactTile - 1) / kCompactTile;
    if (ntiles > 2048) return hipErrorInvalidValue;
    hipLaunchKernelGGL(compact_count_kernel, dim3(ntiles), dim3(1024), 0, st, p);
    hipLaunchKernelGGL(compact_offsets_kernel, dim3(1), dim3(1024), 0, st, p, ntiles);
    hipLaunchKernelGGL(compact_scatter_kernel, dim3(ntiles), dim3(1024), 0, st, p);
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
