// The steps either side of the layer stack [SpecFold summary, App. B: embeddings and the
// language-model head stay outside the folded kernels; the head is not folded].
//
// Embedding gather: one wave per row copies the token's row of E in 16-byte pieces (E may
// exceed the 1 GB a buffer resource addresses, so these are plain 64-bit loads).
//
// Greedy token: the LM head itself is the GEMM with its greedy-token epilogue, which leaves
// per (column group, row) the best logit and its column; one wave per row merges those in
// column-group order: the higher logit wins, ties go to the lower column, NaN never wins.
#include "kernels.h"

namespace specfold {

namespace {

__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ tokens, int R,
                                                    const uint16_t* __restrict__ E, int V, int D,
                                                    uint16_t* __restrict__ H) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & (kWave - 1);
    if (row >= R) return;
    const int tok = tokens[row];
    const int nch = D >> 3;
    uint4* dst = reinterpret_cast<uint4*>(H + static_cast<size_t>(row) * D);
    if (tok < 0 || tok >= V) {
        const uint32_t nan2 = 0x7fc07fc0u;
        for (int k = lane; k < nch; k += kWave) dst[k] = make_uint4(nan2, nan2, nan2, nan2);
        return;
    }
    const uint4* src = reinterpret_cast<const uint4*>(E + static_cast<size_t>(tok) * D);
    for (int k = lane; k < nch; k += kWave) dst[k] = src[k];
}

__global__ __launch_bounds__(256) void argmax_merge_kernel(const float* __restrict__ arg_val,
                                                           const int32_t* __restrict__ arg_idx, int groups,
                                                           int R, int32_t* __restrict__ token,
                                                           float* __restrict__ logit) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & (kWave - 1);
    if (row >= R) return;
    float best = 0.f;
    int bi = -1;
    for (int g = lane; g < groups; g += kWave) {
        const size_t o = static_cast<size_t>(g) * R + row;
        const int i = arg_idx[o];
        const float v = arg_val[o];
        if (i >= 0 && (bi < 0 || v > best || (v == best && i < bi))) { best = v; bi = i; }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float ob = __shfl_xor(best, off, kWave);
        const int oi = __shfl_xor(bi, off, kWave);
        if (oi >= 0 && (bi < 0 || ob > best || (ob == best && oi < bi))) { best = ob; bi = oi; }
    }
    if (lane == 0) {
        token[row] = bi;
        logit[row] = bi < 0 ? __builtin_nanf("") : best;
    }
}

}  // namespace

hipError_t launch_embed(const int32_t* tokens, int R, const uint16_t* E, int V, int D, uint16_t* H, hipStream_t st) {
    if (R <= 0) return hipSuccess;
    hipLaunchKernelGGL(embed_kernel, dim3((R + 3) / 4), dim3(256), 0, st, tokens, R, E, V, D, H);
    return hipGetLastError();
}

hipError_t launch_argmax_merge(const float* arg_val, const int32_t* arg_idx, int groups, int R, int32_t* token,
                               float* logit, hipStream_t st) {
    if (R <= 0) return hipSuccess;
    hipLaunchKernelGGL(argmax_merge_kernel, dim3((R + 3) / 4), dim3(256), 0, st, arg_val, arg_idx, groups, R, token,
                       logit);
    return hipGetLastError();
}

}  // namespace specfold
