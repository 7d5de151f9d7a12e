// Cross-lane reductions that stay in the VALU: DPP lane moves and gfx950's row-swap permutes
// (v_permlane16_swap / v_permlane32_swap) instead of LDS-routed shuffles, which cost one LDS
// round trip per step.  The summation order is fixed, so results are deterministic.
#pragma once
#include "common.h"

namespace specfold {

// x moved by the DPP control CTRL; lanes outside ROW_MASK (16-lane rows) read 0
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_move(float x) {
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xF, false));
}

// Sum over the 64 lanes, returned in every lane (all lanes must be active).  Inside each 16-lane
// row: neighbour pairs, quads, half-row mirror, row mirror (every lane then holds its row's
// sum); row 1 adds row 0 and row 3 adds row 2 (row_bcast:15), rows 2-3 add lane 31
// (row_bcast:31), so lane 63 holds the total, which a scalar register broadcasts.
__device__ __forceinline__ float wave_sum_dpp(float x) {
    x += dpp_move<0xB1>(x);          // quad_perm [1,0,3,2]
    x += dpp_move<0x4E>(x);          // quad_perm [2,3,0,1]
    x += dpp_move<0x141>(x);         // row_half_mirror
    x += dpp_move<0x140>(x);         // row_mirror
    x += dpp_move<0x142, 0xA>(x);    // row_bcast:15 into rows 1 and 3
    x += dpp_move<0x143, 0xC>(x);    // row_bcast:31 into rows 2 and 3
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// The pair {x[l], x[l ^ 16]} in every lane l, from gfx950's v_permlane16_swap on two copies of
// x: it exchanges the odd 16-lane rows of its first operand with the even rows of its second,
// so the first ends up holding the even row of each row pair and the second the odd one.  The
// swap is written as inline asm with both operands read and written (two registers); the
// compiler's intrinsic for it drops the second result here.  The s_nop pads cover the
// VALU-write / permute-read dependency on either side.
__device__ __forceinline__ void pair16(float x, float& a, float& b) {
    unsigned u = __builtin_bit_cast(unsigned, x), v = u;
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(u), "+v"(v));
    a = __builtin_bit_cast(float, u);
    b = __builtin_bit_cast(float, v);
}

// ... and {x[l], x[l ^ 32]} with v_permlane32_swap (the upper half of the first operand with
// the lower half of the second)
__device__ __forceinline__ void pair32(float x, float& a, float& b) {
    unsigned u = __builtin_bit_cast(unsigned, x), v = u;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(u), "+v"(v));
    a = __builtin_bit_cast(float, u);
    b = __builtin_bit_cast(float, v);
}

// max and sum over lanes {l, l ^ 16, l ^ 32, l ^ 48}, in every lane
__device__ __forceinline__ float max_rows4(float x) {
    float a, b;
    pair16(x, a, b);
    x = fmaxf(a, b);
    pair32(x, a, b);
    return fmaxf(a, b);
}

__device__ __forceinline__ float sum_rows4(float x) {
    float a, b;
    pair16(x, a, b);
    x = a + b;
    pair32(x, a, b);
    return a + b;
}

}  // namespace specfold
