// Cross-lane steps of a wave's xor butterflies without the LDS crossbar:
// DPP moves within rows of 16 lanes, v_permlane16_swap / v_permlane32_swap
// across them.  Each step combines a lane's value with that of lane l ^ o,
// the partner __shfl_xor(x, o) would read, so a butterfly built from them
// adds (or takes maxima) in the same order, bit for bit.
#pragma once

#include "common.hpp"

namespace bi {

// The value of lane l ^ O (O = 1, 2, 4, 8: within a row of 16 lanes) by DPP
// moves: quad permutations for 1 and 2, a rotation of the row by 8 for 8, and
// for 4 the half-row mirror (l ^ 7) followed by the quad reversal (l ^ 3).
template <int O>
__device__ __forceinline__ float lane_xor(float v) {
    static_assert(O == 1 || O == 2 || O == 4 || O == 8, "within a row");
    const int x = __float_as_int(v);
    if constexpr (O == 1) return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));
    if constexpr (O == 2) return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));
    if constexpr (O == 8) return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false));
    const int t = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false);
    return __int_as_float(__builtin_amdgcn_update_dpp(0, t, 0x1B, 0xF, 0xF, false));
}

// Xor-butterfly over the 64 lanes, offsets 32, 16, ..., 1: at each step a
// lane combines its value with that of lane l ^ o (every lane ends with the
// same bits).  Offsets 32 and 16 use v_permlane32_swap / v_permlane16_swap,
// which leave each lane the pair (own value, partner's value) in some order;
// the sum and the maximum of a pair do not depend on that order.  The others
// are DPP moves, so no step goes through the LDS crossbar.
__device__ __forceinline__ float wave_sum(float x) {
    {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    x += lane_xor<8>(x);
    x += lane_xor<4>(x);
    x += lane_xor<2>(x);
    x += lane_xor<1>(x);
    return x;
}
__device__ __forceinline__ float wave_max(float x) {
    {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    x = fmaxf(x, lane_xor<8>(x));
    x = fmaxf(x, lane_xor<4>(x));
    x = fmaxf(x, lane_xor<2>(x));
    x = fmaxf(x, lane_xor<1>(x));
    return x;
}

// Lane l plus lane l ^ O (O = 1 .. 32), the step of a xor butterfly sum; for
// O = 16 and 32 the permlane swaps' pair, whose sum does not depend on its
// order.
template <int O>
__device__ __forceinline__ float xor_add(float x) {
    if constexpr (O == 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    } else if constexpr (O == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    } else {
        return x + lane_xor<O>(x);
    }
}

// The butterfly steps O, 2 O, ..., END / 2 in that order (END a power of two
// up to 64): the sum over the lanes that differ from l only in those bits.
template <int O, int END>
__device__ __forceinline__ float xor_sum_steps(float x) {
    if constexpr (O < END) return xor_sum_steps<2 * O, END>(xor_add<O>(x));
    else return x;
}

}  // namespace bi
