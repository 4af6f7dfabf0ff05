// Cross-lane reductions on DPP moves.
//
// Within each row of 16 lanes, four DPP moves pair lane i with i ^ 1, i ^ 2,
// then the mirror lane of its half row and of its row: after combining with
// each partner, all 16 lanes hold the row's result.  A register-to-register
// DPP move replaces the LDS-crossbar round trip a generic shuffle takes.  A
// wave's result then adds (or takes the maximum of) the four row results,
// read out of lanes 0, 16, 32 and 48 in that order.  Integer sums and
// maxima are exact in any order; floating-point sums take this fixed order
// in every call.  Every lane of the wave must be active.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlin {

// The step-th partner of the 16-lane butterfly (0xB1: quad_perm [1,0,3,2];
// 0x4E: quad_perm [2,3,0,1]; 0x141: row_half_mirror; 0x140: row_mirror).
__device__ inline int dpp_partner(int v, int step)
{
    switch (step) {
    case 0: return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);
    case 1: return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);
    case 2: return __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false);
    default: return __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false);
    }
}

__device__ inline float dpp_partner(float v, int step)
{
    return __int_as_float(dpp_partner(__float_as_int(v), step));
}

__device__ inline double dpp_partner(double v, int step)
{
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)dpp_partner((int)(uint32_t)b, step);
    const uint32_t hi = (uint32_t)dpp_partner((int)(uint32_t)(b >> 32), step);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

template <typename T>
__device__ inline T lane_value(T v, int lane);

template <>
__device__ inline int32_t lane_value<int32_t>(int32_t v, int lane)
{
    return __builtin_amdgcn_readlane(v, lane);
}

template <>
__device__ inline float lane_value<float>(float v, int lane)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

template <>
__device__ inline double lane_value<double>(double v, int lane)
{
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Sum / maximum over each aligned group of 16 lanes (all 16 get it).
template <typename T>
__device__ inline T row16_sum(T v)
{
#pragma unroll
    for (int s = 0; s < 4; ++s)
        v += dpp_partner(v, s);
    return v;
}

__device__ inline float row16_max(float v)
{
#pragma unroll
    for (int s = 0; s < 4; ++s)
        v = fmaxf(v, dpp_partner(v, s));
    return v;
}

// Sum / maximum over the wave (every lane gets it).
template <typename T>
__device__ inline T wave_sum(T v)
{
    v = row16_sum(v);
    return ((lane_value(v, 0) + lane_value(v, 16)) + lane_value(v, 32)) + lane_value(v, 48);
}

__device__ inline float wave_max(float v)
{
    v = row16_max(v);
    return fmaxf(fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)), lane_value(v, 32)),
                 lane_value(v, 48));
}

}  // namespace qlin
