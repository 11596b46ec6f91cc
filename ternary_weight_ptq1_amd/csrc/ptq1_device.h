// ptq1_device.h -- device helpers shared by the HIP kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

#include "ptq1_geometry.h"

namespace ptq1 {

// ---------------------------------------------------------------------------
// Float-pipeline trit peel ("A 27B model in 5.5 GB: Bonsai ternary on
// Ferrox, locally", section "What Ferrox does with it"): with u = b / 256,
// digit n of the byte is floor(3^(n+1) u) - 3 floor(3^n u).  Here
// F_m = floor(b * (3^m / 256)); 3^m / 256 is exact in fp32 and b * 3^m is
// below 2^24, so every product, floor and difference below is exact.
// ---------------------------------------------------------------------------
struct Peel5 {
    float d0, d1, d2, d3, d4;  // digits in {0, 1, 2}, most significant first
};

__device__ __forceinline__ Peel5 peel5(float b)
{
    const float f1 = floorf(b * (3.0f / 256.0f));
    const float f2 = floorf(b * (9.0f / 256.0f));
    const float f3 = floorf(b * (27.0f / 256.0f));
    const float f4 = floorf(b * (81.0f / 256.0f));
    const float f5 = floorf(b * (243.0f / 256.0f));
    Peel5 p;
    p.d0 = f1;
    p.d1 = fmaf(-3.0f, f1, f2);
    p.d2 = fmaf(-3.0f, f2, f3);
    p.d3 = fmaf(-3.0f, f3, f4);
    p.d4 = fmaf(-3.0f, f4, f5);
    return p;
}

// Only digit n (0..4) of byte value b.
__device__ __forceinline__ float peel_digit(float b, int n)
{
    float hi = 3.0f, lo = 1.0f;
    for (int i = 0; i < n; ++i) { hi *= 3.0f; lo *= 3.0f; }
    return fmaf(-3.0f, floorf(b * (lo * (1.0f / 256.0f))), floorf(b * (hi * (1.0f / 256.0f))));
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits)
{
    _Float16 h = __builtin_bit_cast(_Float16, static_cast<uint16_t>(bits & 0xffffu));
    return static_cast<float>(h);
}

// fp32 -> bf16 bit pattern, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// ---------------------------------------------------------------------------
// Wave reductions without LDS round trips (DPP and the gfx950 lane swaps).
// ---------------------------------------------------------------------------
// Max over the wave, in every lane: quad permutations, row rotations, then
// the 16- and 32-lane swaps.
__device__ __forceinline__ float wave_max(float m)
{
    int im = __builtin_bit_cast(int, m);
    m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(im, im, 0xB1, 0xF, 0xF, false)));
    im = __builtin_bit_cast(int, m);
    m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(im, im, 0x4E, 0xF, 0xF, false)));
    im = __builtin_bit_cast(int, m);
    m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(im, im, 0x124, 0xF, 0xF, false)));
    im = __builtin_bit_cast(int, m);
    m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(im, im, 0x128, 0xF, 0xF, false)));
    const uint32_t u16 = __builtin_bit_cast(uint32_t, m);
    const auto r16 = __builtin_amdgcn_permlane16_swap(u16, u16, false, false);
    const uint32_t a0 = r16[0], a1 = r16[1];
    m = fmaxf(__builtin_bit_cast(float, a0), __builtin_bit_cast(float, a1));
    const uint32_t u32 = __builtin_bit_cast(uint32_t, m);
    const auto r32 = __builtin_amdgcn_permlane32_swap(u32, u32, false, false);
    const uint32_t b0 = r32[0], b1 = r32[1];
    return fmaxf(__builtin_bit_cast(float, b0), __builtin_bit_cast(float, b1));
}

// v of lane l plus v of lane l ^ H (H = 16 or 32), the lower lane's value
// first, so both lanes get the same sum: one lane-swap instruction instead of
// an LDS permute round trip.  (r[0] holds the lower lane's value and r[1]
// the upper one's in every lane.)
template <int H>
__device__ __forceinline__ float lane_pair_sum(float v)
{
    static_assert(H == 16 || H == 32, "16- or 32-lane swap");
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    uint32_t lo, hi;
    if constexpr (H == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        lo = r[0];
        hi = r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        lo = r[0];
        hi = r[1];
    }
    return __builtin_bit_cast(float, lo) + __builtin_bit_cast(float, hi);
}

// Sum over the wave: quad permutations, the half-row and row mirrors, then
// the 16- and 32-lane swaps.  Every step adds two values that the two lanes
// of a pair hold alike, so every lane ends with the same sum.
__device__ __forceinline__ float wave_sum(float v)
{
    int iv = __builtin_bit_cast(int, v);
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(iv, iv, 0xB1, 0xF, 0xF, false));   // lane ^ 1
    iv = __builtin_bit_cast(int, v);
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(iv, iv, 0x4E, 0xF, 0xF, false));   // lane ^ 2
    iv = __builtin_bit_cast(int, v);
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(iv, iv, 0x141, 0xF, 0xF, false));  // half-row mirror
    iv = __builtin_bit_cast(int, v);
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(iv, iv, 0x140, 0xF, 0xF, false));  // row mirror
    return lane_pair_sum<32>(lane_pair_sum<16>(v));
}

// ---------------------------------------------------------------------------
// Walsh-Hadamard butterflies on one wavefront, natural-order (Sylvester) H:
// the butterfly pairs element i with i ^ h.  Six index bits sit in the lane
// and the rest in the register index; pairs across lanes are exchanged
// without LDS traffic: DPP quad permutations (h = 1, 2), row shifts (h = 4),
// a half-row rotation (h = 8) and the gfx950 lane swaps (h = 16, 32).  A
// butterfly leaves v + o at the lane whose bit h is 0 and o - v at the
// other.  Unnormalised.
// ---------------------------------------------------------------------------
template <int kCtrl>
__device__ __forceinline__ float fwht_dpp(float v)
{
    const int iv = __builtin_bit_cast(int, v);
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(iv, iv, kCtrl, 0xF, 0xF, false));
}

// The six butterfly stages over the lane index (h = 1 .. 32) for each of
// the N values a lane holds.
template <int N>
__device__ __forceinline__ void fwht_lane_stages(float (&v)[N])
{
    const int lane = threadIdx.x & (kWave - 1);
    const float s1 = (lane & 1) ? -1.0f : 1.0f, s2 = (lane & 2) ? -1.0f : 1.0f;
    const float s4 = (lane & 4) ? -1.0f : 1.0f, s8 = (lane & 8) ? -1.0f : 1.0f;
    const float s16 = (lane & 16) ? -1.0f : 1.0f, s32 = (lane & 32) ? -1.0f : 1.0f;
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = fmaf(s1, v[j], fwht_dpp<0xB1>(v[j]));  // quad_perm [1,0,3,2]
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = fmaf(s2, v[j], fwht_dpp<0x4E>(v[j]));  // quad_perm [2,3,0,1]
#pragma unroll
    for (int j = 0; j < N; ++j) {
        // lane + 4 (row_shl:4) or lane - 4 (row_shr:4): both are read by
        // every lane before the select (a DPP read inside a branch would see
        // the inactive lanes' old values)
        const float up = fwht_dpp<0x104>(v[j]);
        const float dn = fwht_dpp<0x114>(v[j]);
        v[j] = fmaf(s4, v[j], (lane & 4) ? dn : up);
    }
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = fmaf(s8, v[j], fwht_dpp<0x128>(v[j]));  // row_ror:8
#pragma unroll
    for (int j = 0; j < N; ++j) {
        // element [0] of the swap holds the own value in lanes 0-15 of each
        // 32 and the partner's in 16-31; element [1] the other way round
        const uint32_t u = __builtin_bit_cast(uint32_t, v[j]);
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        const uint32_t r0 = r[0], r1 = r[1];
        v[j] = fmaf(s16, __builtin_bit_cast(float, r1), __builtin_bit_cast(float, r0));
    }
#pragma unroll
    for (int j = 0; j < N; ++j) {
        const uint32_t u = __builtin_bit_cast(uint32_t, v[j]);
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        const uint32_t r0 = r[0], r1 = r[1];
        v[j] = fmaf(s32, __builtin_bit_cast(float, r1), __builtin_bit_cast(float, r0));
    }
}

// The stages over the value index (h = 1 .. N / 2) in registers.
template <int N>
__device__ __forceinline__ void fwht_value_stages(float (&v)[N])
{
#pragma unroll
    for (int hj = 1; hj < N; hj <<= 1) {
#pragma unroll
        for (int j = 0; j < N; ++j) {
            if ((j & hj) == 0) {
                const float a = v[j], b = v[j + hj];
                v[j] = a + b;
                v[j + hj] = a - b;
            }
        }
    }
}

// 256 values on one wave, four per lane (element 64 j + lane in v[j], or any
// assignment of six index bits to the lane and two to j: the transform is
// the same butterfly on every bit).  Unnormalised: returns H_256 v.
__device__ __forceinline__ void fwht256_wave(float (&v)[4])
{
    fwht_lane_stages<4>(v);
    fwht_value_stages<4>(v);
}

}  // namespace ptq1
