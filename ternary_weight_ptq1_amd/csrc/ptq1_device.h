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
// Walsh-Hadamard transform of one 1024-wide chunk held by one wavefront:
// lane l holds elements l + 64 j in v[j], j = 0..15.  Natural-order
// (Sylvester) H: the butterfly pairs element i with i ^ h for h = 1 .. 512.
// Pairs with h >= 64 sit in one lane (index j ^ (h/64)); pairs with h < 64
// are in lanes l and l ^ h.  Unnormalised: returns H v.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void fwht1024_wave(float (&v)[kRotPerLane])
{
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int h = 1; h < kWave; h <<= 1) {
        const float sgn = (lane & h) ? -1.0f : 1.0f;
#pragma unroll
        for (int j = 0; j < kRotPerLane; ++j) {
            const float o = __shfl_xor(v[j], h, kWave);
            v[j] = fmaf(sgn, v[j], o);  // low index: v + o; high index: o - v
        }
    }
#pragma unroll
    for (int hj = 1; hj < kRotPerLane; hj <<= 1) {
#pragma unroll
        for (int j = 0; j < kRotPerLane; ++j) {
            if ((j & hj) == 0) {
                const float a = v[j], b = v[j + hj];
                v[j] = a + b;
                v[j + hj] = a - b;
            }
        }
    }
}

}  // namespace ptq1
