// codec.hip -- PTQ1_0 encode (pack) and decode (dequant) kernels, and the
// reorder of packed blocks into the library's tiled device layout.
//
// Format: "A 27B model in 5.5 GB: Bonsai ternary on Ferrox, locally",
// section "What Bonsai is" (five trits per byte in base 3, a 16-bit scale
// for every 128 weights); the decode reads digits on the float pipeline as in
// section "What Ferrox does with it".
#include "ptq1_device.h"
#include "ptq1_launch.h"

namespace ptq1 {

// One thread per output byte.  Trit bytes carry v = sum_n (t_n + 1) 3^(4-n)
// (padding digits are 1) as the smallest byte b with floor(243 b / 256) = v,
// b = ceil(256 v / 243); bytes 26..27 are the scale, little-endian.
__global__ void __launch_bounds__(256) k_pack(const int8_t *__restrict__ trits,
                                              const uint16_t *__restrict__ scales, int64_t nb,
                                              int64_t k, int64_t total, uint8_t *__restrict__ out)
{
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t blk = t / kBlockBytes;
        const int i = static_cast<int>(t - blk * kBlockBytes);
        const int64_t row = blk / nb;
        const int64_t b = blk - row * nb;
        uint32_t byte;
        if (i < kTritBytes) {
            const int8_t *src = trits + row * k + b * kBlockWeights + kTritsPerByte * i;
            uint32_t v = 0;
#pragma unroll
            for (int n = 0; n < kTritsPerByte; ++n) {
                int dgt = 1;
                if (kTritsPerByte * i + n < kBlockWeights) {
                    const int tv = src[n];
                    dgt = tv < -1 ? 0 : (tv > 1 ? 2 : tv + 1);
                }
                v = 3u * v + static_cast<uint32_t>(dgt);
            }
            byte = (256u * v + 242u) / 243u;
        } else {
            const uint32_t s = scales[row * nb + b];
            byte = (i == kScaleOffset) ? (s & 0xffu) : (s >> 8);
        }
        out[t] = static_cast<uint8_t>(byte);
    }
}

// One thread per weight: digit (c mod 128) mod 5 of byte (c mod 128) / 5.
__global__ void __launch_bounds__(256) k_dequant(const uint8_t *__restrict__ blocks, int64_t nb,
                                                 int64_t k, int64_t total, float *__restrict__ w)
{
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = t / k;
        const int64_t c = t - row * k;
        const int64_t b = c / kBlockWeights;
        const int j = static_cast<int>(c - b * kBlockWeights);
        const uint8_t *blk = blocks + (row * nb + b) * kBlockBytes;
        const float byte = static_cast<float>(blk[j / kTritsPerByte]);
        const float dgt = peel_digit(byte, j % kTritsPerByte);
        const uint32_t sb = blk[kScaleOffset] | (static_cast<uint32_t>(blk[kScaleOffset + 1]) << 8);
        w[t] = half_bits_to_float(sb) * (dgt - 1.0f);
    }
}

// Packed -> tiled reorder: one thread per 28-byte place of the tiled output
// (tiles of kTileRows rows x kTileBlocks blocks, K-slices outermost, then
// row bands; rows then blocks inside a tile); places past the matrix get
// zero bytes.
__global__ void __launch_bounds__(256) k_tile(const uint8_t *__restrict__ blocks, int64_t n, int64_t nb,
                                              int64_t bands, int64_t total, uint8_t *__restrict__ tiled)
{
    for (int64_t o = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; o < total;
         o += (int64_t)gridDim.x * blockDim.x) {
        const int64_t tile = o / kTileSlots;
        const int pos = static_cast<int>(o - tile * kTileSlots);
        const int64_t t = tile / bands;
        const int64_t band = tile - t * bands;
        const int64_t r = band * kTileRows + pos / kTileBlocks;
        const int64_t j = t * kTileBlocks + pos % kTileBlocks;
        uint32_t d[kBlockDwords];
#pragma unroll
        for (int q = 0; q < kBlockDwords; ++q) d[q] = 0;
        if (r < n && j < nb) {
            const uint32_t *src = reinterpret_cast<const uint32_t *>(blocks + (r * nb + j) * kBlockBytes);
#pragma unroll
            for (int q = 0; q < kBlockDwords; ++q) d[q] = src[q];
        }
        uint32_t *dst = reinterpret_cast<uint32_t *>(tiled + o * kBlockBytes);
#pragma unroll
        for (int q = 0; q < kBlockDwords; ++q) dst[q] = d[q];
    }
}

// ---- PQ2_0 codec -------------------------------------------------------------
// One thread per output byte: code bytes carry sum_f (t_f + 1) << 2f over the
// four weights 4i + f (trits outside {-1, 0, 1} are clamped, as in k_pack);
// bytes 32..33 are the scale, little-endian.
__global__ void __launch_bounds__(256) k_pq2_pack(const int8_t *__restrict__ trits,
                                                  const uint16_t *__restrict__ scales, int64_t nb,
                                                  int64_t k, int64_t total, uint8_t *__restrict__ out)
{
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t blk = t / kPq2BlockBytes;
        const int i = static_cast<int>(t - blk * kPq2BlockBytes);
        const int64_t row = blk / nb;
        const int64_t b = blk - row * nb;
        uint32_t byte = 0;
        if (i < kPq2CodeBytes) {
            const int8_t *src = trits + row * k + b * kBlockWeights + kPq2CodesPerByte * i;
#pragma unroll
            for (int f = 0; f < kPq2CodesPerByte; ++f) {
                const int tv = src[f];
                byte |= static_cast<uint32_t>(tv < -1 ? 0 : (tv > 1 ? 2 : tv + 1)) << (2 * f);
            }
        } else {
            const uint32_t s = scales[row * nb + b];
            byte = (i == kPq2CodeBytes) ? (s & 0xffu) : (s >> 8);
        }
        out[t] = static_cast<uint8_t>(byte);
    }
}

// One thread per weight: field (c mod 128) mod 4 of code byte (c mod 128) / 4.
__global__ void __launch_bounds__(256) k_pq2_dequant(const uint8_t *__restrict__ blocks, int64_t nb,
                                                     int64_t k, int64_t total, float *__restrict__ w)
{
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = t / k;
        const int64_t c = t - row * k;
        const int64_t b = c / kBlockWeights;
        const int j = static_cast<int>(c - b * kBlockWeights);
        const uint8_t *blk = blocks + (row * nb + b) * kPq2BlockBytes;
        const int q = (blk[j / kPq2CodesPerByte] >> (2 * (j % kPq2CodesPerByte))) & 3;
        const uint32_t sb = blk[kPq2CodeBytes] | (static_cast<uint32_t>(blk[kPq2CodeBytes + 1]) << 8);
        w[t] = half_bits_to_float(sb) * static_cast<float>(q == 3 ? 0 : q - 1);
    }
}

// Packed -> PQ2_0 tiled reorder: one thread per place of the tiled output
// (tile order as k_tile); places past the matrix get zero codes and a zero
// scale, so they contribute nothing.
__global__ void __launch_bounds__(256) k_pq2_tile(const uint8_t *__restrict__ blocks, int64_t n, int64_t nb,
                                                  int64_t bands, int64_t total, uint8_t *__restrict__ tiled)
{
    for (int64_t o = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; o < total;
         o += (int64_t)gridDim.x * blockDim.x) {
        const int64_t tile = o / kTileSlots;
        const int pos = static_cast<int>(o - tile * kTileSlots);
        const int64_t t = tile / bands;
        const int64_t band = tile - t * bands;
        const int64_t r = band * kTileRows + pos / kTileBlocks;
        const int64_t j = t * kTileBlocks + pos % kTileBlocks;
        uint32_t d[kPq2CodeBytes / 4];
        uint32_t sc = 0;
#pragma unroll
        for (int q = 0; q < kPq2CodeBytes / 4; ++q) d[q] = 0;
        if (r < n && j < nb) {
            // blocks are 34 bytes: only 2-byte aligned
            const uint16_t *src = reinterpret_cast<const uint16_t *>(blocks + (r * nb + j) * kPq2BlockBytes);
#pragma unroll
            for (int q = 0; q < kPq2CodeBytes / 4; ++q)
                d[q] = static_cast<uint32_t>(src[2 * q]) | (static_cast<uint32_t>(src[2 * q + 1]) << 16);
            sc = src[kPq2CodeBytes / 2];
        }
        uint8_t *tb = tiled + tile * kPq2TileBytes;
        uint32_t *dst = reinterpret_cast<uint32_t *>(tb + pos * kPq2CodeBytes);
#pragma unroll
        for (int q = 0; q < kPq2CodeBytes / 4; ++q) dst[q] = d[q];
        reinterpret_cast<uint16_t *>(tb + kPq2TileCodeBytes)[pos] = static_cast<uint16_t>(sc);
    }
}

static unsigned grid_for(int64_t total, int threads)
{
    int64_t g = (total + threads - 1) / threads;
    const int64_t cap = 256 * 1024;  // grid-stride beyond this
    if (g > cap) g = cap;
    if (g < 1) g = 1;
    return static_cast<unsigned>(g);
}

hipError_t launch_pack(const int8_t *trits, const uint16_t *scales, int64_t n, int64_t k,
                       uint8_t *blocks, hipStream_t s)
{
    const int64_t nb = k / kBlockWeights;
    const int64_t total = n * nb * kBlockBytes;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(k_pack, dim3(grid_for(total, 256)), dim3(256), 0, s, trits, scales, nb, k,
                       total, blocks);
    return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t *blocks, int64_t n, int64_t k, float *w, hipStream_t s)
{
    const int64_t total = n * k;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(k_dequant, dim3(grid_for(total, 256)), dim3(256), 0, s, blocks,
                       k / kBlockWeights, k, total, w);
    return hipGetLastError();
}

hipError_t launch_pq2_pack(const int8_t *trits, const uint16_t *scales, int64_t n, int64_t k, uint8_t *blocks,
                           hipStream_t s)
{
    const int64_t nb = k / kBlockWeights;
    const int64_t total = n * nb * kPq2BlockBytes;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(k_pq2_pack, dim3(grid_for(total, 256)), dim3(256), 0, s, trits, scales, nb, k, total, blocks);
    return hipGetLastError();
}

hipError_t launch_pq2_dequant(const uint8_t *blocks, int64_t n, int64_t k, float *w, hipStream_t s)
{
    const int64_t total = n * k;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(k_pq2_dequant, dim3(grid_for(total, 256)), dim3(256), 0, s, blocks, k / kBlockWeights, k,
                       total, w);
    return hipGetLastError();
}

hipError_t launch_pq2_tile(const uint8_t *blocks, int64_t n, int64_t k, uint8_t *tiled, hipStream_t s)
{
    const int64_t nb = k / kBlockWeights;
    const int64_t tiles_k = (nb + kTileBlocks - 1) / kTileBlocks;
    const int64_t bands = (n + kTileRows - 1) / kTileRows;
    const int64_t total = bands * tiles_k * kTileSlots;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(k_pq2_tile, dim3(grid_for(total, 256)), dim3(256), 0, s, blocks, n, nb, bands, total,
                       tiled);
    return hipGetLastError();
}

hipError_t launch_tile(const uint8_t *blocks, int64_t n, int64_t k, uint8_t *tiled, hipStream_t s)
{
    const int64_t nb = k / kBlockWeights;
    const int64_t tiles_k = (nb + kTileBlocks - 1) / kTileBlocks;
    const int64_t bands = (n + kTileRows - 1) / kTileRows;
    const int64_t total = bands * tiles_k * kTileSlots;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(k_tile, dim3(grid_for(total, 256)), dim3(256), 0, s, blocks, n, nb, bands, total,
                       tiled);
    return hipGetLastError();
}

}  // namespace ptq1
