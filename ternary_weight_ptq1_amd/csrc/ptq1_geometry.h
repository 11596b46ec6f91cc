// ptq1_geometry.h -- the one place the PTQ1_0 block geometry and the launch
// geometry of every kernel are defined.  Host validation, launch code and
// kernels all read these constants; ptq1_geometry() exports them so a test
// can hold them against the public header and the oracle.
//
// Block format ("A 27B model in 5.5 GB: Bonsai ternary on Ferrox, locally",
// section "What Bonsai is"): 128 ternary weights with one 16-bit scale, five
// trits per byte in base 3 -> ceil(128/5) = 26 trit bytes, then the scale:
// 28 bytes = 224 bits = 1.75 bits per weight.  The fold uses a 1024-wide
// Walsh-Hadamard butterfly (same section).
#pragma once
#include <cstdint>

namespace ptq1 {

constexpr int kBlockWeights = 128;   // weights per block
constexpr int kTritsPerByte = 5;     // 3^5 = 243 <= 256
constexpr int kTritBytes = 26;       // ceil(128 / 5)
constexpr int kScaleOffset = 26;     // fp16 scale, little-endian, after the trits
constexpr int kBlockBytes = 28;      // 26 + 2
constexpr int kBlockDwords = 7;      // 28 / 4
constexpr int kHadamard = 1024;      // rotation width
constexpr int kBlocksPerChunk = kHadamard / kBlockWeights;  // 8

static_assert(kTritBytes * kTritsPerByte >= kBlockWeights, "trit bytes hold a block");
static_assert((kTritBytes - 1) * kTritsPerByte < kBlockWeights, "no spare trit byte");
static_assert(kBlockBytes == kTritBytes + 2 && kBlockBytes % 4 == 0, "block is whole dwords");

// ---- device weight layout (this library's, not the file format's) ----------
// The blocks of a matrix reordered into tiles of 32 rows x 2 blocks: one tile
// is 64 whole blocks = 1792 contiguous bytes, so a wave that needs 32 rows x
// 256 weights of K reads one contiguous run instead of 32 strided pieces.
// Tiles are stored K-slice-major (tile of band g, slice t at t * G + g), the
// order in which the decode matvec walks them.
constexpr int kTileRows = 32;
constexpr int kTileBlocks = 2;
constexpr int kTileSlots = kTileRows * kTileBlocks;   // 64 blocks
constexpr int kTileBytes = kTileSlots * kBlockBytes;  // 1792
static_assert(kTileBytes % 128 == 0, "tiles are whole 128-byte lines");

// ---- PQ2_0 ("Why I Am Building Another Inference Engine", Level 2: two bits
// per ternary weight plus a 16-bit scale for every 128 weights).  Block: 32 code
// bytes (weight 4i+n = 2-bit field n of byte i, low field first; code q is
// weight q - 1, code 3 reads as 0), then the scale: 34 bytes.  Device tile:
// 32 rows x 2 blocks as above, the 64 code records first (32 bytes each,
// place 2i + b = block b of row i) and then the 64 scales in the same order,
// so every record is 16-byte aligned.
constexpr int kPq2CodesPerByte = 4;
constexpr int kPq2CodeBytes = 32;                                  // 128 / 4
constexpr int kPq2BlockBytes = 34;                                 // 32 + 2
constexpr int kPq2TileCodeBytes = kTileSlots * kPq2CodeBytes;      // 2048
constexpr int kPq2TileBytes = kPq2TileCodeBytes + kTileSlots * 2;  // 2176
static_assert(kPq2CodeBytes * kPq2CodesPerByte == kBlockWeights, "code bytes hold a block");
static_assert(kPq2TileBytes % 16 == 0, "PQ2_0 tiles keep 16-byte alignment");

// ---- launch geometry -------------------------------------------------------
constexpr int kWave = 64;                       // CDNA wavefront

// float-peel matvec: lane <-> output row, workgroup <-> (row tile, 1024-chunk)
constexpr int kMvWaves = 4;
constexpr int kMvThreads = kMvWaves * kWave;    // 256 rows per workgroup
constexpr int kMvRowsPerWg = kMvThreads;

// reductions / element-wise kernels
constexpr int kEwThreads = 256;

// MFMA GEMM tile (bf16 32x32x16 MFMA, fp32 accumulate)
constexpr int kGemmBN = 128;                    // weight rows (output columns) per workgroup
constexpr int kGemmThreads = 256;

}  // namespace ptq1
