// layout.h -- device layout of a packed compressed linear layer.
//
// Shared by the host packer and the HIP runtime.  Plain C++, no HIP types.
//
// Every dense stream is row-major in 16-byte chunks,
//
//     stream[row][chunk][bytes_per_chunk],
//
// a chunk covering `span` consecutive k of the row.  Rows are padded to whole
// chunks and N to whole 64-row tiles; padding bytes are zero.  A wavefront
// whose lanes take consecutive chunks of one row issues fully coalesced
// 128-bit loads (1 KiB per wavefront); a wavefront whose lanes take one row
// each reads one 128-byte line per lane every eight chunks.
//
// Per dense kind (bit positions count from the least significant bit):
//
//   LUT3  span 40: the chunk is 4 words; word i holds the ten 3-bit codes of
//         k = 40c + 10i + t, t = 0..9 (the same ten codes as the i-th canonical
//         10-per-word word of the row), rearranged so that the code pair
//         p_j = code[2j] | code[2j+1] << 3 (j = 0..4) sits in
//           p_0..p_3 : bits 2..7 of byte j (so the byte reads 4 * p_j);
//           p_4      : bits 0..1 of bytes 0, 1, 2 (two bits each, low bits first);
//         bits 0..1 of byte 3 are zero.
//   LUT4  span 32: word i holds codes k = 32c + 8i + t, t = 0..7; byte b of the
//         word holds the pair p_b = code[2b] | code[2b+1] << 4 rotated left by
//         two bits, so that bits 2..7 of the byte read 4 * (p_b mod 64) and bits
//         0..1 read p_b / 64 (a 1 KiB pair table is addressed with one v_perm).
//   INT4  span 32 (no mask): word i holds u = q + 8 of k = 32c + 8i + t; the
//         pair (2j, 2j+1) sits at bits 4j..4j+3 and 16+4j..16+4j+3.
//   INT4 + 2:4, span 64: 16 groups of four k per chunk.  DENSE word i holds
//         the two kept values (u = q + 8) of groups 4i..4i+3, group g' of the
//         word at bits 4g'..4g'+3 (first kept) and 16+4g'.. (second kept).
//         META (8 bytes per chunk) word i holds groups 8i..8i+7, a nibble
//         i0 | i1 << 2 per group (positions 0..3 of the two kept weights,
//         i0 < i1) at bits 4t..4t+3.
//   INT8  span 16 (no mask): byte t holds u = q + 128 of k = 16c + t.
//   INT8 + BITMAP, span 128: META (16 bytes per chunk) holds the keep bits,
//         bit t of word i <-> k = 128c + 32i + t.  The kept values (signed
//         int8, ascending k) of each row are contiguous in DENSE starting at
//         NZOFF[n] (a multiple of 16).
#pragma once
#include <stdint.h>

namespace cl {

constexpr int kTileRows = 64;
constexpr int kChunkBytes = 16;

struct KindInfo {
  int span;               // logical k per chunk of the dense stream (bitmap: per meta chunk)
  int meta_chunk_bytes;   // bytes of META per row per chunk
  int table_entries;      // LUT entries per row (0 for integer formats)
};

inline KindInfo kind_info(int dense, int mask) {
  // dense: 0 LUT3, 1 LUT4, 2 INT4, 3 INT8; mask: 0 none, 1 2:4, 2 bitmap
  if (dense == 0) return {40, 0, 8};
  if (dense == 1) return {32, 0, 16};
  if (dense == 2 && mask == 0) return {32, 0, 0};
  if (dense == 2 && mask == 1) return {64, 8, 0};
  if (dense == 3 && mask == 0) return {16, 0, 0};
  if (dense == 3 && mask == 2) return {128, 16, 0};
  return {0, 0, 0};
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Matrix-core prefill: output tiles of kPfTileN weight rows; K advances in steps
// of pf_step_k() (a whole number of chunks, a multiple of 16).
constexpr int kPfTileN = 128;
inline int pf_step_k(int dense, int mask) {
  if (dense == 0) return 80;               // LUT3: two chunks of 40
  if (dense == 2 && mask == 1) return 128;  // INT4 2:4: two chunks of 64
  return 64;
}
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
// Weight rows per prefill tile: the 3-bit LUT format runs the wide kernel
// (256-row tiles, outlier entries with an 8-bit row), the others 128.
inline int pf_tile_rows(int dense) { return dense == 0 ? 256 : kPfTileN; }

// Matrix-core decode (batch 2..32): 128-row tiles, split along K into slices
// of whole passes (a pass is eight chunks of every row of the tile).
constexpr int kMfRows = 128;    // weight rows per workgroup (four wavefronts of 32)
constexpr int kMfCph = 4;       // chunks per lane half per pass (two halves read one 128-byte line of a row)
constexpr int kLrCntWords = 128 + 32 * 32;  // low-rank prologue counters and generation words (u32)
constexpr int kMfKzMax = 1024;  // largest K slice (bounds the activation staging in LDS)
// (the bitmap format: one chunk per lane half and pass)
inline int mf_pass_k(int dense, int mask) {
  return 2 * (dense == 3 && mask == 2 ? 1 : kMfCph) * kind_info(dense, mask).span;
}
// Passes per K slice: about 1024 columns (768 for the 4-bit LUT, whose tables
// take more LDS), fewer when the layer would give under two workgroups per CU
// of a 256-CU device.  Independent of M, so that the outlier lists built at
// create serve every batch size.
inline int mf_passes(int dense, int mask, int K, int N) {
  const int passk = mf_pass_k(dense, mask);
  const int target = dense == 1 ? 768 : kMfKzMax;
  int npw = target / passk > 0 ? target / passk : 1;
  const int64_t tiles = ceil_div(N, kMfRows);
  while (npw > 1 && tiles * ceil_div(K, (int64_t)npw * passk) < 2 * 256) npw = npw / 2 > 0 ? npw / 2 : 1;
  return npw;
}

}  // namespace cl
