// Shared geometry of the gathered latent-row blocks (gfx950): the MLA row, the 32-key
// blocks the sparse attention and the group centroid gather into LDS, and the
// direct-to-LDS loads that fill them.
#pragma once
#include "dsa_common.hpp"

namespace dsa {

constexpr int kMlaD = 576;                      // latent row: 512-d compressed KV + 64-d RoPE key
constexpr int kMlaDv = 512;
constexpr int kBlk = 16;                        // keys per 16-key block
constexpr int kRowBytes = kMlaD * 2;            // 1152
constexpr int kChunks = kRowBytes / 16;         // 72 chunks of 16 B per row
constexpr int kBlkBytes = kBlk * kRowBytes;     // 18432
constexpr float kLog2e = 1.4426950408889634f;

// compile-time index carrier for the unrolled load parts
template <int N>
struct Phase {
  static constexpr int value = N;
};

constexpr int kBlk2 = 32;                        // keys per 32-key block
constexpr int kBlk2Bytes = 2 * kBlkBytes;        // 36864
constexpr int kDmaPerBlk2 = kBlk2Bytes / 1024;   // 36 wave-wide 1 KB direct-to-LDS loads

// LDS layout of a 36 KB block of 32 latent rows: key group w (keys 8 w .. 8 w + 7)
// occupies 9 KB, whose 1 KB segment u holds bytes [128 u, 128 u + 128) of the 8 rows, row r
// at 128 r with its 16-byte chunks XOR-swizzled by the row: chunk c sits in slot c ^ r.  One
// direct-to-LDS load fills one segment of one group (lane l: row l / 8, slot l % 8), so a
// lane needs one key per group, the nine segments of a row differ only by an immediate
// offset, and each load covers eight whole 128-byte lines.  Measured on gfx950 (an LDS
// access probe): with this swizzle the K operand reads (ds_read_b128) run conflict-free at
// about 246 bytes per clock and CU, and the transposed V^T reads (ds_read_b64_tr_b16) at
// about 206; the row-major layout reached 128 on the V^T reads, and a swizzle by
// ((r & 3) << 1) | (r >> 2) about 130 on both.
constexpr int kSegBytes = 1024;                   // one 128-byte segment of 8 rows
constexpr int kGroupBytes = 9 * kSegBytes;        // 8 rows of 1152 bytes

__device__ __forceinline__ int sw8(int r) { return r; }

// byte offset of 16-byte chunk c of row r of a block in that layout
__device__ __forceinline__ int blk_chunk_off(int r, int c) {
  return (r >> 3) * kGroupBytes + (c >> 3) * kSegBytes + (r & 7) * 128 + 16 * ((c & 7) ^ sw8(r & 7));
}

// segments U .. U1-1 of one key group: src is the lane's address in its row (slot included),
// lds the group's LDS address
template <int U, int U1>
__device__ __forceinline__ void dma_group_segs(const uint8_t* src, uint32_t lds) {
  if constexpr (U < U1) {
    // the instruction offset moves the LDS destination as well as the global address
    dma_16o<128 * U>(src, lds + (kSegBytes - 128) * U);
    dma_group_segs<U + 1, U1>(src, lds);
  }
}

}  // namespace dsa
