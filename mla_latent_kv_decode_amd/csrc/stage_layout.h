// LDS layout of the decode cores' latent stages (gfx950).
//
// A 16-row block of cached latent rows is stored with the c_kv part (64
// chunks of 16 bytes) of row r at r * 1024 and the rope part (8 chunks) of row
// r at rope_off + r * 128.  Chunk c of a row sits at c ^ lat_swz(r) (inside
// its aligned group of 16 chunks) and rope chunk c at c ^ rope_swz(r).  With
// 64 four-byte banks, ds_read_b128 served 16 lanes at a time and
// ds_read_b64_tr_b16 32 lanes at a time:
//  - the row-wise operand reads (lane l: row l % 16, one 16-byte chunk) hit
//    16 distinct chunk positions, because lat_swz is a permutation of 0..15;
//  - the transposing reads (lanes of a 16-lane group: rows 4g .. 4g+3, the
//    chunk pair 2cb, 2cb+1) hit 8 distinct chunk pairs per 32 lanes, because
//    lat_swz(r) / 2 = r & 7 differs for the 8 rows and keeps pairs together.
#pragma once

namespace mla {

__device__ __forceinline__ constexpr int lat_swz(int r) { return 2 * (r & 7) | ((r >> 3) & 1); }
__device__ __forceinline__ constexpr int rope_swz(int r) { return (r >> 1) & 7; }

}  // namespace mla
