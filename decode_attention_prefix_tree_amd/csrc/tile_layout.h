// Device-side layout of the chunk pool, shared by the decode-step kernels
// and the KV write kernel.
//
// Tile layout.  The pool is a sequence of 64-key tiles, pool_tile_halves(H)
// apart (every head's K and V tile, one head's more when H is a power of
// two from 16 up); tile t, head h: K tile at t * pool_tile_halves(H) + (2h + 0) * 8192
// halves, V tile right after it (a chunk slot of 64 tokens is one tile, of
// 128 two, two slots of 32 share one).
// Within a tile the 64 x 128 fp16 elements
// are ordered so that every MFMA operand fetch is one contiguous 1 KB wave
// load (64 lanes x 16 bytes):
//  * K, as the A operand of S^T = K * Q^T (v_mfma_f32_32x32x16_f16, A lane
//    l = half*32 + i holds A[i][8*half + e], e < 8): load index
//    L = (key/32)*8 + dim/16, lane (dim/8 % 2)*32 + key%32, element dim%8.
//  * V, as the A operand of O^T = V^T * P^T: load index L = (dim/32)*4 +
//    key/16, lane ((key/4) % 2)*32 + dim%32, element (key%4) + 4*((key/8)%2).
//    That key order is the order in which the S^T accumulators of a lane
//    hold P^T, so P goes from the first product to the second without any
//    lane exchange.
//
// Row layout.  A chunk grown by decode appends keeps its keys row-major in
// the same 16 KiB K and V regions, so one token is one 256-byte K row and one
// 256-byte V row per head instead of pieces of two dozen lines of the tile
// layout.  Key k of the tile: K row at k * 128 halves; V row at
// (4 * ((k % 32) / 8) + 2 * (k / 32)) * 512 + (k % 8) * 128 halves.  Both keep
// keys 0..31 and 32..63 inside the units the tile layout gives those halves
// (K load blocks 0..7 and 8..15; V load blocks 4nb + 0, 1 and 4nb + 2, 3), so
// two 32-token chunks that share a tile never overlap in either layout, and
// rows 4j .. 4j + 3 are always 1 KiB of contiguous memory.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>

#include "kernels.h"

namespace chunkattn {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int D = kHeadDim;
constexpr int C = kChunk;
constexpr int TILE = C * D;  // halves per tile

__device__ __forceinline__ size_t tile_base(int tile, int head, int heads, int kv) {
  return static_cast<size_t>(tile) * static_cast<size_t>(pool_tile_halves(heads)) + (static_cast<size_t>(head) * 2 + kv) * TILE;
}

__device__ __forceinline__ int k_off(int key, int dim) {
  return ((((key >> 5) * 8 + (dim >> 4)) * 2 + ((dim >> 3) & 1)) * 32 + (key & 31)) * 8 + (dim & 7);
}

__device__ __forceinline__ int k_row_off(int key) { return key * D; }

__device__ __forceinline__ int v_row_off(int key) {
  return (4 * ((key & 31) >> 3) + 2 * (key >> 5)) * 512 + (key & 7) * D;
}

__device__ __forceinline__ int v_off(int key, int dim) {
  return ((((dim >> 5) * 4 + (key >> 4)) * 2 + ((key >> 2) & 1)) * 32 + (dim & 31)) * 8 +
         ((key & 3) | (((key >> 3) & 1) << 2));
}

}  // namespace chunkattn
