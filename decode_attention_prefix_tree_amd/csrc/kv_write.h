// Host-callable launcher of the KV write kernel: copies new tokens' K/V (or
// another slot's keys, after a chunk split) into chunk tiles.  Plain types
// only, so the C-ABI layer never sees HIP device code.
#pragma once

#include <cstdint>

#include "kernels.h"

namespace chunkattn {

constexpr int kOpsPerLaunch = 64;  // 2 KiB of kernel arguments

// One copy into one 64-key tile: keys [dst_key0, dst_key0 + n_rows) of tile
// dst_tile.  Source row r is caller row src0 + r, or (from_pool) key
// (src0 + r) % 64 of pool tile (src0 + r) / 64, so a chunk split's tail may
// come from two tiles.  Keys in [zero_lo, zero_hi) that are not written
// become zeros (a chunk's first write clears the chunk's part of the tile);
// every other key keeps its value.
// mode kKvRowWrite: the chunk is stored row-major (tile_layout.h): the caller
// rows go to their key rows, nothing else is written (rows past a chunk's
// fill are never read).  mode kKvToTiles: the chunk's part of the tile,
// keys [zero_lo, zero_hi), is rewritten from the row layout to the tile
// layout: keys below zero_lo + n_rows keep their values, the rest become
// zeros (the chunk becomes shared, or is split, and the chunk-first path and
// pool-to-pool copies read tiles).
enum { kKvTileWrite = 0, kKvRowWrite = 1, kKvToTiles = 2 };
struct KvOpDev {
  int32_t dst_tile, dst_key0, n_rows, src0, from_pool, zero_lo, zero_hi, mode;
};

struct KvOpBatch {
  KvOpDev ops[kOpsPerLaunch];
};

// int32 stores into the device chunk table done by the same launch (fill
// counts of chunks that grew in place), offsets in int32 units.
constexpr int kMaxPatches = 2 * kOpsPerLaunch;
struct TablePatches {
  int32_t n;
  int32_t off[kMaxPatches];
  int32_t val[kMaxPatches];
};

// Returns a hipError_t value (0 = success) from the launch.  Block 0 also
// does the table stores (table: the workspace base, device address).
int launch_kv_write(void* pool, int heads, const KvOpBatch& batch, int n_ops, const void* k_src,
                    const void* v_src, int32_t* table, const TablePatches& patches, void* stream);

}  // namespace chunkattn
