// gfx950 kernel that writes new tokens' K and V into chunk tiles (the
// layout of tile_layout.h): rows of the caller's [row][head][128] fp16 K/V,
// or keys of another slot when a chunk split moves a tail into a new slot
// (prefix tree of chunks: paperlayer.ai summary of arXiv 2402.15220v4,
// section 3.1).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kv_write.h"
#include "tile_layout.h"

namespace chunkattn {

namespace {

// KV writes: caller rows or pool keys into one 64-key tile (K and V).
// grid (n_ops, heads, 2), 256 threads; a thread owns 4 of the tile's 1024
// 16-byte units.  Unless the piece clears the whole tile, only the units
// holding a written or cleared key are read and rewritten (a one-token
// append touches 16 K units and 128 V units of a head, not the whole 32 KiB
// pair).  Block (0, 0, 0) also stores the
// fill counts of chunks that grew in place into the device chunk table, so
// the next step on the stream sees them without a table upload.
__global__ __launch_bounds__(256) void kv_write_kernel(_Float16* pool, int heads, KvOpBatch batch,
                                                       const _Float16* k_src, const _Float16* v_src,
                                                       int32_t* table, TablePatches patches) {
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && static_cast<int>(threadIdx.x) < patches.n)
    table[patches.off[threadIdx.x]] = patches.val[threadIdx.x];
  const KvOpDev op = batch.ops[blockIdx.x];
  const int head = blockIdx.y, kv = blockIdx.z;
  _Float16* dst = pool + tile_base(op.dst_tile, head, heads, kv);
  const _Float16* src = kv ? v_src : k_src;
  if (op.mode == kKvRowWrite) {
    // 16 units of 16 bytes per row
    for (int w = threadIdx.x; w < op.n_rows * 16; w += 256) {
      const int r = w >> 4, u = w & 15, key = op.dst_key0 + r;
      *reinterpret_cast<h8*>(dst + (kv == 0 ? k_row_off(key) : v_row_off(key)) + u * 8) =
          *reinterpret_cast<const h8*>(src + (static_cast<size_t>(op.src0 + r) * heads + head) * D + u * 8);
    }
    return;
  }
  if (op.mode == kKvToTiles) {
    // every unit of the chunk's part is read (from rows) before any is
    // written, since both layouts share the same memory
    h8 val[4];
    int units[4], n = 0;
    for (int u = threadIdx.x; u < TILE / 8; u += 256) {
      const int L = u >> 6, lane = u & 63, half = lane >> 5, i = lane & 31;
      const int first = kv == 0 ? (L >> 3) * 32 + i : (L & 3) * 16 + half * 4;  // a key of the unit
      if (first < op.zero_lo || first >= op.zero_hi) continue;
      h8 x;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        int key, dim;
        if (kv == 0) {
          key = first;
          dim = (L & 7) * 16 + half * 8 + e;
        } else {
          key = first + (e & 3) + ((e >> 2) << 3);
          dim = (L >> 2) * 32 + i;
        }
        x[e] = key < op.zero_lo + op.n_rows ? dst[(kv == 0 ? k_row_off(key) : v_row_off(key)) + dim]
                                             : static_cast<_Float16>(0.0f);
      }
      val[n] = x;
      units[n++] = u;
    }
    __syncthreads();
    for (int j = 0; j < n; ++j) *reinterpret_cast<h8*>(dst + units[j] * 8) = val[j];
    return;
  }
  const int lo = op.dst_key0, hi = op.dst_key0 + op.n_rows;  // written keys [lo, hi)
  const int zlo = op.zero_lo, zhi = op.zero_hi;                // cleared keys [zlo, zhi)
  const bool whole = zlo == 0 && zhi == C;  // every unit rewritten, none read
  for (int u = threadIdx.x; u < TILE / 8; u += 256) {
    const int L = u >> 6, lane = u & 63, half = lane >> 5, i = lane & 31;
    if (!whole) {
      bool touched;
      if (kv == 0) {
        const int key = (L >> 3) * 32 + i;
        touched = (key >= lo && key < hi) || (key >= zlo && key < zhi);
      } else {
        const int k0 = (L & 3) * 16 + half * 4;  // keys k0..k0+3 and k0+8..k0+11
        touched = (k0 < hi && k0 + 4 > lo) || (k0 + 8 < hi && k0 + 12 > lo) ||
                  (k0 < zhi && k0 + 4 > zlo) || (k0 + 8 < zhi && k0 + 12 > zlo);
      }
      if (!touched) continue;
    }
    const h8 cur = whole ? h8{} : *reinterpret_cast<const h8*>(dst + u * 8);
    h8 val;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int key, dim;
      if (kv == 0) {
        key = (L >> 3) * 32 + i;
        dim = (L & 7) * 16 + half * 8 + e;
      } else {
        key = (L & 3) * 16 + half * 4 + (e & 3) + ((e >> 2) << 3);
        dim = (L >> 2) * 32 + i;
      }
      const int r = key - op.dst_key0;
      _Float16 x;
      if (r >= 0 && r < op.n_rows) {
        const int sr = op.src0 + r;
        if (op.from_pool) {
          const int t = sr / kTileKeys, key_in = sr % kTileKeys;
          x = pool[tile_base(t, head, heads, kv) + (kv == 0 ? k_off(key_in, dim) : v_off(key_in, dim))];
        } else {
          x = src[(static_cast<size_t>(sr) * heads + head) * D + dim];
        }
      } else {
        x = key >= zlo && key < zhi ? static_cast<_Float16>(0.0f) : cur[e];
      }
      val[e] = x;
    }
    *reinterpret_cast<h8*>(dst + u * 8) = val;
  }
}

}  // namespace

int launch_kv_write(void* pool, int heads, const KvOpBatch& batch, int n_ops, const void* k_src,
                    const void* v_src, int32_t* table, const TablePatches& patches, void* stream) {
  if (n_ops <= 0) return 0;
  dim3 grid(n_ops, heads, 2);
  hipLaunchKernelGGL(kv_write_kernel, grid, dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<_Float16*>(pool), heads, batch, static_cast<const _Float16*>(k_src),
                     static_cast<const _Float16*>(v_src), table, patches);
  return static_cast<int>(hipGetLastError());
}

}  // namespace chunkattn
