// Host-callable launchers of the gfx950 decode-step kernels.  Plain types only, so the
// C-ABI layer and the manager never see HIP device code.
#pragma once

#include <cstdint>

namespace chunkattn {

constexpr int kHeadDim = 128;
constexpr int kChunk = 64;
constexpr int kTileKeys = kChunk;  // keys per K/V tile read by the kernels

// Pool stride from one 64-key tile to the next, in fp16 elements: the K and
// V tile of every head, and of one head more when the head count is a power
// of two from 16 up (the extra head then costs at most 1/16 of the pool).  A
// tile of 32 heads would otherwise span exactly 1 MiB, so the same head's
// tiles in tiles that decoding has allocated 32 (or 64, ...) apart lie a
// power-of-two distance apart; on MI355X blocks streaming such tiles together
// run slower (the batch-32 decode step 57.5 against 55.0 us).
constexpr bool pool_pads_tiles(int heads) { return heads >= 16 && (heads & (heads - 1)) == 0; }
constexpr int64_t pool_tile_halves(int heads) {
  return static_cast<int64_t>(heads + (pool_pads_tiles(heads) ? 1 : 0)) * 2 * kTileKeys * kHeadDim;
}
constexpr int kCfInline = 8;   // chunk refs carried by a chunk-first unit record
constexpr int kSfInline = 4;   // chunk refs carried by a sequence-first task record
// Record fields (int32 index) saying that other blocks of the step read the
// same chunks, so the block reads them with loads that keep them cached.
constexpr int kCfReuseField = 6;
constexpr int kSfReuseField = 5;
// Sequence-first record field: index in the task of the chunk where the
// sequence ends (where a decoded token is appended), or -1.
constexpr int kSfAppendField = 6;
// Fill counts (at most 64) in the device table may carry, above bit 8, the
// epoch of the decode step that last grew them in the kernel; readers mask.
// Bit 7 marks a chunk stored row-major (chunks grown by appends: see
// tile_layout.h); it rides along with the count wherever the count goes.
constexpr int kFillBits = 8;
constexpr int kRowBit = 1 << 7;
constexpr int kFillMask = kRowBit - 1;
constexpr unsigned kEpochMask = (1u << (32 - kFillBits)) - 1;
constexpr int kDenseParts = 16; // most partials per sequence for the dense partial layout

// Arguments of one decode step.  All pointers are device addresses.
struct StepArgs {
  const void* pool;            // fp16 slots: [slot][head][K|V][64 x 128 tile]
  const void* q;               // fp16 [n_live][H][128], ascending seq id
  void* out;                   // fp16 [n_live][H][128]
  const int32_t* cf_units;     // 32 ints per unit (CfUnit)
  const int32_t* sf_tasks;     // 16 ints per task (SfTask)
  const int32_t* chunk_refs;   // (slot, n_valid) pairs
  const int32_t* dfs_qrow;     // caller row per DFS position
  const int32_t* seq_parts;    // (first, count) per DFS position
  const int32_t* part_list;    // partial ids
  float* part_o;               // [n_parts][H][128]
  float* part_ms;              // [n_parts][H][2]: running max (log2 units), sum
  unsigned* arrivals;          // [n_seq][H] partials written so far in a one-launch step (zero between launches)
  int heads;
  int dense_parts;             // > 0: sequence i's j-th partial is i * dense_parts + j (j < count)
  int part_stride;             // partial id step between rows of a chunk-first unit
  int n_cf_units;
  int n_sf_tasks;
  int n_seq;
  float scale_log2e;           // (1/sqrt(128)) * log2(e)
  // Decode step with in-kernel appends (null when not): row r of app_k /
  // app_v ([n_live][H][128] fp16) is the new token of the sequence at caller
  // row r; the block owning that sequence's last chunk writes it into the
  // pool, uses it, and stores the grown fill count tagged with app_epoch.
  const void* app_k;
  const void* app_v;
  unsigned app_epoch;          // 1 .. kEpochMask
  // Chunks of 32 tokens: chunk slot s is half s % 2 (keys 32 * (s % 2) ..
  // +32) of tile s / 2, and a chunk ref's slot field is s.
  int half_tiles;
  // One-launch step: polls a merge wave makes before it gives up and writes
  // NaN (0: the built-in bound, about 0.1 s).
  int max_polls;
  // Some chunk of the plan is stored row-major (kRowBit in its fill count):
  // the launch takes the kernel instance that reads both layouts.
  int row_chunks;
};

// Which blocks of the partials kernel to launch.
enum PartialsPart { kPartsBoth = 0, kPartsChunkFirst = 1, kPartsSequenceFirst = 2 };

// Each returns a hipError_t value (0 = success) from the launch.
// One grid with the chunk-first blocks first and the sequence-first blocks
// after them; `part` restricts the launch to one side.  With fuse_merge (and
// part == kPartsBoth) merge blocks close the grid and write out: the whole
// step in one launch, whose arrival counters are zero again when it ends.
int launch_partials(const StepArgs& a, int part, bool fuse_merge, void* stream);
int launch_merge(const StepArgs& a, void* stream);

// Device scratch for steps whose caller cannot allocate: a file-scope array
// of the kernels' module, one copy per device, held until the process ends.
// static_scratch() returns its device address on the current device (looked
// up once per device and kept) and that device's index; a hipError_t value.
constexpr size_t kStaticScratchBytes = size_t{16} << 20;  // CA_NOALLOC_SCRATCH_BYTES
constexpr int kMaxScratchDevices = 64;
int static_scratch(void** ptr, int* device);

}  // namespace chunkattn
