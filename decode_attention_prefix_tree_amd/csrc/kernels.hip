// gfx950 (CDNA4) kernels of the ChunkAttention decode step.
//
// Two-phase partition (paperlayer.ai summary of arXiv 2402.15220v4, section
// 3.2 and Figure 2): chunk-first blocks batch the queries of all sequences
// that share a chunk into a matrix and run both products on MFMA;
// sequence-first blocks stream each sequence's private chunks; both write
// partial results (o, m, s) that the merge combines by log-sum-exp
// (explainer 0h-n0.github.io/posts/paper-2402-15220, output combination
// formula; m is a running max, s and o are unnormalised).  Both phases share
// one grid; the merge is a second launch or, in the one-launch step, blocks
// at the end of the same grid.
//
// The chunk tile layout is described in tile_layout.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "kernels.h"
#include "tile_layout.h"

namespace chunkattn {

namespace {

// Blocks are handed to the 8 XCDs round robin; give each XCD a contiguous
// range of logical ids so work that reads the same chunk shares an L2.
__device__ __forceinline__ int xcd_remap(int b, int n) {
  int xcd = b & 7, local = b >> 3, q = n >> 3, r = n & 7;
  return xcd * q + min(xcd, r) + local;
}

// Cross-lane steps that need no address registers: DPP within quads and
// rows of 16, ds_swizzle across the two rows of a 32-lane half, and gfx950's
// v_permlane32_swap across the two halves of the wave.
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

__device__ __forceinline__ float swap16(float x) {  // lane i <- lane i^16, within 32
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
}

// x[i] + x[i^32] (or the max) on every lane: the swap leaves the low half's
// values in one result and the high half's in the other, on all 64 lanes.
__device__ __forceinline__ float sum_halves(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(p[0]) + __int_as_float(p[1]);
}
__device__ __forceinline__ float max_halves(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(p[0]), __int_as_float(p[1]));
}

// max over the 32 lanes of each half-wave (butterfly: once quads agree, the
// mirrors pair lanes of different groups)
__device__ __forceinline__ float wave_max32(float x) {
  x = fmaxf(x, dpp<kQuadXor1>(x));
  x = fmaxf(x, dpp<kQuadXor2>(x));
  x = fmaxf(x, dpp<kRowHalfMirror>(x));
  x = fmaxf(x, dpp<kRowMirror>(x));
  x = fmaxf(x, swap16(x));
  return x;
}

__device__ __forceinline__ float wave_sum64(float x) {
  x = sum_halves(x);
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  x += dpp<kRowHalfMirror>(x);
  x += dpp<kRowMirror>(x);
  x += swap16(x);
  return x;
}

// A chunk read once per step streams with nontemporal loads, which do not
// keep its lines in the caches and let HBM reads run closer to peak.  Blocks
// whose chunks other blocks of the step read too (a shared run of more than
// 32 rows, or shared chunks without the chunk-first phase) use ordinary
// loads, so the other readers find the lines in L2 or the Infinity Cache.
template <bool kNT>
__device__ __forceinline__ h8 ld_tile(const _Float16* p) {
  if constexpr (kNT) return __builtin_nontemporal_load(reinterpret_cast<const h8*>(p));
  return *reinterpret_cast<const h8*>(p);
}

// A chunk-table entry read by a decode step that also grows fill counts in
// the table (kAppend: its blocks store into the table, so the compiler would
// read every entry with a vector load waited for at once).  Through the
// constant address space the load is a scalar one and leaves the vector
// memory counter to the tile loads.  Every entry holds its value for the
// whole step except the growing chunks' fill counts, which a block may read
// before or after another head's block tags them: both give the same key
// (see the epoch test of the sequence-first block).
template <bool kScalar>
__device__ __forceinline__ int ld_table(const int* p) {
  if constexpr (kScalar) return *(const __attribute__((address_space(4))) int*)p;
  return *p;
}

__device__ __forceinline__ h2 lo2(h8 v, int j) {
  switch (j) {
    case 0: return __builtin_shufflevector(v, v, 0, 1);
    case 1: return __builtin_shufflevector(v, v, 2, 3);
    case 2: return __builtin_shufflevector(v, v, 4, 5);
    default: return __builtin_shufflevector(v, v, 6, 7);
  }
}

// Step-local communication between blocks (the one-launch step).  Partials
// are written with agent-scope relaxed atomic stores and read back with
// agent-scope atomic loads: on gfx950 both are device-scope accesses (sc1)
// that write through and read past the XCD's L2, so they are coherent across
// the XCDs by themselves.  A writer waits for its stores to be acknowledged
// (s_waitcnt vmcnt(0), then its block's barrier) before it counts its
// arrival; a merger issues its partial loads only after its poll has
// returned the full count.  The memory model's own release/acquire at agent
// scope would add a write-back of the whole L2 to every arrival and an
// invalidate of the whole L2 to every merge: measured, that doubles the
// multi-branch step (201 -> 420 us), so the ordering rests on these two
// hardware facts instead.
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---------------------------------------------------------------------------
// Merge of one (sequence, head) by one wave: folds the sequence's partials in
// the fixed order of its list (shared runs root first, then private tasks):
// M = max m_j, o = sum e^{m_j - M} o_j, s = sum e^{m_j - M} s_j,
// out = o / s in fp16.  Lane j fetches partial j's (m, s) and all lanes then
// fetch o rows eight partials at a time, so the loads of a round are in
// flight together; lane l owns dims 2l, 2l+1.  Partials are taken 64 at a
// time; a later round rescales what the earlier ones summed.
template <bool kCoherent>
__device__ __forceinline__ float ld(const float* p) {
  if constexpr (kCoherent) return load_agent(p);
  return *p;
}

template <bool kCoherent>
__device__ __forceinline__ void merge_one(const StepArgs& a, int pos, int head, int lane) {
  const int H = a.heads;
  const int first = a.seq_parts[2 * pos], cnt = a.seq_parts[2 * pos + 1];
  float s = 0.f, o0 = 0.f, o1 = 0.f, M = -INFINITY;
  for (int j0 = 0; j0 < cnt; j0 += 64) {
    // lane j holds partial j0+j: its id, running max and sum
    const int n = min(64, cnt - j0);
    int my_pid = 0;
    float my_m = -INFINITY, my_s = 0.f;
    if (lane < n) {
      my_pid = a.part_list[first + j0 + lane];
      const size_t pid = static_cast<size_t>(my_pid) * H + head;
      my_m = ld<kCoherent>(a.part_ms + pid * 2);
      my_s = ld<kCoherent>(a.part_ms + pid * 2 + 1);
    }
    float Mr = max_halves(my_m);
    Mr = fmaxf(M, wave_max32(Mr));
    // rescale what earlier rounds accumulated (only with more than 64 partials)
    const float r = M == -INFINITY ? 0.f : exp2f(M - Mr);
    o0 *= r;
    o1 *= r;
    s *= r;
    M = Mr;
    const float my_w = lane < n ? exp2f(my_m - M) : 0.f;
    s += wave_sum64(my_w * my_s);
    // the o rows of all partials are independent loads: issue 8 at a time
    for (int j = 0; j < n; j += 8) {
      float2 ov[8];
      float wv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int jj = min(j + u, n - 1);
        wv[u] = j + u < n ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), jj)) : 0.f;
        const size_t pid = static_cast<size_t>(__builtin_amdgcn_readlane(my_pid, jj)) * H + head;
        const float* src = a.part_o + pid * D + 2 * lane;
        if constexpr (kCoherent) {
          ov[u].x = load_agent(src);
          ov[u].y = load_agent(src + 1);
        } else {
          ov[u] = *reinterpret_cast<const float2*>(src);
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        o0 = fmaf(wv[u], ov[u].x, o0);
        o1 = fmaf(wv[u], ov[u].y, o1);
      }
    }
  }
  const float inv = 1.0f / s;
  const int qrow = a.dfs_qrow[pos];
  _Float16* out = static_cast<_Float16*>(a.out) + (static_cast<size_t>(qrow) * H + head) * D + 2 * lane;
  h2 res = {static_cast<_Float16>(o0 * inv), static_cast<_Float16>(o1 * inv)};
  *reinterpret_cast<h2*>(out) = res;
}

// One more partial of (pos, head) is written.  Each counter is zero when a
// launch starts (the table upload clears them, and every merge returns its
// counter to zero): the producers of a (sequence, head) add one each, its
// merge waits for the count and then takes it off again.
__device__ __forceinline__ void arrive(const StepArgs& a, int pos, int head) {
  __hip_atomic_fetch_add(a.arrivals + pos * a.heads + head, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge of one (sequence, head) with the dense partial layout: partial j of
// the sequence at DFS position pos is pos * P + j, so every load of the merge
// (all (m, s) and o rows) is issued at once, together with the caller's
// loads of cnt and qrow, and the merge costs one round trip to memory.
// Slots past the sequence's count are loaded but never used.  Same fold as
// merge_one: M = max m_j, w_j = e^{m_j - M}, s = sum w_j s_j (wave sum),
// o = sum w_j o_j in list order, out = o / s in fp16.
template <bool kCoherent>
__device__ __forceinline__ void merge_dense(const StepArgs& a, int pos, int head, int lane, int cnt, int qrow) {
  const int H = a.heads, P = a.dense_parts;
  float my_m = -INFINITY, my_s = 0.f;
  if (lane < P) {
    const size_t pid = static_cast<size_t>(pos * P + lane) * H + head;
    my_m = ld<kCoherent>(a.part_ms + pid * 2);
    my_s = ld<kCoherent>(a.part_ms + pid * 2 + 1);
  }
  float2 ov[kDenseParts];
#pragma unroll
  for (int j = 0; j < kDenseParts; ++j)
    if (j < P) {
      const float* src = a.part_o + (static_cast<size_t>(pos * P + j) * H + head) * D + 2 * lane;
      if constexpr (kCoherent) {
        ov[j].x = load_agent(src);
        ov[j].y = load_agent(src + 1);
      } else {
        ov[j] = *reinterpret_cast<const float2*>(src);
      }
    }
  if (lane >= cnt) {
    my_m = -INFINITY;
    my_s = 0.f;
  }
  const float M = wave_max32(max_halves(my_m));
  const float my_w = lane < cnt ? exp2f(my_m - M) : 0.f;
  const float s = wave_sum64(my_w * my_s);
  float o0 = 0.f, o1 = 0.f;
#pragma unroll
  for (int j = 0; j < kDenseParts; ++j) {
    if (j < cnt) {
      const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), j));
      o0 = fmaf(w, ov[j].x, o0);
      o1 = fmaf(w, ov[j].y, o1);
    }
  }
  const float inv = 1.0f / s;
  _Float16* out = static_cast<_Float16*>(a.out) + (static_cast<size_t>(qrow) * H + head) * D + 2 * lane;
  h2 res = {static_cast<_Float16>(o0 * inv), static_cast<_Float16>(o1 * inv)};
  *reinterpret_cast<h2*>(out) = res;
}

// Polls of a merge wave waiting for the partials of its (sequence, head):
// about 0.1 s in all.  The wait ends long before that (a merge block only
// waits for blocks before it in the grid, which never wait themselves); if
// it did not, the wave writes NaN rather than read incomplete partials.
constexpr int kMaxPolls = 1 << 20;

// Merge blocks close the one-launch step.  They come after every partials
// block in the grid, so they are dispatched last, into the step's tail, and
// only ever wait for blocks dispatched before them.  Wave w of merge block mb
// merges item mb*4 + w = (DFS position, head), once the item's counter has
// reached the sequence's partial count; then it subtracts that count, so the
// counter is zero again when every producer has arrived.  Nothing carries
// over from one launch to the next, so a step can be captured in a graph and
// replayed.  A wave that gives up subtracts the count too: producers always
// arrive, and the late ones bring the counter back to zero by the end of the
// launch.
__device__ __forceinline__ void merge_block(const StepArgs& a, int mb) {
  const int item = mb * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (item >= a.n_seq * a.heads) return;
  const int pos = item / a.heads, head = item - pos * a.heads;
  const int cnt = a.seq_parts[2 * pos + 1];
  const int qrow = a.dfs_qrow[pos];
  unsigned* ctr = a.arrivals + item;
  const unsigned target = static_cast<unsigned>(cnt);
  // the first poll goes out with the loads of cnt and qrow
  unsigned seen = __builtin_amdgcn_readfirstlane(__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  bool ok = true;
  const int limit = a.max_polls > 0 ? a.max_polls : kMaxPolls;
  for (int tries = 0; seen < target; ++tries) {
    if (tries == limit) {
      ok = false;
      break;
    }
    __builtin_amdgcn_s_sleep(2);
    seen = __builtin_amdgcn_readfirstlane(__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  }
  // keep the partial loads after the poll (the compiler must not hoist them)
  asm volatile("" ::: "memory");
  if (!ok) {
    _Float16* out = static_cast<_Float16*>(a.out) + (static_cast<size_t>(qrow) * a.heads + head) * D + 2 * lane;
    *reinterpret_cast<h2*>(out) = h2{static_cast<_Float16>(NAN), static_cast<_Float16>(NAN)};
  } else if (a.dense_parts > 0) {
    merge_dense<true>(a, pos, head, lane, cnt, qrow);
  } else {
    merge_one<true>(a, pos, head, lane);
  }
  if (lane == 0) __hip_atomic_fetch_sub(ctr, target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Partials.  One grid holds both phases: blocks [0, n_cf) are chunk-first
// blocks and come first so they start first, the rest are sequence-first
// blocks, so the two phases run at the same time with no launch between
// them.  256 threads (4 waves) per block; a block owns one task and its
// waves take the task's chunks w, w+4, ...  Both paths fit 168 VGPRs and
// share one 42.5 KB LDS scratch, so three blocks share a CU.

constexpr int kOStride = 132;                        // padded row stride of wave states
constexpr int kQBytes = 32 * D * 2;                  // Q block in operand order, fp16
constexpr int kStateFloats = 32 * kOStride + 64;     // one wave state: O rows, then (m, l)
constexpr int kSmemBytes = kQBytes + 2 * kStateFloats * 4;
// the sequence-first layout of the same scratch
constexpr int kSfP = D * 2;                // after the query row (fp16)
constexpr int kSfO = kSfP + 4 * 64 * 4;    // after the probability rows
constexpr int kSfM = kSfO + 4 * D * 4;     // after the wave states' o rows
constexpr int kSfA = kSfM + 8 * 4;         // after the wave states' (m, l): an appended K and V row
static_assert(kSfA + 2 * D * 2 <= kSmemBytes, "sequence-first scratch fits the block's LDS");

__device__ __forceinline__ float weight(float m, float M) {
  // e^(m - M) in base 2; an empty state (m = -inf) weighs 0 even when M = -inf
  return m == -INFINITY ? 0.f : exp2f(m - M);
}

// Chunk-first: unit = (run of shared chunks, 32-row block), one head.
// Lane (half, i) owns query row i.  Per 32-key half of a chunk:
// S^T[32 keys x 32 rows] = K Q^T (8 MFMA; Q^T comes from LDS), online softmax
// along keys (the lane holds 16 keys of its row, its twin lane the other 16),
// O^T[128 x 32] += V^T P^T (8 MFMA).  P^T needs no exchange: the V tile
// stores keys in the order the S^T accumulators hold them.
template <bool kFuse, bool kNT, bool kHalf>
__device__ __forceinline__ void chunk_first_block(const StepArgs& a, int logical, char* smem) {
  const int unit = logical % a.n_cf_units, head = logical / a.n_cf_units;
  const int* u = a.cf_units + unit * 32;
  const int chunk_begin = u[0], n_chunks = u[1], row_begin = u[2], n_rows = u[3], part_base = u[4];
  const int qrow_base = u[5];  // >= 0: the rows' caller rows are qrow_base + row
  // wave index in an SGPR: chunk lookups and tile bases stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, half = lane >> 5, i = lane & 31;
  const int H = a.heads;
  const _Float16* pool = static_cast<const _Float16*>(a.pool);

  // Q rows of the block into LDS in B-operand order: piece (kk, lane) at
  // (kk*64 + lane)*8 halves holds Q[row lane%32][16kk + 8(lane/32) .. +8].
  _Float16* q_lds = reinterpret_cast<_Float16*>(smem);
  for (int p = threadIdx.x; p < 32 * 16; p += 256) {
    const int row = p >> 4, c16 = p & 15, kk = c16 >> 1, hf = c16 & 1;
    h8 v = h8{};
    if (row < n_rows) {
      const int qrow = qrow_base >= 0 ? qrow_base + row : a.dfs_qrow[row_begin + row];
      v = *reinterpret_cast<const h8*>(static_cast<const _Float16*>(a.q) +
                                       (static_cast<size_t>(qrow) * H + head) * D + c16 * 8);
    }
    *reinterpret_cast<h8*>(q_lds + ((kk * 64 + hf * 32 + row) * 8)) = v;
  }
  __syncthreads();

  float m = -INFINITY, l = 0.f;
  f16v acc[4];

  if (!kHalf && n_chunks <= 4) {
    // At most one chunk per wave: no accumulator has to survive another
    // chunk's loads, so the wave loads its whole chunk at once (32 KiB in
    // flight, one round trip, like a sequence-first wave): K 64 VGPRs, V 64,
    // one half's scores 16 while the first half's K is still live.
    if (wave < n_chunks) {
      const int slot = u[8 + wave], nvalid = u[16 + wave] & kFillMask;  // inline: wave < 4 <= kCfInline
      const _Float16* kt = pool + tile_base(slot, head, H, 0);
      const _Float16* vt = kt + TILE;
      h8 kr[16], vr[16];
#pragma unroll
      for (int L = 0; L < 16; ++L) kr[L] = ld_tile<kNT>(kt + (L * 64 + lane) * 8);
#pragma unroll
      for (int L = 0; L < 16; ++L) vr[L] = ld_tile<kNT>(vt + (L * 64 + lane) * 8);
      // keep every load ahead of the first product (the scheduler would
      // otherwise trade them for registers, one load per MFMA)
      __builtin_amdgcn_sched_barrier(0);
      // One 32-key half after the other, each reading its Q operands from
      // LDS afresh: holding all eight across both halves would not fit.
      f16v sc[2];
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        sc[jb] = f16v{};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const h8 qb = *reinterpret_cast<const h8*>(q_lds + (kk * 64 + lane) * 8);
          sc[jb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kr[jb * 8 + kk], qb, sc[jb], 0, 0, 0);
        }
        if (jb == 0) {
          asm volatile("" ::: "memory");
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // sc[jb][r] is key 32jb + 8(r/4) + 4half + r%4 of row i
      float mx = -INFINITY;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * jb + 8 * (r >> 2) + 4 * half + (r & 3);
          const float x = key < nvalid ? sc[jb][r] * a.scale_log2e : -INFINITY;
          sc[jb][r] = x;
          mx = fmaxf(mx, x);
        }
      m = max_halves(mx);  // finite: key 0 of a chunk is always filled
      h8 pb[2][2];
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = exp2f(sc[jb][r] - m);
          l += pr;
          pb[jb][r >> 3][r & 7] = static_cast<_Float16>(pr);
        }
      // the accumulators come to life only here, after the tile loads
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vr[nb * 4], pb[0][0], f16v{}, 0, 0, 0);
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vr[nb * 4 + 1], pb[0][1], acc[nb], 0, 0, 0);
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vr[nb * 4 + 2], pb[1][0], acc[nb], 0, 0, 0);
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vr[nb * 4 + 3], pb[1][1], acc[nb], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[nb] = f16v{};
    }
  } else {
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) acc[nb] = f16v{};
  for (int c = wave; c < n_chunks; c += 4) {
    const int slot = c < kCfInline ? u[8 + c] : a.chunk_refs[2 * (chunk_begin + c)];
    const int nvalid = (c < kCfInline ? u[16 + c] : a.chunk_refs[2 * (chunk_begin + c) + 1]) & kFillMask;
    // a 32-token chunk is one half of its tile: the tile pointers move to
    // that half (K blocks 8h.., V blocks 4nb + 2h ..) and the loop below
    // runs once, over keys 0..31 of the half
    const int tile = kHalf ? slot >> 1 : slot, hh = kHalf ? slot & 1 : 0;
    const _Float16* kt = pool + tile_base(tile, head, H, 0) + hh * 8 * 512;
    const _Float16* vt = pool + tile_base(tile, head, H, 1) + hh * 2 * 512;
    // The halves stay a loop: unrolled, the second half's loads would be
    // hoisted over the first half's MFMAs and the block would not fit three
    // waves per SIMD.
#pragma unroll 1
    for (int jb = 0; jb < (kHalf ? 1 : 2); ++jb) {
      h8 kr[8], vr[8];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) kr[kk] = ld_tile<kNT>(kt + ((jb * 8 + kk) * 64 + lane) * 8);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          vr[nb * 2 + t] = ld_tile<kNT>(vt + ((nb * 4 + 2 * jb + t) * 64 + lane) * 8);
      // all 16 loads of the half go out before its first product (left
      // alone, the scheduler issues K one load per MFMA and V only after the
      // softmax: two or more dependent round trips per half instead of one)
      __builtin_amdgcn_sched_barrier(0);
      f16v sc = f16v{};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const h8 qb = *reinterpret_cast<const h8*>(q_lds + (kk * 64 + lane) * 8);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(kr[kk], qb, sc, 0, 0, 0);
      }
      // sc[r] is key 32jb + 8(r/4) + 4half + r%4 of row i
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * jb + 8 * (r >> 2) + 4 * half + (r & 3);
        const float x = key < nvalid ? sc[r] * a.scale_log2e : -INFINITY;
        sc[r] = x;
        mx = fmaxf(mx, x);
      }
      mx = max_halves(mx);
      const float mnew = fmaxf(m, mx);
      if (mnew == -INFINITY) continue;  // every key of this half is past the fill
      const float alpha = weight(m, mnew);
      float psum = 0.f;
      h8 pb[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(sc[r] - mnew);
        psum += p;
        pb[r >> 3][r & 7] = static_cast<_Float16>(p);
      }
      l = l * alpha + psum;
      m = mnew;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        acc[nb] *= alpha;
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vr[nb * 2 + t], pb[t], acc[nb], 0, 0, 0);
      }
    }
  }
  }
  l = sum_halves(l);

  // Pairwise merge of the four wave states: (w0 + w2) + (w1 + w3).
  float* st = reinterpret_cast<float*>(smem + kQBytes);
  auto put = [&](int slotw) {
    float* o = st + slotw * kStateFloats;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f4 v = {acc[nb][4 * g + 0], acc[nb][4 * g + 1], acc[nb][4 * g + 2], acc[nb][4 * g + 3]};
        *reinterpret_cast<f4*>(o + i * kOStride + 32 * nb + 8 * g + 4 * half) = v;
      }
    if (half == 0) {
      o[32 * kOStride + 2 * i] = m;
      o[32 * kOStride + 2 * i + 1] = l;
    }
  };
  auto take = [&](int slotw) {
    const float* o = st + slotw * kStateFloats;
    const float mb = o[32 * kOStride + 2 * i], lb = o[32 * kOStride + 2 * i + 1];
    const float M = fmaxf(m, mb);
    const float wa = weight(m, M), wb = weight(mb, M);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f4 v = *reinterpret_cast<const f4*>(o + i * kOStride + 32 * nb + 8 * g + 4 * half);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[nb][4 * g + e] = wa * acc[nb][4 * g + e] + wb * v[e];
      }
    m = M;
    l = wa * l + wb * lb;
  };
  if (wave >= 2) put(wave - 2);
  __syncthreads();
  if (wave < 2) take(wave);
  __syncthreads();
  if (wave == 1) put(0);
  __syncthreads();
  if constexpr (kFuse) {
    // The partials go out coherently (another block merges them), and a
    // coherent store writes through: wave 0 puts the final state into LDS row
    // by row, then all four waves store consecutive words, so every store
    // instruction writes two whole 512-byte rows.
    if (wave == 0) {
      take(0);
      put(0);
    }
    __syncthreads();
    const float* o = st;
#pragma unroll 4
    for (int k = 0; k < 32 * D / 256; ++k) {
      const int idx = k * 256 + threadIdx.x, row = idx / D, col = idx % D;
      if (row < n_rows)
        store_agent(a.part_o + (static_cast<size_t>(part_base + row * a.part_stride) * H + head) * D + col,
                    o[row * kOStride + col]);
    }
    if (threadIdx.x < n_rows) {
      const size_t pid = static_cast<size_t>(part_base + threadIdx.x * a.part_stride) * H + head;
      store_agent(a.part_ms + pid * 2 + 0, o[32 * kOStride + 2 * threadIdx.x]);
      store_agent(a.part_ms + pid * 2 + 1, o[32 * kOStride + 2 * threadIdx.x + 1]);
    }
    wait_stores();
    __syncthreads();  // every thread's stores have completed
    if (threadIdx.x < n_rows) arrive(a, row_begin + threadIdx.x, head);
    return;
  }
  if (wave != 0) return;
  take(0);
  if (i < n_rows) {
    const size_t pid = static_cast<size_t>(part_base + i * a.part_stride) * H + head;
    float* po = a.part_o + pid * D;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f4 v = {acc[nb][4 * g + 0], acc[nb][4 * g + 1], acc[nb][4 * g + 2], acc[nb][4 * g + 3]};
        *reinterpret_cast<f4*>(po + 32 * nb + 8 * g + 4 * half) = v;
      }
    if (half == 0) {
      a.part_ms[pid * 2 + 0] = m;
      a.part_ms[pid * 2 + 1] = l;
    }
  }
}

// Sequence-first: task = some private chunks of one sequence, one head.
// Lane (half, i): for K it holds dims [16kk + 8half, +8) of keys i and 32+i,
// so a score needs one exchange with the twin lane; for V it holds dim
// 32nb + i at 8 keys per load and reads the matching probabilities from a
// 64-entry LDS row of its wave.  Three waves per SIMD keep about 384 KiB of
// loads in flight per CU.  kAppend: a decode step whose blocks also write the
// new tokens; the attend-only kernel has no stores into the pool or the
// table, so its table reads stay scalar loads.  kRow: some chunks are stored
// row-major (tile_layout.h); a wave reads such a chunk by rows: lane group
// g = lane / 16 takes rows 4j + g, each lane 8 dims of them (every load is
// 1 KiB of contiguous rows), scores are summed across the group's 16 lanes,
// and the chunk's output rows join the tile-layout accumulators through LDS.
template <bool kFuse, bool kNT, bool kAppend, bool kHalf, bool kRow>
__device__ __forceinline__ void sequence_first_block(const StepArgs& a, int logical, char* smem) {
  // heads vary fastest: blocks that run together read neighbouring 32 KiB
  // tiles of the same slots, which keeps HBM accesses close to sequential
  const int task = logical / a.heads, head = logical % a.heads;
  const int* t = a.sf_tasks + task * 16;
  const int chunk_begin = ld_table<kAppend>(t), n_chunks = ld_table<kAppend>(t + 1),
            dfs_pos = ld_table<kAppend>(t + 2), part_id = ld_table<kAppend>(t + 3), qrow = ld_table<kAppend>(t + 4);
  // wave index in an SGPR: chunk lookups and tile bases stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, half = lane >> 5, i = lane & 31;
  const int H = a.heads;
  const _Float16* pool = static_cast<const _Float16*>(a.pool);

  // The query row is the same for the four waves: keep it in LDS (256 B)
  // rather than in 32 VGPRs of every lane.
  // LDS (the block's scratch, shared with the chunk-first layout): query row,
  // one probability row per wave, the four wave states
  _Float16* q_lds = reinterpret_cast<_Float16*>(smem);
  float(*p_lds)[64] = reinterpret_cast<float(*)[64]>(smem + kSfP);
  float(*w_o)[D] = reinterpret_cast<float(*)[D]>(smem + kSfO);
  float* w_m = reinterpret_cast<float*>(smem + kSfM);
  float* w_l = w_m + 4;
  _Float16* new_lds = reinterpret_cast<_Float16*>(smem + kSfA);  // appended token: K row, then V row
  // In a decode step with in-kernel appends, the chunk (index in the task)
  // that takes this sequence's new token.
  const int append_at = kAppend ? ld_table<kAppend>(t + kSfAppendField) : -1;
  if (threadIdx.x < D / 8) {
    const _Float16* qp = static_cast<const _Float16*>(a.q) + (static_cast<size_t>(qrow) * H + head) * D;
    *reinterpret_cast<h8*>(q_lds + threadIdx.x * 8) = *reinterpret_cast<const h8*>(qp + threadIdx.x * 8);
  } else if (append_at >= 0 && threadIdx.x < 3 * D / 8) {
    const int kv = threadIdx.x / (D / 8) - 1, piece = threadIdx.x % (D / 8);
    const _Float16* src = static_cast<const _Float16*>(kv ? a.app_v : a.app_k) +
                          (static_cast<size_t>(qrow) * H + head) * D + piece * 8;
    *reinterpret_cast<h8*>(new_lds + kv * D + piece * 8) = *reinterpret_cast<const h8*>(src);
  }
  __syncthreads();

  float m = -INFINITY, l = 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};

  // The appended token goes to key p of chunk append_at, the chunk's fill
  // before this step: the blocks of the other heads of this task share the
  // fill count, and one that ran first may already have stored p + 1 tagged
  // with this step's epoch.  The wave that will read the chunk writes the
  // token into its tiles before its loop starts, with the very lanes that
  // later load those 16-byte units, so its loads read it back in program
  // order; the fill count the loop uses is p + 1.
  int append_fill = 0;
  if (kAppend && append_at >= 0) {
    const int ac = append_at;
    const int fill = ld_table<kAppend>(ac < kSfInline ? t + 12 + ac : a.chunk_refs + 2 * (chunk_begin + ac) + 1);
    int p = (static_cast<unsigned>(fill) >> kFillBits) == a.app_epoch ? (fill & kFillMask) - 1 : fill & kFillMask;
    append_fill = p + 1;
    if ((ac & 3) == wave) {
      const int cslot = ld_table<kAppend>(ac < kSfInline ? t + 8 + ac : a.chunk_refs + 2 * (chunk_begin + ac));
      // key p of a 32-token chunk is key 32 * (slot % 2) + p of its tile
      const int slot = kHalf ? cslot >> 1 : cslot;
      _Float16* kw = const_cast<_Float16*>(pool) + tile_base(slot, head, H, 0);
      _Float16* vw = kw + TILE;
      if (kRow && (fill & kRowBit)) {
        // row layout: one K row and one V row, written by the lanes that
        // read row p in the loop below (group p % 4, 16 bytes each)
        const int key = (kHalf ? (cslot & 1) * 32 : 0) + p;
        if ((lane >> 4) == (p & 3)) {
          const int sub = lane & 15;
          *reinterpret_cast<h8*>(kw + k_row_off(key) + sub * 8) = *reinterpret_cast<const h8*>(new_lds + sub * 8);
          *reinterpret_cast<h8*>(vw + v_row_off(key) + sub * 8) =
              *reinterpret_cast<const h8*>(new_lds + D + sub * 8);
        }
      } else {
        if (kHalf) p += (cslot & 1) * 32;
        // K: load (p/32)*8 + j, lanes (half, p%32): dims 16j + 8half .. +8
        if (i == (p & 31)) {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            *reinterpret_cast<h8*>(kw + (((p >> 5) * 8 + j) * 64 + lane) * 8) =
                *reinterpret_cast<const h8*>(new_lds + j * 16 + half * 8);
        }
        // V: load 4nb + p/16, lanes (half (p/4)%2, i): dim 32nb + i, key p at element e
        if (half == ((p >> 2) & 1)) {
          const int e = (p & 3) | (((p >> 3) & 1) << 2);
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) vw[((nb * 4 + (p >> 4)) * 64 + lane) * 8 + e] = new_lds[D + nb * 32 + i];
        }
      }
      if (lane == 0) {
        const int tagged = append_fill | (fill & kRowBit) | static_cast<int>(a.app_epoch << kFillBits);
        const_cast<int32_t*>(a.chunk_refs)[2 * (chunk_begin + ac) + 1] = tagged;
        if (ac < kSfInline) const_cast<int*>(t)[12 + ac] = tagged;
      }
    }
  }

  for (int c = wave; c < n_chunks; c += 4) {
    const int slot = ld_table<kAppend>(c < kSfInline ? t + 8 + c : a.chunk_refs + 2 * (chunk_begin + c));
    const int fill = ld_table<kAppend>(c < kSfInline ? t + 12 + c : a.chunk_refs + 2 * (chunk_begin + c) + 1);
    int nvalid = fill & kFillMask;
    // a 32-token chunk is one half of its tile: its K blocks 8h .. 8h+7 and
    // V blocks 4nb + 2h, +1 land where keys 0..31 of a whole tile would
    const int tile = kHalf ? slot >> 1 : slot, hh = kHalf ? slot & 1 : 0;
    const _Float16* kt = pool + tile_base(tile, head, H, 0) + hh * 8 * 512;
    const _Float16* vt = pool + tile_base(tile, head, H, 1) + hh * 2 * 512;
    if (kAppend && c == append_at) nvalid = append_fill;
    if (kRow && (fill & kRowBit)) {
      // Row layout.  Loads j of K and V bring rows 4j .. 4j+3 of the chunk
      // (1 KiB each); a load past the fill reads rows 0..3 again (its rows
      // get zero weight).  Lane (g, sub) holds dims 8 sub .. 8 sub + 7 of row
      // 4j + g.
      constexpr int kJ = kHalf ? 8 : 16;
      const int g = lane >> 4, sub = lane & 15;
      const int key0 = kHalf ? hh * 32 : 0;
      const _Float16* kr = pool + tile_base(tile, head, H, 0) + sub * 8;
      const _Float16* vr = pool + tile_base(tile, head, H, 1) + sub * 8;
      h8 kq[kJ], vq[kJ];
#pragma unroll
      for (int j = 0; j < kJ; ++j) {
        const int r = key0 + (4 * j < nvalid ? 4 * j : 0) + g;
        kq[j] = ld_tile<kNT>(kr + k_row_off(r));
        vq[j] = ld_tile<kNT>(vr + v_row_off(r));
      }
      const h8 qv = *reinterpret_cast<const h8*>(q_lds + sub * 8);
      float x[kJ];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < kJ; ++j) {
        float d = 0.f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) d = __builtin_amdgcn_fdot2(lo2(kq[j], jj), lo2(qv, jj), d, false);
        // the row's 16 pieces are in the 16 lanes of the group
        d += dpp<kQuadXor1>(d);
        d += dpp<kQuadXor2>(d);
        d += dpp<kRowHalfMirror>(d);
        d += dpp<kRowMirror>(d);
        x[j] = 4 * j + g < nvalid ? d * a.scale_log2e : -INFINITY;
        mx = fmaxf(mx, x[j]);
      }
      mx = max_halves(fmaxf(mx, swap16(mx)));
      const float mnew = fmaxf(m, mx);  // finite: row 0 of a chunk is always filled
      const float alpha = exp2f(m - mnew);
      float psum = 0.f;
      float o8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < kJ; ++j) {
        const float pr = exp2f(x[j] - mnew);
        psum += pr;
        // rows past the fill hold anything: they add nothing
        const bool live = 4 * j + g < nvalid;
#pragma unroll
        for (int e = 0; e < 8; ++e) o8[e] = fmaf(pr, live ? static_cast<float>(vq[j][e]) : 0.f, o8[e]);
      }
      // each row's weight is in all 16 lanes of its group: count it once
      l = l * alpha + (sub == 0 ? psum : 0.f);
      m = mnew;
#pragma unroll
      for (int e = 0; e < 8; ++e) o8[e] = sum_halves(o8[e] + swap16(o8[e]));
      // into the tile-layout accumulators (dim 32 nb + i at lane (half, i))
      // through the wave's output row in LDS; half 1 adds nothing
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[nb] *= alpha;
      if (lane < 16) {
        *reinterpret_cast<f4*>(&w_o[wave][8 * sub]) = f4{o8[0], o8[1], o8[2], o8[3]};
        *reinterpret_cast<f4*>(&w_o[wave][8 * sub + 4]) = f4{o8[4], o8[5], o8[6], o8[7]};
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (half == 0) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[nb] += w_o[wave][32 * nb + i];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      continue;
    }
    // Keys past the fill get zero weight, so the tile blocks that hold only
    // such keys are not fetched from memory: a K load block covers 32 keys,
    // a V block 16, and a block wholly past the fill reads the chunk's first
    // block of its row again (already on its way: a cache hit).  Its finite
    // values meet zero probabilities, so the result is unchanged.
    // (The choice is one wave-uniform base per 32-key K half and per 16-key
    // V group, so every load keeps its immediate offset.)
    const _Float16* kb[2] = {kt, nvalid > 32 ? kt + 8 * 512 : kt};
    const _Float16* vb[4] = {vt, nvalid > 16 ? vt + 512 : vt, nvalid > 32 ? vt + 2 * 512 : vt,
                             nvalid > 48 ? vt + 3 * 512 : vt};
    h8 ka[16], va[16];
#pragma unroll
    for (int L = 0; L < (kHalf ? 8 : 16); ++L) ka[L] = ld_tile<kNT>(kb[L >> 3] + ((L & 7) * 64 + lane) * 8);
#pragma unroll
    for (int L = 0; L < 16; ++L)
      if (!kHalf || (L & 3) < 2) va[L] = ld_tile<kNT>(vb[L & 3] + ((L & ~3) * 64 + lane) * 8);

    float d0 = 0.f, d1 = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const h8 qv = *reinterpret_cast<const h8*>(q_lds + kk * 16 + half * 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        d0 = __builtin_amdgcn_fdot2(lo2(ka[kk], j), lo2(qv, j), d0, false);
        if (!kHalf) d1 = __builtin_amdgcn_fdot2(lo2(ka[8 + kk], j), lo2(qv, j), d1, false);
      }
    }
    d0 = sum_halves(d0);
    if (!kHalf) d1 = sum_halves(d1);
    const float x0 = i < nvalid ? d0 * a.scale_log2e : -INFINITY;
    const float x1 = !kHalf && i + 32 < nvalid ? d1 * a.scale_log2e : -INFINITY;
    const float mx = wave_max32(fmaxf(x0, x1));
    const float mnew = fmaxf(m, mx);  // finite: key 0 of a chunk is always filled
    const float alpha = exp2f(m - mnew);
    const float p0 = exp2f(x0 - mnew), p1 = exp2f(x1 - mnew);
    l = l * alpha + (half == 0 ? p0 + p1 : 0.f);
    m = mnew;
    if (half == 0) {
      p_lds[wave][i] = p0;
      p_lds[wave][32 + i] = p1;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[nb] *= alpha;
#pragma unroll
    for (int s = 0; s < (kHalf ? 2 : 4); ++s) {
      const f4 pa = *reinterpret_cast<const f4*>(&p_lds[wave][16 * s + 4 * half]);
      const f4 pc = *reinterpret_cast<const f4*>(&p_lds[wave][16 * s + 8 + 4 * half]);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const h8 v = va[nb * 4 + s];
        float x = acc[nb];
        x = fmaf(pa[0], static_cast<float>(v[0]), x);
        x = fmaf(pa[1], static_cast<float>(v[1]), x);
        x = fmaf(pa[2], static_cast<float>(v[2]), x);
        x = fmaf(pa[3], static_cast<float>(v[3]), x);
        x = fmaf(pc[0], static_cast<float>(v[4]), x);
        x = fmaf(pc[1], static_cast<float>(v[5]), x);
        x = fmaf(pc[2], static_cast<float>(v[6]), x);
        x = fmaf(pc[3], static_cast<float>(v[7]), x);
        acc[nb] = x;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) acc[nb] = sum_halves(acc[nb]);
  l = wave_sum64(l);

  if (half == 0) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) w_o[wave][32 * nb + i] = acc[nb];
  }
  if (lane == 0) {
    w_m[wave] = m;
    w_l[wave] = l;
  }
  __syncthreads();
  if (threadIdx.x < D) {
    // wave 0 always has a chunk, so M is finite and empty waves weigh 0
    const float M = fmaxf(fmaxf(w_m[0], w_m[1]), fmaxf(w_m[2], w_m[3]));
    float o = 0.f, s = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float wt = exp2f(w_m[w] - M);
      o += wt * w_o[w][threadIdx.x];
      s += wt * w_l[w];
    }
    const size_t pid = static_cast<size_t>(part_id) * H + head;
    if constexpr (kFuse) {
      store_agent(a.part_o + pid * D + threadIdx.x, o);
      if (threadIdx.x == 0) {
        store_agent(a.part_ms + pid * 2 + 0, M);
        store_agent(a.part_ms + pid * 2 + 1, s);
      }
      wait_stores();
    } else {
      a.part_o[pid * D + threadIdx.x] = o;
      if (threadIdx.x == 0) {
        a.part_ms[pid * 2 + 0] = M;
        a.part_ms[pid * 2 + 1] = s;
      }
    }
  }
  if constexpr (!kFuse) return;
  __syncthreads();  // every thread's partial stores have completed
  if (threadIdx.x == 0) arrive(a, dfs_pos, head);
}

// n_cf, n_sf: chunk-first and sequence-first blocks of the step; first:
// index of this launch's first block in the step's grid (0, or n_cf to launch
// only the sequence-first part).  kFuse: the one-launch step, whose grid ends
// with the merge blocks.  kAppend: a decode step
// with in-kernel appends (StepArgs::app_k set).
template <bool kFuse, bool kAppend, bool kHalf, bool kRow>
__global__ __launch_bounds__(256, 3) void partials_kernel(StepArgs a, int n_cf, int n_sf, int first) {
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  const int b = blockIdx.x + first;
  if (b < n_cf) {
    const int logical = xcd_remap(b, n_cf);
    if (a.cf_units[(logical % a.n_cf_units) * 32 + kCfReuseField])
      chunk_first_block<kFuse, false, kHalf>(a, logical, smem);
    else
      chunk_first_block<kFuse, true, kHalf>(a, logical, smem);
  } else if (b < n_cf + n_sf) {
    const int logical = b - n_cf;
    if (a.sf_tasks[(logical / a.heads) * 16 + kSfReuseField])
      sequence_first_block<kFuse, false, kAppend, kHalf, kRow>(a, logical, smem);
    else
      sequence_first_block<kFuse, true, kAppend, kHalf, kRow>(a, logical, smem);
  }
  else if constexpr (kFuse)
    merge_block(a, b - n_cf - n_sf);
}

// Merge of every (sequence, head), four per block (the unfused step).
__global__ __launch_bounds__(256) void merge_kernel(StepArgs a) {
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= a.n_seq * a.heads) return;
  const int pos = item / a.heads, head = item - pos * a.heads;
  if (a.dense_parts > 0)
    merge_dense<false>(a, pos, head, threadIdx.x & 63, a.seq_parts[2 * pos + 1], a.dfs_qrow[pos]);
  else
    merge_one<false>(a, pos, head, threadIdx.x & 63);
}

}  // namespace

int launch_partials(const StepArgs& a, int part, bool fuse_merge, void* stream) {
  const int n_cf = a.n_cf_units * a.heads, n_sf = a.n_sf_tasks * a.heads;
  const bool fuse = fuse_merge && part == kPartsBoth;
  const int n_merge = fuse ? (a.n_seq * a.heads + 3) / 4 : 0;
  const int first = part == kPartsSequenceFirst ? n_cf : 0;
  const int count = part == kPartsChunkFirst ? n_cf : part == kPartsSequenceFirst ? n_sf : n_cf + n_sf + n_merge;
  if (count <= 0) return 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool append = a.app_k != nullptr;
  const dim3 grid(count), block(256);
#define CA_LAUNCH(F, A, HT, R) \
  hipLaunchKernelGGL((partials_kernel<F, A, HT, R>), grid, block, 0, st, a, n_cf, n_sf, first)
#define CA_LAUNCH_FA(HT, R)                 \
  if (fuse && append) CA_LAUNCH(true, true, HT, R);   \
  else if (fuse) CA_LAUNCH(true, false, HT, R);       \
  else if (append) CA_LAUNCH(false, true, HT, R);     \
  else CA_LAUNCH(false, false, HT, R);
  if (a.half_tiles) {
    if (a.row_chunks) { CA_LAUNCH_FA(true, true) } else { CA_LAUNCH_FA(true, false) }
  } else {
    if (a.row_chunks) { CA_LAUNCH_FA(false, true) } else { CA_LAUNCH_FA(false, false) }
  }
#undef CA_LAUNCH_FA
#undef CA_LAUNCH
  return static_cast<int>(hipGetLastError());
}

int launch_merge(const StepArgs& a, void* stream) {
  if (a.n_seq <= 0) return 0;
  dim3 grid((a.n_seq * a.heads + 3) / 4);
  hipLaunchKernelGGL(merge_kernel, grid, dim3(256), 0, static_cast<hipStream_t>(stream), a);
  return static_cast<int>(hipGetLastError());
}

// The workspace of the allocation-free step: chunk table, arrival counters
// and partial results of one step, at most kStaticScratchBytes.  On the host
// the name stands for a host-side shadow, never for the device memory: host
// code uses only the address that hipGetSymbolAddress returns per device.
static __device__ __align__(256) char scratch[kStaticScratchBytes];

int static_scratch(void** ptr, int* device) {
  static std::mutex mu;
  static void* addr[kMaxScratchDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return static_cast<int>(e);
  if (dev < 0 || dev >= kMaxScratchDevices) return static_cast<int>(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return static_cast<int>(e);
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *device = dev;
  return 0;
}

}  // namespace chunkattn
