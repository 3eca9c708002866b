// gfx950 (CDNA4) kernels of the ChunkAttention decode step.
//
// Two-phase partition (paperlayer.ai summary of arXiv 2402.15220v4, section
// 3.2 and Figure 2): the chunk-first kernel batches the queries of all
// sequences that share a chunk into a matrix and runs both products on MFMA;
// the sequence-first kernel streams each sequence's private chunks; both
// write partial results (o, m, s) that the merge kernel combines by
// log-sum-exp (explainer 0h-n0.github.io/posts/paper-2402-15220, output
// combination formula; m is a running max, s and o are unnormalised).
//
// Chunk tile layout.  Slot s, head h: K tile at ((s*H + h)*2 + 0) * 8192
// halves, V tile right after it.  Within a tile the 64 x 128 fp16 elements
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
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kernels.h"

namespace chunkattn {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int D = kHeadDim;
constexpr int C = kChunk;
constexpr int TILE = C * D;  // halves per tile

__device__ __forceinline__ size_t tile_base(int slot, int head, int heads, int kv) {
  return ((static_cast<size_t>(slot) * heads + head) * 2 + kv) * TILE;
}

__device__ __forceinline__ int k_off(int key, int dim) {
  return ((((key >> 5) * 8 + (dim >> 4)) * 2 + ((dim >> 3) & 1)) * 32 + (key & 31)) * 8 + (dim & 7);
}

__device__ __forceinline__ int v_off(int key, int dim) {
  return ((((dim >> 5) * 4 + (key >> 4)) * 2 + ((key >> 2) & 1)) * 32 + (dim & 31)) * 8 +
         ((key & 3) | (((key >> 3) & 1) << 2));
}

// Blocks are handed to the 8 XCDs round robin; give each XCD a contiguous
// range of logical ids so work that reads the same chunk shares an L2.
__device__ __forceinline__ int xcd_remap(int b, int n) {
  int xcd = b & 7, local = b >> 3, q = n >> 3, r = n & 7;
  return xcd * q + min(xcd, r) + local;
}

__device__ __forceinline__ float wave_max32(float x) {
  // max over the 32 lanes of each half-wave
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 8));
  x = fmaxf(x, __shfl_xor(x, 4));
  x = fmaxf(x, __shfl_xor(x, 2));
  x = fmaxf(x, __shfl_xor(x, 1));
  return x;
}

__device__ __forceinline__ float wave_sum64(float x) {
  x += __shfl_xor(x, 32);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 8);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 1);
  return x;
}

__device__ __forceinline__ h2 lo2(h8 v, int j) {
  switch (j) {
    case 0: return __builtin_shufflevector(v, v, 0, 1);
    case 1: return __builtin_shufflevector(v, v, 2, 3);
    case 2: return __builtin_shufflevector(v, v, 4, 5);
    default: return __builtin_shufflevector(v, v, 6, 7);
  }
}

// ---------------------------------------------------------------------------
// KV writes: caller rows or another slot's rows into one slot's tiles.
// grid (n_ops, heads, 2), 256 threads; each thread writes 4 x 16 bytes.
__global__ __launch_bounds__(256) void kv_write_kernel(_Float16* pool, int heads, KvOpBatch batch,
                                                       const _Float16* k_src, const _Float16* v_src) {
  const KvOpDev op = batch.ops[blockIdx.x];
  const int head = blockIdx.y, kv = blockIdx.z;
  _Float16* dst = pool + tile_base(op.dst_slot, head, heads, kv);
  const _Float16* src_pool = op.from_pool ? pool + tile_base(op.src_slot, head, heads, kv) : nullptr;
  const _Float16* src = kv ? v_src : k_src;
  for (int u = threadIdx.x; u < TILE / 8; u += 256) {
    const int L = u >> 6, lane = u & 63, half = lane >> 5, i = lane & 31;
    h8 cur = *reinterpret_cast<const h8*>(dst + u * 8);
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
        const int sr = op.src_row0 + r;
        if (op.from_pool)
          x = src_pool[kv == 0 ? k_off(sr, dim) : v_off(sr, dim)];
        else
          x = src[(static_cast<size_t>(sr) * heads + head) * D + dim];
      } else {
        x = op.zero_rest ? static_cast<_Float16>(0.0f) : cur[e];
      }
      val[e] = x;
    }
    *reinterpret_cast<h8*>(dst + u * 8) = val;
  }
}

// ---------------------------------------------------------------------------
// Chunk-first: one block per (unit = run of shared chunks x 32-row block,
// head).  Wave w takes chunks w, w+4, ... of the run; lane (half, i) owns
// query row i.  Per chunk: S^T[64 keys x 32 rows] = K Q^T (16 MFMA), online
// softmax along keys (each lane holds 32 keys of its row, its twin lane the
// other 32), O^T[128 x 32] += V^T P^T (16 MFMA).  The four waves' states are
// merged in LDS and one partial per row is written.
constexpr int kOStride = 132;  // padded row stride of the LDS merge buffer

__global__ __launch_bounds__(256) void chunk_first_kernel(StepArgs a) {
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int unit = logical % a.n_cf_units, head = logical / a.n_cf_units;
  const int* u = a.cf_units + unit * 8;
  const int chunk_begin = u[0], n_chunks = u[1], row_begin = u[2], n_rows = u[3], part_base = u[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, half = lane >> 5, i = lane & 31;
  const int H = a.heads;
  const _Float16* pool = static_cast<const _Float16*>(a.pool);

  h8 qb[8];
  {
    const bool ok = i < n_rows;
    const int qrow = a.dfs_qrow[row_begin + (ok ? i : 0)];
    const _Float16* qp = static_cast<const _Float16*>(a.q) + (static_cast<size_t>(qrow) * H + head) * D;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      h8 v = *reinterpret_cast<const h8*>(qp + kk * 16 + half * 8);
      qb[kk] = ok ? v : h8{};
    }
  }

  float m = -INFINITY, l = 0.f;
  f16v acc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) acc[nb] = f16v{};

  for (int c = wave; c < n_chunks; c += 4) {
    const int slot = a.chunk_refs[2 * (chunk_begin + c)];
    const int nvalid = a.chunk_refs[2 * (chunk_begin + c) + 1];
    const _Float16* kt = pool + tile_base(slot, head, H, 0);
    const _Float16* vt = kt + TILE;

    f16v s0 = f16v{}, s1 = f16v{};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      h8 k0 = *reinterpret_cast<const h8*>(kt + ((0 * 8 + kk) * 64 + lane) * 8);
      h8 k1 = *reinterpret_cast<const h8*>(kt + ((1 * 8 + kk) * 64 + lane) * 8);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(k0, qb[kk], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(k1, qb[kk], s1, 0, 0, 0);
    }
    h8 va[16];
#pragma unroll
    for (int L = 0; L < 16; ++L) va[L] = *reinterpret_cast<const h8*>(vt + (L * 64 + lane) * 8);

    // s0[r] is key 8*(r/4) + 4*half + r%4 of row i; s1 the same key + 32.
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r >> 2) + 4 * half + (r & 3);
      const float x0 = key < nvalid ? s0[r] * a.scale_log2e : -INFINITY;
      const float x1 = key + 32 < nvalid ? s1[r] * a.scale_log2e : -INFINITY;
      s0[r] = x0;
      s1[r] = x1;
      mx = fmaxf(mx, fmaxf(x0, x1));
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m, mx);
    const float alpha = exp2f(m - mnew);
    float psum = 0.f;
    h8 pb[4];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p0 = exp2f(s0[r] - mnew);
      const float p1 = exp2f(s1[r] - mnew);
      psum += p0 + p1;
      pb[(r >> 3)][r & 7] = static_cast<_Float16>(p0);
      pb[2 + (r >> 3)][r & 7] = static_cast<_Float16>(p1);
    }
    l = l * alpha + psum;
    m = mnew;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      acc[nb] *= alpha;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[nb * 4 + s], pb[s], acc[nb], 0, 0, 0);
    }
  }
  l += __shfl_xor(l, 32);

  __shared__ float lds_o[4][32][kOStride];
  __shared__ float lds_m[4][32];
  __shared__ float lds_l[4][32];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f4 v = {acc[nb][4 * g + 0], acc[nb][4 * g + 1], acc[nb][4 * g + 2], acc[nb][4 * g + 3]};
      *reinterpret_cast<f4*>(&lds_o[wave][i][32 * nb + 8 * g + 4 * half]) = v;
    }
  if (half == 0) {
    lds_m[wave][i] = m;
    lds_l[wave][i] = l;
  }
  __syncthreads();

  const int row = threadIdx.x >> 3, d0 = (threadIdx.x & 7) * 16;
  if (row < n_rows) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, lds_m[w][row]);
    float wt[4], s = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      wt[w] = exp2f(lds_m[w][row] - M);
      s += wt[w] * lds_l[w][row];
    }
    const size_t pid = static_cast<size_t>(part_base + row) * H + head;
    float* po = a.part_o + pid * D + d0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f4 o = f4{};
#pragma unroll
      for (int w = 0; w < 4; ++w) o += wt[w] * *reinterpret_cast<const f4*>(&lds_o[w][row][d0 + 4 * g]);
      *reinterpret_cast<f4*>(po + 4 * g) = o;
    }
    if ((threadIdx.x & 7) == 0) {
      a.part_ms[pid * 2 + 0] = M;
      a.part_ms[pid * 2 + 1] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// Sequence-first: one block per (task = some private chunks of one sequence,
// head).  Wave w takes chunks w, w+4, ...  Lane (half, i): for K it holds
// dims [16kk + 8half, +8) of keys i and 32+i, so a score needs one exchange
// with the twin lane; for V it holds dims 32nb + i at 8 keys per load, and
// reads the matching probabilities from a 64-entry LDS row.
__global__ __launch_bounds__(256) void sequence_first_kernel(StepArgs a) {
  const int task = blockIdx.x % a.n_sf_tasks, head = blockIdx.x / a.n_sf_tasks;
  const int* t = a.sf_tasks + task * 4;
  const int chunk_begin = t[0], n_chunks = t[1], dfs_pos = t[2], part_id = t[3];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, half = lane >> 5, i = lane & 31;
  const int H = a.heads;
  const _Float16* pool = static_cast<const _Float16*>(a.pool);

  h8 qv[8];
  {
    const int qrow = a.dfs_qrow[dfs_pos];
    const _Float16* qp = static_cast<const _Float16*>(a.q) + (static_cast<size_t>(qrow) * H + head) * D;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qv[kk] = *reinterpret_cast<const h8*>(qp + kk * 16 + half * 8);
  }

  __shared__ float p_lds[4][64];
  float m = -INFINITY, l = 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};

  for (int c = wave; c < n_chunks; c += 4) {
    const int slot = a.chunk_refs[2 * (chunk_begin + c)];
    const int nvalid = a.chunk_refs[2 * (chunk_begin + c) + 1];
    const _Float16* kt = pool + tile_base(slot, head, H, 0);
    const _Float16* vt = kt + TILE;
    h8 ka[16], va[16];
#pragma unroll
    for (int L = 0; L < 16; ++L) ka[L] = *reinterpret_cast<const h8*>(kt + (L * 64 + lane) * 8);
#pragma unroll
    for (int L = 0; L < 16; ++L) va[L] = *reinterpret_cast<const h8*>(vt + (L * 64 + lane) * 8);

    float d0 = 0.f, d1 = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        d0 = __builtin_amdgcn_fdot2(lo2(ka[kk], j), lo2(qv[kk], j), d0, false);
        d1 = __builtin_amdgcn_fdot2(lo2(ka[8 + kk], j), lo2(qv[kk], j), d1, false);
      }
    d0 += __shfl_xor(d0, 32);
    d1 += __shfl_xor(d1, 32);
    const float x0 = i < nvalid ? d0 * a.scale_log2e : -INFINITY;
    const float x1 = i + 32 < nvalid ? d1 * a.scale_log2e : -INFINITY;
    const float mx = wave_max32(fmaxf(x0, x1));
    const float mnew = fmaxf(m, mx);
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
    for (int s = 0; s < 4; ++s) {
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
  for (int nb = 0; nb < 4; ++nb) acc[nb] += __shfl_xor(acc[nb], 32);
  l = wave_sum64(l);

  __shared__ float w_o[4][D];
  __shared__ float w_m[4], w_l[4];
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
    float M = fmaxf(fmaxf(w_m[0], w_m[1]), fmaxf(w_m[2], w_m[3]));
    float o = 0.f, s = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float wt = exp2f(w_m[w] - M);
      o += wt * w_o[w][threadIdx.x];
      s += wt * w_l[w];
    }
    const size_t pid = static_cast<size_t>(part_id) * H + head;
    a.part_o[pid * D + threadIdx.x] = o;
    if (threadIdx.x == 0) {
      a.part_ms[pid * 2 + 0] = M;
      a.part_ms[pid * 2 + 1] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// Merge: one wave per (sequence, head).  Folds the sequence's partials in the
// fixed order of its list (shared runs root first, then private tasks):
// M = max m_j, o = sum e^{m_j - M} o_j, s = sum e^{m_j - M} s_j, out = o / s.
__global__ __launch_bounds__(64) void merge_kernel(StepArgs a) {
  const int H = a.heads;
  const int pos = blockIdx.x / H, head = blockIdx.x % H, lane = threadIdx.x;
  const int first = a.seq_parts[2 * pos], cnt = a.seq_parts[2 * pos + 1];
  float M = -INFINITY;
  for (int j = lane; j < cnt; j += 64) {
    const size_t pid = static_cast<size_t>(a.part_list[first + j]) * H + head;
    M = fmaxf(M, a.part_ms[pid * 2]);
  }
  M = fmaxf(M, __shfl_xor(M, 32));
  M = wave_max32(M);
  float s = 0.f, o0 = 0.f, o1 = 0.f;
  for (int j = 0; j < cnt; ++j) {
    const size_t pid = static_cast<size_t>(a.part_list[first + j]) * H + head;
    const float wt = exp2f(a.part_ms[pid * 2] - M);
    s += wt * a.part_ms[pid * 2 + 1];
    const float2 o = *reinterpret_cast<const float2*>(a.part_o + pid * D + 2 * lane);
    o0 += wt * o.x;
    o1 += wt * o.y;
  }
  const float inv = 1.0f / s;
  const int qrow = a.dfs_qrow[pos];
  _Float16* out = static_cast<_Float16*>(a.out) + (static_cast<size_t>(qrow) * H + head) * D + 2 * lane;
  h2 r = {static_cast<_Float16>(o0 * inv), static_cast<_Float16>(o1 * inv)};
  *reinterpret_cast<h2*>(out) = r;
}

}  // namespace

int launch_kv_write(void* pool, int heads, const KvOpBatch& batch, int n_ops, const void* k_src,
                    const void* v_src, void* stream) {
  if (n_ops <= 0) return 0;
  dim3 grid(n_ops, heads, 2);
  hipLaunchKernelGGL(kv_write_kernel, grid, dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<_Float16*>(pool), heads, batch, static_cast<const _Float16*>(k_src),
                     static_cast<const _Float16*>(v_src));
  return static_cast<int>(hipGetLastError());
}

int launch_chunk_first(const StepArgs& a, void* stream) {
  if (a.n_cf_units <= 0) return 0;
  dim3 grid(a.n_cf_units * a.heads);
  hipLaunchKernelGGL(chunk_first_kernel, grid, dim3(256), 0, static_cast<hipStream_t>(stream), a);
  return static_cast<int>(hipGetLastError());
}

int launch_sequence_first(const StepArgs& a, void* stream) {
  if (a.n_sf_tasks <= 0) return 0;
  dim3 grid(a.n_sf_tasks * a.heads);
  hipLaunchKernelGGL(sequence_first_kernel, grid, dim3(256), 0, static_cast<hipStream_t>(stream), a);
  return static_cast<int>(hipGetLastError());
}

int launch_merge(const StepArgs& a, void* stream) {
  if (a.n_seq <= 0) return 0;
  dim3 grid(a.n_seq * a.heads);
  hipLaunchKernelGGL(merge_kernel, grid, dim3(64), 0, static_cast<hipStream_t>(stream), a);
  return static_cast<int>(hipGetLastError());
}

}  // namespace chunkattn
