// S3 / S4: adaptive block selection. VSA page ("Faster Video Diffusion with
// Trainable Sparse Attention"), Research Type row: a coarse stage picks key
// blocks per query block; FVAttn summary: Top-p routing with a Top-k safety
// floor, per head, over video-aware blocks.
//
// Three kernels, all deterministic (fixed reduction orders, no float atomics):
//   pool   : per (tensor, b, head, tile) mean over real rows, fp32; a second
//            form reads the natural order and writes the tiled copy on the
//            way (the tile permute with the pool folded in);
//   score  : s_ij = coarse_scale * <qbar_i, kbar_j>, fp32, one 64x64 block of
//            (i, j) per workgroup through LDS;
//   select : per (b, head, i) row, bitonic sort of 64-bit keys
//            (score desc, index asc), top-k or top-p + floor, then the kept
//            indices compacted in ascending order.
#include <float.h>

#include "vsa_internal.h"

namespace vsa {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxTiles = 4096;

// ---------------------------------------------------------------- pool
// MOVE = false: grid (n_tiles, heads, B * 2); z selects tiled Q (even) or K
// (odd); pooled is [2][B][heads][n_tiles][d], counts gets the real rows per tile.
// MOVE = true: the tile permute with the pool folded in. grid (n_tiles, heads,
// B); q is the natural-order tensor [B, n_tokens, heads, d]; every row read is
// also written to its tiled position in `tiled` (pad rows as zeros), pooled is
// [B][heads][n_tiles][d]. Both forms give each thread the same rows and
// chunks and sum them in the same order, so their means are bit-identical.
template <bool MOVE>
__global__ __launch_bounds__(kThreads) void pool_kernel(DevLayout L, const uint4* __restrict__ q,
                                                        const uint4* __restrict__ k,
                                                        uint4* __restrict__ tiled,
                                                        float* __restrict__ pooled,
                                                        int* __restrict__ counts) {
  const int tile = blockIdx.x;
  const int head = blockIdx.y;
  const int b = MOVE ? (int)blockIdx.z : (int)(blockIdx.z >> 1);
  const int which = MOVE ? 0 : (int)(blockIdx.z & 1);
  const uint4* x = which ? k : q;
  const int chunks = L.d >> 3;                       // 8 bf16 per chunk
  const int groups = kThreads / chunks;              // row groups summed in parallel
  const int ch = threadIdx.x % chunks;
  const int rg = threadIdx.x / chunks;
  const long long row0 = (long long)(b * L.heads + head) * L.n_padded + (long long)tile * L.C;
  const TileValid tv = tile_valid(L, tile);

  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  if (rg < groups) {
    for (int r = rg; r < L.C; r += groups) {
      const long long t_off = (row0 + r) * chunks + ch;
      uint4 w;
      if (MOVE) {
        const int nat = natural_index(L, tile, r);
        if (nat < 0) {
          tiled[t_off] = make_uint4(0u, 0u, 0u, 0u);
          continue;
        }
        w = x[(((long long)b * L.n_tokens + nat) * L.heads + head) * chunks + ch];
        tiled[t_off] = w;
      } else {
        if (!row_is_real(L, tv, r)) continue;
        w = x[t_off];
      }
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += __uint_as_float(ws[e] << 16);
        acc[2 * e + 1] += __uint_as_float(ws[e] & 0xFFFF0000u);
      }
    }
  }
  __shared__ float part[kThreads * 8];
#pragma unroll
  for (int e = 0; e < 8; ++e) part[threadIdx.x * 8 + e] = acc[e];
  __syncthreads();
  const int n = real_rows(L, tv);
  const long long out0 = (((long long)which * L.B + b) * L.heads + head) * L.n_tiles + tile;
  for (int c = threadIdx.x; c < L.d; c += kThreads) {
    const int cch = c >> 3, ce = c & 7;
    float s = 0.0f;
    for (int g = 0; g < groups; ++g) s += part[(g * chunks + cch) * 8 + ce];
    pooled[out0 * L.d + c] = n > 0 ? s / (float)n : 0.0f;
  }
  if (!MOVE && threadIdx.x == 0 && which == 0 && b == 0 && head == 0) counts[tile] = n;
}

// Real rows per tile, for routing from means pooled elsewhere.
__global__ __launch_bounds__(kThreads) void counts_kernel(DevLayout L, int* __restrict__ counts) {
  const int t = blockIdx.x * kThreads + threadIdx.x;
  if (t < L.n_tiles) counts[t] = real_rows(L, tile_valid(L, t));
}

// ---------------------------------------------------------------- score
// grid (ceil(n/64) key blocks, ceil(n/64) query blocks, B * heads)
constexpr int kSB = 64;
__global__ __launch_bounds__(kThreads) void score_kernel(DevLayout L, const float* __restrict__ q_pooled,
                                                         const float* __restrict__ k_pooled,
                                                         const int* __restrict__ counts,
                                                         float coarse_scale,
                                                         float* __restrict__ scores) {
  const int j0 = blockIdx.x * kSB;
  const int i0 = blockIdx.y * kSB;
  const int bh = blockIdx.z;
  const int n = L.n_tiles;
  const float* qb = q_pooled + (long long)bh * n * L.d;
  const float* kb = k_pooled + (long long)bh * n * L.d;
  __shared__ float qs[kSB][33];
  __shared__ float ks[kSB][33];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;   // 16 x 16 threads, 4 x 4 outputs each
  float acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = 0.0f;
  for (int e0 = 0; e0 < L.d; e0 += 32) {
    for (int idx = threadIdx.x; idx < kSB * 32; idx += kThreads) {
      const int r = idx >> 5, e = idx & 31;
      const int ei = e0 + e;
      qs[r][e] = (i0 + r < n && ei < L.d) ? qb[(long long)(i0 + r) * L.d + ei] : 0.0f;
      ks[r][e] = (j0 + r < n && ei < L.d) ? kb[(long long)(j0 + r) * L.d + ei] : 0.0f;
    }
    __syncthreads();
#pragma unroll 8
    for (int e = 0; e < 32; ++e) {
      float qv[4], kv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) qv[a] = qs[ty * 4 + a][e];
#pragma unroll
      for (int c = 0; c < 4; ++c) kv[c] = ks[tx * 4 + c][e];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[a][c] = fmaf(qv[a], kv[c], acc[a][c]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int i = i0 + ty * 4 + a;
    if (i >= n) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = j0 + tx * 4 + c;
      if (j >= n) continue;
      scores[((long long)bh * n + i) * n + j] = counts[j] > 0 ? coarse_scale * acc[a][c] : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------- select
__device__ __forceinline__ uint32_t float_order(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float order_float(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// Inclusive scan over one value per thread in a fixed order (Hillis-Steele).
__device__ float block_scan_f(float v, float* buf) {
  buf[threadIdx.x] = v;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const float add = threadIdx.x >= off ? buf[threadIdx.x - off] : 0.0f;
    __syncthreads();
    buf[threadIdx.x] += add;
    __syncthreads();
  }
  const float r = buf[threadIdx.x];
  __syncthreads();
  return r;
}
__device__ int block_scan_i(int v, int* buf) {
  buf[threadIdx.x] = v;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const int add = threadIdx.x >= off ? buf[threadIdx.x - off] : 0;
    __syncthreads();
    buf[threadIdx.x] += add;
    __syncthreads();
  }
  const int r = buf[threadIdx.x];
  __syncthreads();
  return r;
}

// grid (n_tiles, heads, B); dynamic LDS: npow2 * 8 bytes of keys + n_tiles flags
__global__ __launch_bounds__(kThreads) void select_kernel(DevLayout L, const float* __restrict__ scores,
                                                          const int* __restrict__ counts, int npow2,
                                                          int top_k, float top_p, int k_floor,
                                                          int max_kv, int32_t* __restrict__ kv_idx,
                                                          int32_t* __restrict__ kv_cnt) {
  extern __shared__ unsigned long long keys[];
  __shared__ float fbuf[kThreads];
  __shared__ int ibuf[kThreads];
  __shared__ int s_count;
  const int i = blockIdx.x, head = blockIdx.y, b = blockIdx.z;
  const int n = L.n_tiles;
  const long long bh = (long long)b * L.heads + head;
  const float* row = scores + (bh * n + i) * n;
  int32_t* out_idx = kv_idx + (bh * n + i) * max_kv;
  int32_t* out_cnt = kv_cnt + bh * n + i;
  unsigned char* flags = reinterpret_cast<unsigned char*>(keys + npow2);

  if (counts[i] == 0) {                       // query tile without real tokens
    if (threadIdx.x == 0) *out_cnt = 0;
    return;
  }
  // build keys: (order(score) << 32) | (~index); invalid key tiles and padding -> 0
  int nvalid_local = 0;
  for (int j = threadIdx.x; j < npow2; j += kThreads) {
    unsigned long long key = 0ull;
    if (j < n && counts[j] > 0) {
      key = ((unsigned long long)float_order(row[j]) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)j);
      ++nvalid_local;
    }
    keys[j] = key;
    if (j < n) flags[j] = 0;
  }
  const int nvalid = block_scan_i(nvalid_local, ibuf);   // inclusive; last thread holds total
  if (threadIdx.x == kThreads - 1) s_count = nvalid;
  __syncthreads();
  const int n_valid = s_count;
  __syncthreads();

  // bitonic sort, descending
  for (int kk = 2; kk <= npow2; kk <<= 1) {
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      for (int p = threadIdx.x; p < (npow2 >> 1); p += kThreads) {
        const int a = ((p & ~(jj - 1)) << 1) | (p & (jj - 1));
        const int c = a + jj;
        const bool desc = (a & kk) == 0;
        const unsigned long long ka = keys[a], kc = keys[c];
        if ((ka < kc) == desc) {
          keys[a] = kc;
          keys[c] = ka;
        }
      }
      __syncthreads();
    }
  }

  int count;
  if (top_p > 0.0f) {
    // probabilities in sorted order; each thread owns a contiguous run
    const int per = npow2 / kThreads > 0 ? npow2 / kThreads : 1;
    const int lo = threadIdx.x * per;
    const float smax = order_float((uint32_t)(keys[0] >> 32));
    float local = 0.0f;
    for (int m = lo; m < lo + per && m < n_valid; ++m)
      local += exp2f((order_float((uint32_t)(keys[m] >> 32)) - smax) * 1.4426950408889634f);
    const float incl = block_scan_f(local, fbuf);
    if (threadIdx.x == kThreads - 1) fbuf[0] = incl;    // total mass (after scan's last sync)
    __syncthreads();
    const float total = fbuf[0];
    __syncthreads();
    const float target = top_p * total;
    float cum = incl - local;                             // exclusive prefix of this run
    int first = 0x7FFFFFFF;
    for (int m = lo; m < lo + per && m < n_valid; ++m) {
      cum += exp2f((order_float((uint32_t)(keys[m] >> 32)) - smax) * 1.4426950408889634f);
      if (cum >= target) {
        first = m;
        break;
      }
    }
    // min over threads
    ibuf[threadIdx.x] = first;
    __syncthreads();
    for (int off = kThreads / 2; off > 0; off >>= 1) {
      if (threadIdx.x < off) ibuf[threadIdx.x] = min(ibuf[threadIdx.x], ibuf[threadIdx.x + off]);
      __syncthreads();
    }
    const int m_star = ibuf[0];
    __syncthreads();
    count = (m_star == 0x7FFFFFFF) ? n_valid : m_star + 1;
    count = min(max(count, k_floor), n_valid);
  } else {
    count = min(top_k, n_valid);
  }

  for (int m = threadIdx.x; m < count; m += kThreads)
    flags[0xFFFFFFFFu - (uint32_t)(keys[m] & 0xFFFFFFFFull)] = 1;
  __syncthreads();
  // compact kept indices in ascending order
  const int per = (n + kThreads - 1) / kThreads;
  const int lo = threadIdx.x * per;
  int mine = 0;
  for (int j = lo; j < lo + per && j < n; ++j) mine += flags[j];
  int pos = block_scan_i(mine, ibuf) - mine;
  for (int j = lo; j < lo + per && j < n; ++j)
    if (flags[j]) out_idx[pos++] = j;
  if (threadIdx.x == 0) *out_cnt = count;
}

}  // namespace

size_t route_workspace_bytes(const DevLayout& L) {
  const size_t n = (size_t)L.n_tiles;
  const size_t pooled = 2ull * L.B * L.heads * n * L.d * sizeof(float);
  const size_t counts = ((n * sizeof(int) + 255) / 256) * 256;
  const size_t scores = (size_t)L.B * L.heads * n * n * sizeof(float);
  return ((pooled + 255) / 256) * 256 + counts + scores;
}

// Score and select from pooled means; counts already hold the real rows per tile.
static hipError_t route_from_pooled(const DevLayout& L, const float* q_pooled, const float* k_pooled,
                                    const int* counts, float coarse_scale, int top_k, float top_p,
                                    int k_floor, int max_kv, int32_t* kv_idx, int32_t* kv_cnt,
                                    float* sc, hipStream_t s) {
  const int nb = (L.n_tiles + kSB - 1) / kSB;
  hipLaunchKernelGGL(score_kernel, dim3(nb, nb, L.B * L.heads), dim3(kThreads), 0, s, L, q_pooled,
                     k_pooled, counts, coarse_scale, sc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int npow2 = 256;
  while (npow2 < L.n_tiles) npow2 <<= 1;
  const size_t lds = (size_t)npow2 * 8 + ((L.n_tiles + 15) / 16) * 16;
  hipLaunchKernelGGL(select_kernel, dim3(L.n_tiles, L.heads, L.B), dim3(kThreads), lds, s, L, sc,
                     counts, npow2, top_k, top_p, k_floor, max_kv, kv_idx, kv_cnt);
  return hipGetLastError();
}

struct RouteScratch {
  float* pooled;
  int* counts;
  float* scores;
};

static RouteScratch carve(const DevLayout& L, void* ws, float* scores) {
  const size_t n = (size_t)L.n_tiles;
  char* base = static_cast<char*>(ws);
  const size_t pooled_b = ((2ull * L.B * L.heads * n * L.d * sizeof(float) + 255) / 256) * 256;
  const size_t counts_b = ((n * sizeof(int) + 255) / 256) * 256;
  RouteScratch r;
  r.pooled = reinterpret_cast<float*>(base);
  r.counts = reinterpret_cast<int*>(base + pooled_b);
  r.scores = scores ? scores : reinterpret_cast<float*>(base + pooled_b + counts_b);
  return r;
}

hipError_t launch_route(const DevLayout& L, const void* q, const void* k, float coarse_scale,
                        int top_k, float top_p, int k_floor, int max_kv, int32_t* kv_idx,
                        int32_t* kv_cnt, float* scores, void* ws, hipStream_t s) {
  const RouteScratch r = carve(L, ws, scores);
  hipLaunchKernelGGL(pool_kernel<false>, dim3(L.n_tiles, L.heads, L.B * 2), dim3(kThreads), 0, s,
                     L, static_cast<const uint4*>(q), static_cast<const uint4*>(k), nullptr,
                     r.pooled, r.counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t per = (size_t)L.B * L.heads * L.n_tiles * L.d;
  return route_from_pooled(L, r.pooled, r.pooled + per, r.counts, coarse_scale, top_k, top_p,
                           k_floor, max_kv, kv_idx, kv_cnt, r.scores, s);
}

hipError_t launch_route_pooled(const DevLayout& L, const float* q_pooled, const float* k_pooled,
                               float coarse_scale, int top_k, float top_p, int k_floor, int max_kv,
                               int32_t* kv_idx, int32_t* kv_cnt, float* scores, void* ws,
                               hipStream_t s) {
  const RouteScratch r = carve(L, ws, scores);
  hipLaunchKernelGGL(counts_kernel, dim3((L.n_tiles + kThreads - 1) / kThreads), dim3(kThreads), 0,
                     s, L, r.counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return route_from_pooled(L, q_pooled, k_pooled, r.counts, coarse_scale, top_k, top_p, k_floor,
                           max_kv, kv_idx, kv_cnt, r.scores, s);
}

hipError_t launch_permute_pool(const DevLayout& L, const void* src, void* dst, float* pooled,
                               hipStream_t s) {
  hipLaunchKernelGGL(pool_kernel<true>, dim3(L.n_tiles, L.heads, L.B), dim3(kThreads), 0, s, L,
                     static_cast<const uint4*>(src), nullptr, static_cast<uint4*>(dst), pooled,
                     nullptr);
  return hipGetLastError();
}

}  // namespace vsa
