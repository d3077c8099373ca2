// S3 / S4: adaptive block selection. VSA page ("Faster Video Diffusion with
// Trainable Sparse Attention"), Research Type row: a coarse stage picks key
// blocks per query block; FVAttn summary: Top-p routing with a Top-k safety
// floor, per head, over video-aware blocks.
//
// Two kernels, both deterministic (fixed reduction orders, no float atomics):
//   pool  : per (tensor, b, head, tile) mean over real rows, fp32; a second
//           form reads the natural order and writes the tiled copy on the
//           way (the tile permute with the pool folded in);
//   route : coarse scores s_ij = coarse_scale * <qbar_i, kbar_j> for a block
//           of query tiles, kept in LDS, then per (b, head, i) row a
//           wavefront selects top-k, or top-p with a floor, by threshold
//           searches over order-preserving score keys, and writes the kept
//           indices in ascending order.
#include <float.h>

#include "vsa_internal.h"

namespace vsa {
namespace {

constexpr int kThreads = 256;
constexpr int kRowBatch = 4;      // rows whose loads a pool thread issues together

// ---------------------------------------------------------------- pool
// MOVE = false: grid (n_tiles, heads, B * 2); z selects tiled Q (even) or K
// (odd); pooled is [2][B][heads][n_tiles][d], counts gets the real rows per tile.
// MOVE = true: the tile permute with the pool folded in. grid (n_tiles, heads,
// B); q is the natural-order tensor [B, n_tokens, heads, d]; every row read is
// also written to its tiled position in `tiled` (pad rows as zeros; no copy
// when tiled is null), pooled is [B][heads][n_tiles][d]. Both forms give each thread the same rows and
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
    // rows rg, rg + groups, ... summed in increasing order; kRowBatch rows'
    // loads are issued before any of them is stored or summed
    for (int r0 = rg; r0 < L.C; r0 += kRowBatch * groups) {
      uint4 w[kRowBatch];
      bool real[kRowBatch];
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) {
        const int r = r0 + u * groups;
        real[u] = false;
        if (r >= L.C) continue;
        if (MOVE) {
          const int nat = natural_index(L, tile, r);
          real[u] = nat >= 0;
          if (real[u]) w[u] = x[(((long long)b * L.n_tokens + nat) * L.heads + head) * chunks + ch];
        } else {
          real[u] = row_is_real(L, tv, r);
          if (real[u]) w[u] = x[(row0 + r) * chunks + ch];
        }
      }
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) {
        const int r = r0 + u * groups;
        if (r >= L.C) break;
        if (MOVE && tiled) tiled[(row0 + r) * chunks + ch] = real[u] ? w[u] : make_uint4(0u, 0u, 0u, 0u);
        if (!real[u]) continue;
        const uint32_t ws[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += __uint_as_float(ws[e] << 16);
          acc[2 * e + 1] += __uint_as_float(ws[e] & 0xFFFF0000u);
        }
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
  if (!MOVE && counts && threadIdx.x == 0 && which == 0 && b == 0 && head == 0) counts[tile] = n;
}

// ---------------------------------------------------------------- route
// Order-preserving 32-bit key of a float: a larger float gives a larger key.
__device__ __forceinline__ uint32_t float_order(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Coarse scores and selection fused, one workgroup per (b, head, R query
// tiles): the R rows of scores stay in LDS (R * n_tiles floats), so no
// n_tiles^2 buffer exists. Scores first (all 256 threads), then each wave
// selects for its rows from LDS on its own, with no barrier.
//
// Scores: s_ij = coarse_scale * <qbar_i, kbar_j> on the fp32 matrix core
// (v_mfma_f32_16x16x4_f32, products of 16 query tiles x 16 key tiles, 4
// channels per step, fp32 accumulation in a fixed order), -inf for key tiles
// without real tokens. Each lane holds its qbar operands for the whole row
// block in registers and loads its kbar operands straight from memory, one
// block of 16 key tiles ahead; the 8 waves take the key blocks in turn.
//
// Selection of row i among the real key tiles, by (score desc, index asc):
// lane l holds tiles l, l + 64, ...; each tile's 32-bit order key (larger
// score, larger key) is compared against a threshold found by a 32-step
// binary search, bit by bit from the top:
//   top-k : T = the largest key with #(key >= T) >= k' (k' = min(k, #real));
//   top-p : e_j = exp2((s_j - smax) * log2 e), Z = sum e_j, and
//           T = the largest key with mass(key >= T) >= top_p * Z, where the
//           mass of a key set is a fixed-order sum (per lane in increasing j,
//           then a butterfly over the lanes); then the count is raised to
//           k_floor (capped at #real) by a count search as for top-k.
// Tiles with key > T are kept; among tiles with key == T (equal scores) the
// lower indices are kept first, as many as the count (or the mass) needs.
// The kept tiles are written in ascending order through ballots.
constexpr int kRouteThreads = 512;        // 8 waves
constexpr int kRouteMaxK = 64;            // channel groups of 4 (head_dim <= 256)
constexpr int kRouteRow = 132;            // LDS floats per staged kbar row (128 channels + 4 pad)
typedef float f32x4v __attribute__((ext_vector_type(4)));

// Wave-wide sum / max, the same value in every lane and the same order on
// every call: within each row of 16 lanes by DPP (lane pairs, quads, half
// rows, rows), then the four row results in a fixed order.
template <int OP>   // 0: sum, 1: max, 2: min
__device__ __forceinline__ float wave_reduce(float x) {
  auto op = [](float a, float b) { return OP == 1 ? fmaxf(a, b) : OP == 2 ? fminf(a, b) : a + b; };
  auto dpp = [](float v, int ctrl) -> float {
    switch (ctrl) {
      case 0: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
      case 1: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
      case 2: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
      default: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
    }
  };
  x = op(x, dpp(x, 0));   // quad_perm [1,0,3,2]
  x = op(x, dpp(x, 1));   // quad_perm [2,3,0,1]
  x = op(x, dpp(x, 2));   // row_half_mirror
  x = op(x, dpp(x, 3));   // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return op(op(r0, r1), op(r2, r3));
}
__device__ __forceinline__ float wave_sum(float x) { return wave_reduce<0>(x); }
__device__ __forceinline__ float wave_max(float x) { return wave_reduce<1>(x); }
__device__ __forceinline__ float wave_min(float x) { return wave_reduce<2>(x); }

template <int R, int MT, int KG>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(DevLayout L, const float* __restrict__ q_pooled,
                                                              const float* __restrict__ k_pooled,
                                                              float coarse_scale, int top_k, float top_p,
                                                              int k_floor, int max_kv,
                                                              int32_t* __restrict__ kv_idx,
                                                              int32_t* __restrict__ kv_cnt,
                                                              float* __restrict__ scores) {
  static_assert(R == 4 || R == 8 || R == 16, "4, 8 or 16 query tiles per workgroup");
  extern __shared__ float sc[];                     // [R][n] scores of this workgroup's rows, then
                                                    // each wave's [16][kRouteRow] kbar staging
  const int n = L.n_tiles, d = L.d;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int i0 = blockIdx.x * R;
  const int rows = min(R, n - i0);
  const long long bh = (long long)blockIdx.z * L.heads + blockIdx.y;
  const float* qb = q_pooled + bh * n * d;
  const float* kb = k_pooled + bh * n * d;

  // A operand (16 x 4 per step): lane l holds qbar[i0 + l % 16][4 ks + l / 16]
  // (zero past the block's rows); B operand: kbar[j0 + l % 16][4 ks + l / 16],
  // read from the wave's own LDS copy of the block's 16 rows of kbar, which
  // the wave fills 128 channels at a time with coalesced 16-byte loads (the
  // next chunk's loads are in flight while the current one is used).
  const int m16 = lane & 15, k4 = lane >> 4;
  float qa[KG];
#pragma unroll
  for (int ks = 0; ks < KG; ++ks)
    qa[ks] = (m16 < rows && 4 * ks < d) ? qb[(long long)(i0 + m16) * d + 4 * ks + k4] : 0.0f;
  float* kS = sc + R * n + wave * (16 * kRouteRow);      // this wave's [16][kRouteRow] floats
  const int nblk = (n + 15) / 16;
  const int nch = (d + 127) / 128;                          // 128-channel chunks per row
  constexpr int NW = kRouteThreads / 64;
  float4 kr[8];
  // chunk q of this wave's work: block wave + NW * (q / nch), channels 128 * (q % nch) ..
  auto load_chunk = [&](int q) {
    const int blk = wave + NW * (q / nch), c0 = 128 * (q % nch);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = 64 * u + lane, jj = c >> 5, e = c0 + 4 * (c & 31);
      const int j = min(16 * blk + jj, n - 1);
      kr[u] = e < d ? *reinterpret_cast<const float4*>(kb + (long long)j * d + e) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  const int my_blocks = wave < nblk ? (nblk - wave + NW - 1) / NW : 0;
  const int nq = my_blocks * nch;
  if (nq > 0) load_chunk(0);
  f32x4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int q = 0; q < nq; ++q) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = 64 * u + lane;
      *reinterpret_cast<float4*>(kS + (c >> 5) * kRouteRow + 4 * (c & 31)) = kr[u];
    }
    if (q + 1 < nq) load_chunk(q + 1);
    const int cq = q % nch;
    if (cq == 0) acc = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < 32; ++kk) {
      const int ks = 32 * cq + kk;
      if (ks < KG && 4 * ks < d)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[ks], kS[m16 * kRouteRow + 4 * kk + k4], acc, 0, 0, 0);
    }
    if (cq == nch - 1) {
      // lane l holds rows 4 (l / 16) .. +3 of key tile 16 blk + l % 16
      const int blk = wave + NW * (q / nch);
      const int j = 16 * blk + m16;
      if (j < n) {
        const bool real = real_rows(L, tile_valid(L, j)) > 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int r = 4 * k4 + t;
          if (r >= rows) continue;
          const float v = real ? coarse_scale * acc[t] : -INFINITY;
          sc[r * n + j] = v;
          if (scores) scores[(bh * n + i0 + r) * n + j] = v;
        }
      }
    }
  }
  __syncthreads();

  const unsigned long long below = (1ull << lane) - 1ull;
  for (int r = wave; r < rows; r += kRouteThreads / 64) {
    const int i = i0 + r;
    int32_t* out_idx = kv_idx + (bh * n + i) * max_kv;
    if (real_rows(L, tile_valid(L, i)) == 0) {    // query tile without real tokens
      if (lane == 0) kv_cnt[bh * n + i] = 0;
      continue;
    }
    uint32_t key[MT];
    float sv[MT];
    int n_valid = 0;
    float smax = -INFINITY, smin = INFINITY;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int j = lane + 64 * m;
      const bool valid = j < n && real_rows(L, tile_valid(L, j)) > 0;
      sv[m] = valid ? sc[r * n + j] : -INFINITY;
      key[m] = valid ? float_order(sv[m]) : 0u;
      n_valid += __popcll(__ballot(valid));
      smax = fmaxf(smax, sv[m]);
      smin = valid ? fminf(smin, sv[m]) : smin;
    }
    smax = wave_max(smax);
    smin = wave_min(smin);
    if (n_valid == 0 || (top_p <= 0.0f && top_k <= 0)) {
      if (lane == 0) kv_cnt[bh * n + i] = 0;
      continue;
    }
    // counts of real tiles with key >= t / key > t, and the threshold search by counts
    auto count_ge = [&](uint32_t t) {
      int c = 0;
#pragma unroll
      for (int m = 0; m < MT; ++m) c += __popcll(__ballot(key[m] >= t && key[m] != 0u));
      return c;
    };
    auto count_gt = [&](uint32_t t) { return t == 0xFFFFFFFFu ? 0 : count_ge(t + 1u); };
    // Every threshold searched for lies in [key of smin, key of smax], so it
    // shares their common leading bits; the search runs over the bits below.
    const uint32_t kmax = float_order(smax), kmin = float_order(smin);
    const int hb = (kmin ^ kmax) ? 31 - __builtin_clz(kmin ^ kmax) : -1;
    const uint32_t T0 = hb < 0 ? kmax : hb == 31 ? 0u : kmax & ~((2u << hb) - 1u);
    auto search = [&](auto pred) {              // largest T in range with pred(T)
      uint32_t T = T0;
      for (int bit = hb; bit >= 0; --bit) {
        const uint32_t cand = T | (1u << bit);
        if (pred(cand)) T = cand;
      }
      return T;
    };
    auto search_count = [&](int want) {         // largest T with #(key >= T) >= want (want >= 1)
      return search([&](uint32_t t) { return count_ge(t) >= want; });
    };
    int count;
    uint32_t T;
    int need_tied;                               // tiles with key == T to keep, lowest indices first
    if (top_p > 0.0f) {
      float ev[MT];
      float zl = 0.0f;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        ev[m] = key[m] != 0u ? exp2f((sv[m] - smax) * 1.4426950408889634f) : 0.0f;
        zl += ev[m];
      }
      const float target = top_p * wave_sum(zl);
      auto mass_ge = [&](uint32_t t) {
        float ms = 0.0f;
#pragma unroll
        for (int m = 0; m < MT; ++m) ms += key[m] >= t ? ev[m] : 0.0f;
        return wave_sum(ms);
      };
      T = search([&](uint32_t t) { return mass_ge(t) >= target; });
      // the crossing key T: keys above it, then tied tiles in index order until the mass is reached
      const int above = count_gt(T);
      const int tied = count_ge(T) - above;
      need_tied = tied;
      if (tied > 1) {
        float cum = T == 0xFFFFFFFFu ? 0.0f : mass_ge(T + 1u);
        need_tied = 0;
        for (int m = 0; m < MT && cum < target; ++m) {
          const unsigned long long tm = __ballot(key[m] == T);
          for (unsigned long long bits = tm; bits && cum < target; bits &= bits - 1) {
            const int src = __builtin_ctzll(bits);
            cum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ev[m]), src));
            ++need_tied;
          }
        }
      }
      count = above + need_tied;
      if (count < k_floor && count < n_valid) {
        count = min(k_floor, n_valid);
        T = search_count(count);
        need_tied = count - count_gt(T);
      }
    } else {
      count = min(top_k, n_valid);
      T = search_count(count);
      need_tied = count - count_gt(T);
    }
    // write the kept tiles in ascending order
    int base = 0, tied_seen = 0;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const bool is_tied = key[m] == T && key[m] != 0u;
      const unsigned long long tmask = __ballot(is_tied);
      const int trank = tied_seen + __popcll(tmask & below);
      tied_seen += __popcll(tmask);
      const bool keep = key[m] != 0u && (key[m] > T || (is_tied && trank < need_tied));
      const unsigned long long kmask = __ballot(keep);
      if (keep) out_idx[base + __popcll(kmask & below)] = lane + 64 * m;
      base += __popcll(kmask);
    }
    if (lane == 0) kv_cnt[bh * n + i] = count;
  }
}

// R query tiles per workgroup (scores of the rows in LDS: R * n * 4 bytes),
// MT key tiles per lane in the selection, KG channel groups of 4.
template <int R, int MT>
static hipError_t launch_route_rm(const DevLayout& L, const float* qp, const float* kp, float coarse_scale,
                                  int top_k, float top_p, int k_floor, int max_kv, int32_t* kv_idx,
                                  int32_t* kv_cnt, float* scores, hipStream_t s) {
  const size_t lds = ((size_t)R * L.n_tiles + (kRouteThreads / 64) * 16 * kRouteRow) * sizeof(float);
  dim3 grid((L.n_tiles + R - 1) / R, L.heads, L.B);
  if (L.d <= 128)
    hipLaunchKernelGGL((route_kernel<R, MT, 32>), grid, dim3(kRouteThreads), lds, s, L, qp, kp,
                       coarse_scale, top_k, top_p, k_floor, max_kv, kv_idx, kv_cnt, scores);
  else
    hipLaunchKernelGGL((route_kernel<R, MT, kRouteMaxK>), grid, dim3(kRouteThreads), lds, s, L, qp, kp,
                       coarse_scale, top_k, top_p, k_floor, max_kv, kv_idx, kv_cnt, scores);
  return hipGetLastError();
}

static hipError_t route_from_pooled(const DevLayout& L, const float* qp, const float* kp,
                                    float coarse_scale, int top_k, float top_p, int k_floor,
                                    int max_kv, int32_t* kv_idx, int32_t* kv_cnt, float* scores,
                                    hipStream_t s) {
  const int n = L.n_tiles;
  if (n <= 256)
    return launch_route_rm<16, 4>(L, qp, kp, coarse_scale, top_k, top_p, k_floor, max_kv, kv_idx, kv_cnt, scores, s);
  // LDS: R * n * 4 bytes of scores + 8 waves x 16 rows x 132 floats of staging (66 KB) <= 160 KB
  if (n <= 1504)
    return launch_route_rm<16, 24>(L, qp, kp, coarse_scale, top_k, top_p, k_floor, max_kv, kv_idx, kv_cnt, scores, s);
  if (n <= 3008)
    return launch_route_rm<8, 48>(L, qp, kp, coarse_scale, top_k, top_p, k_floor, max_kv, kv_idx, kv_cnt, scores, s);
  return launch_route_rm<4, 64>(L, qp, kp, coarse_scale, top_k, top_p, k_floor, max_kv, kv_idx, kv_cnt, scores, s);
}

}  // namespace

size_t route_workspace_bytes(const DevLayout& L) {
  return 2ull * L.B * L.heads * L.n_tiles * L.d * sizeof(float);
}

hipError_t launch_route(const DevLayout& L, const void* q, const void* k, float coarse_scale,
                        int top_k, float top_p, int k_floor, int max_kv, int32_t* kv_idx,
                        int32_t* kv_cnt, float* scores, void* ws, hipStream_t s) {
  float* pooled = static_cast<float*>(ws);
  hipLaunchKernelGGL(pool_kernel<false>, dim3(L.n_tiles, L.heads, L.B * 2), dim3(kThreads), 0, s,
                     L, static_cast<const uint4*>(q), static_cast<const uint4*>(k), nullptr,
                     pooled, nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t per = (size_t)L.B * L.heads * L.n_tiles * L.d;
  return route_from_pooled(L, pooled, pooled + per, coarse_scale, top_k, top_p, k_floor, max_kv,
                           kv_idx, kv_cnt, scores, s);
}

hipError_t launch_route_pooled(const DevLayout& L, const float* q_pooled, const float* k_pooled,
                               float coarse_scale, int top_k, float top_p, int k_floor, int max_kv,
                               int32_t* kv_idx, int32_t* kv_cnt, float* scores, hipStream_t s) {
  return route_from_pooled(L, q_pooled, k_pooled, coarse_scale, top_k, top_p, k_floor, max_kv,
                           kv_idx, kv_cnt, scores, s);
}

hipError_t launch_permute_pool(const DevLayout& L, const void* src, void* dst, float* pooled,
                               hipStream_t s) {
  hipLaunchKernelGGL(pool_kernel<true>, dim3(L.n_tiles, L.heads, L.B), dim3(kThreads), 0, s, L,
                     static_cast<const uint4*>(src), nullptr, static_cast<uint4*>(dst), pooled,
                     nullptr);
  return hipGetLastError();
}

}  // namespace vsa
