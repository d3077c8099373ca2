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
// CT, DT: tile tokens and head_dim fixed at compile time (0: taken from L).
template <bool MOVE, int CT = 0, int DT = 0>
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
  const int C = CT ? CT : L.C, d = DT ? DT : L.d;
  const int chunks = d >> 3;                         // 8 bf16 per chunk
  const int groups = kThreads / chunks;              // row groups summed in parallel
  const int ch = threadIdx.x % chunks;
  const int rg = threadIdx.x / chunks;
  const long long row0 = (long long)(b * L.heads + head) * L.n_padded + (long long)tile * C;
  const TileValid tv = tile_valid(L, tile);

  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  if (rg < groups) {
    // rows rg, rg + groups, ... summed in increasing order; kRowBatch rows'
    // loads are issued before any of them is stored or summed
    for (int r0 = rg; r0 < C; r0 += kRowBatch * groups) {
      uint4 w[kRowBatch];
      bool real[kRowBatch];
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) {
        const int r = r0 + u * groups;
        real[u] = false;
        if (r >= C) continue;
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
        if (r >= C) break;
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
  for (int c = threadIdx.x; c < d; c += kThreads) {
    const int cch = c >> 3, ce = c & 7;
    float s = 0.0f;
    for (int g = 0; g < groups; ++g) s += part[(g * chunks + cch) * 8 + ce];
    pooled[out0 * d + c] = n > 0 ? s / (float)n : 0.0f;
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
// n_tiles^2 buffer exists. Scores first (all waves), then each wave
// selects for its rows from LDS on its own, with no barrier.
//
// Scores: s_ij = coarse_scale * <qbar_i, kbar_j> on the fp32 matrix core
// (v_mfma_f32_16x16x4_f32, products of 16 query tiles x 16 key tiles, 4
// channels per step, fp32 accumulation in a fixed order), -inf for key tiles
// without real tokens. The channel that lane group g of step t contracts is
// chosen so that each lane's operands for four consecutive steps are four
// consecutive channels: the kbar operands then come straight from memory as
// one 16-byte load per lane and four steps, with no staging through LDS, and
// the qbar operands of the same channels stay in registers for the whole
// row block. The waves take the key blocks in turn, loading each block two
// blocks before it is multiplied. The key tiles' real-token flags are taken
// once per workgroup, not per row.
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
// Once at most 64 tiles remain between the decided bits (checked every
// fourth bit) they are gathered one per lane and the remaining bits test one
// value per lane; a mass is then the gathered tiles' fixed-order sum added to
// the mass of the tiles above them. Tiles with key > T are kept; among tiles with key == T
// (equal scores) the lower indices are kept first, as many as the count (or
// the mass) needs.
// The kept tiles are written in ascending order through ballots.
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

// FULL: d == 128 * NCH, so every channel step is real and the loads and
// products need no per-step test.
template <int R, int MT, int NCH, int THREADS, bool FULL>
__global__ __launch_bounds__(THREADS) void route_kernel(DevLayout L, const float* __restrict__ q_pooled,
                                                              const float* __restrict__ k_pooled,
                                                              float coarse_scale, int top_k, float top_p,
                                                              int k_floor, int max_kv,
                                                              int32_t* __restrict__ kv_idx,
                                                              int32_t* __restrict__ kv_cnt,
                                                              float* __restrict__ scores) {
  static_assert(R == 4 || R == 8 || R == 16, "4, 8 or 16 query tiles per workgroup");
  extern __shared__ float sc[];                     // [R][n] scores of this workgroup's rows
  const int n = L.n_tiles, d = L.d;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int i0 = blockIdx.x * R;
  const int rows = min(R, n - i0);
  const long long bh = (long long)blockIdx.z * L.heads + blockIdx.y;
  const float* qb = q_pooled + bh * n * d;
  const float* kb = k_pooled + bh * n * d;

  // Step t (0..31) of channel chunk cq: lane l (m16 = l % 16, g = l / 16)
  // contracts channel 128 cq + 16 (t / 4) + 4 g + t % 4 of query tile
  // i0 + m16 (A operand) and of key tile j0 + m16 (B operand); channels past
  // d are zero on both sides.
  constexpr int NW = THREADS / 64;
  const int m16 = lane & 15, k4 = lane >> 4;
  float qa[NCH][32];
#pragma unroll
  for (int cq = 0; cq < NCH; ++cq)
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = 128 * cq + 16 * u + 4 * k4;
      const float4 v = (m16 < rows && (FULL || e < d))
                           ? *reinterpret_cast<const float4*>(qb + (long long)(i0 + m16) * d + e)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
      qa[cq][4 * u + 0] = v.x;
      qa[cq][4 * u + 1] = v.y;
      qa[cq][4 * u + 2] = v.z;
      qa[cq][4 * u + 3] = v.w;
    }
  const int nblk = (n + 15) / 16;
  auto load_blk = [&](int blk, float4 (&kr)[NCH][8]) {
    const int j = min(16 * blk + m16, n - 1);
#pragma unroll
    for (int cq = 0; cq < NCH; ++cq)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = 128 * cq + 16 * u + 4 * k4;
        if constexpr (FULL) kr[cq][u] = *reinterpret_cast<const float4*>(kb + (long long)j * d + e);
        else kr[cq][u] = e < d ? *reinterpret_cast<const float4*>(kb + (long long)j * d + e) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
  };
  auto score_blk = [&](int blk, const float4 (&kr)[NCH][8]) {
    f32x4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int cq = 0; cq < NCH; ++cq)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (!FULL && 128 * cq + 16 * u >= d) continue;
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[cq][4 * u + 0], kr[cq][u].x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[cq][4 * u + 1], kr[cq][u].y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[cq][4 * u + 2], kr[cq][u].z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[cq][4 * u + 3], kr[cq][u].w, acc, 0, 0, 0);
      }
    // lane l holds rows 4 (l / 16) .. +3 of key tile 16 blk + l % 16; the
    // selection masks key tiles without real tokens itself, so only the
    // optional score output needs the -inf
    const int j = 16 * blk + m16;
    if (j < n) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = 4 * k4 + t;
        if (r < rows) sc[r * n + j] = coarse_scale * acc[t];
      }
      if (scores) {
        const bool real = real_rows(L, tile_valid(L, j)) > 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int r = 4 * k4 + t;
          if (r < rows) scores[(bh * n + i0 + r) * n + j] = real ? coarse_scale * acc[t] : -INFINITY;
        }
      }
    }
  };
  {
    // three block buffers: the loads of a block are issued two blocks ahead
    float4 ka[NCH][8], kc[NCH][8], ke[NCH][8];
    int blk = wave;
    if (blk < nblk) load_blk(blk, ka);
    if (blk + NW < nblk) load_blk(blk + NW, kc);
    while (blk < nblk) {
      if (blk + 2 * NW < nblk) load_blk(blk + 2 * NW, ke);
      score_blk(blk, ka);
      blk += NW;
      if (blk >= nblk) break;
      if (blk + 2 * NW < nblk) load_blk(blk + 2 * NW, ka);
      score_blk(blk, kc);
      blk += NW;
      if (blk >= nblk) break;
      if (blk + 2 * NW < nblk) load_blk(blk + 2 * NW, kc);
      score_blk(blk, ke);
      blk += NW;
    }
  }
  __syncthreads();

  const unsigned long long below = (1ull << lane) - 1ull;
  // which of this lane's key tiles hold real tokens (the same for every row)
  unsigned long long vbits = 0ull;
  int n_valid = 0;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int j = lane + 64 * m;
    const bool valid = j < n && real_rows(L, tile_valid(L, j)) > 0;
    vbits |= (unsigned long long)valid << m;
    n_valid += __popcll(__ballot(valid));
  }
  for (int r = wave; r < rows; r += THREADS / 64) {
    const int i = i0 + r;
    int32_t* out_idx = kv_idx + (bh * n + i) * max_kv;
    if (real_rows(L, tile_valid(L, i)) == 0) {    // query tile without real tokens
      if (lane == 0) kv_cnt[bh * n + i] = 0;
      continue;
    }
    uint32_t key[MT];
    float sv[MT];
    float smax = -INFINITY, smin = INFINITY;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const bool valid = (vbits >> m) & 1ull;
      sv[m] = valid ? sc[r * n + lane + 64 * m] : -INFINITY;
      key[m] = valid ? float_order(sv[m]) : 0u;
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
    auto count_ge = [&](uint32_t t) __attribute__((always_inline)) {
      int c = 0;
#pragma unroll
      for (int m = 0; m < MT; ++m) c += __popcll(__ballot(key[m] >= t && key[m] != 0u));
      return c;
    };
    auto count_gt = [&](uint32_t t) __attribute__((always_inline)) { return t == 0xFFFFFFFFu ? 0 : count_ge(t + 1u); };
    // Every threshold searched for lies in [key of smin, key of smax], so it
    // shares their common leading bits; the search runs over the bits below.
    const uint32_t kmax = float_order(smax), kmin = float_order(smin);
    const int hb = (kmin ^ kmax) ? 31 - __builtin_clz(kmin ^ kmax) : -1;
    const uint32_t T0 = hb < 0 ? kmax : hb == 31 ? 0u : kmax & ~((2u << hb) - 1u);
    // The largest T in that range with weight(key >= T) >= goal, bit by bit
    // from the top (weight: the tiles' masses, or 1 each for counts). Once
    // at most 64 tiles are left whose keys share T's decided leading bits
    // (checked every fourth bit), they are gathered one per lane through this
    // row's LDS slots, whose scores are already in registers; the tiles
    // above that range add their weight once, and the remaining bits test
    // one value per lane.
    uint32_t* gk = reinterpret_cast<uint32_t*>(sc + r * n);   // gathered keys (64), then weights (64)
    float* gw = sc + r * n + 64;
    auto search = [&](auto weight_ge, auto weight_of, float goal) __attribute__((always_inline)) {
      uint32_t T = T0;
      int bit = hb;
      for (; bit >= 0; --bit) {
        if (MT > 4 && ((hb - bit) & 3) == 0) {
          const uint32_t pre = bit == 31 ? 0u : ~((2u << bit) - 1u);
          int left = 0;
#pragma unroll
          for (int m = 0; m < MT; ++m) left += __popcll(__ballot(key[m] != 0u && (key[m] & pre) == (T & pre)));
          if (left <= 64) break;
        }
        const uint32_t cand = T | (1u << bit);
        if (weight_ge(cand) >= goal) T = cand;
      }
      if (bit < 0) return T;
      const uint32_t pre = bit == 31 ? 0u : ~((2u << bit) - 1u);
      float above = 0.0f;
      int base = 0;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const bool in = key[m] != 0u && (key[m] & pre) == (T & pre);
        above += (key[m] != 0u && (key[m] & pre) > (T & pre)) ? weight_of(m) : 0.0f;
        const unsigned long long msk = __ballot(in);
        if (in) {
          const int p = base + __popcll(msk & below);
          gk[p] = key[m];
          gw[p] = weight_of(m);
        }
        base += __popcll(msk);
      }
      const float A = wave_sum(above);
      __builtin_amdgcn_wave_barrier();
      const bool have = lane < base;
      const uint32_t ck = have ? gk[lane] : 0u;
      const float cw = have ? gw[lane] : 0.0f;
      for (; bit >= 0; --bit) {
        const uint32_t cand = T | (1u << bit);
        if (A + wave_sum(have && ck >= cand ? cw : 0.0f) >= goal) T = cand;
      }
      __builtin_amdgcn_wave_barrier();
      return T;
    };
    auto search_count = [&](int want) __attribute__((always_inline)) {   // largest T with #(key >= T) >= want (want >= 1)
      return search([&](uint32_t t) __attribute__((always_inline)) { return (float)count_ge(t); },
                    [&](int) __attribute__((always_inline)) { return 1.0f; }, (float)want);
    };
    int count;
    uint32_t T;
    int need_tied;                               // tiles with key == T to keep, lowest indices first
    int n_tied;                                  // tiles with key == T
    if (top_p > 0.0f) {
      float ev[MT];
      float zl = 0.0f;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        ev[m] = key[m] != 0u ? exp2f((sv[m] - smax) * 1.4426950408889634f) : 0.0f;
        zl += ev[m];
      }
      const float target = top_p * wave_sum(zl);
      auto mass_ge = [&](uint32_t t) __attribute__((always_inline)) {
        float ms = 0.0f;
#pragma unroll
        for (int m = 0; m < MT; ++m) ms += key[m] >= t ? ev[m] : 0.0f;
        return wave_sum(ms);
      };
      T = search(mass_ge, [&](int m) __attribute__((always_inline)) { return ev[m]; }, target);
      // the crossing key T: keys above it, then tied tiles in index order until the mass is reached
      const int above = count_gt(T);
      const int tied = count_ge(T) - above;
      need_tied = tied;
      n_tied = tied;
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
        const int gt = count_gt(T);
        need_tied = count - gt;
        n_tied = count_ge(T) - gt;
      }
    } else {
      count = min(top_k, n_valid);
      T = search_count(count);
      const int gt = count_gt(T);
      need_tied = count - gt;
      n_tied = count_ge(T) - gt;
    }
    // write the kept tiles in ascending order; when every tile at the
    // threshold is kept (the common case) no tie ranks are needed
    int base = 0, tied_seen = 0;
    if (need_tied == n_tied) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const bool keep = key[m] != 0u && key[m] >= T;
        const unsigned long long kmask = __ballot(keep);
        if (keep) out_idx[base + __popcll(kmask & below)] = lane + 64 * m;
        base += __popcll(kmask);
      }
    } else
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
// MT key tiles per lane in the selection, NCH chunks of 128 channels.
template <int R, int MT, int NCH, int THREADS>
static hipError_t launch_route_rm(const DevLayout& L, const float* qp, const float* kp, float coarse_scale,
                                  int top_k, float top_p, int k_floor, int max_kv, int32_t* kv_idx,
                                  int32_t* kv_cnt, float* scores, hipStream_t s) {
  const size_t lds = (size_t)R * L.n_tiles * sizeof(float);
  dim3 grid((L.n_tiles + R - 1) / R, L.heads, L.B);
  if (L.d == 128 * NCH)
    hipLaunchKernelGGL((route_kernel<R, MT, NCH, THREADS, true>), grid, dim3(THREADS), lds, s, L, qp, kp,
                       coarse_scale, top_k, top_p, k_floor, max_kv, kv_idx, kv_cnt, scores);
  else
    hipLaunchKernelGGL((route_kernel<R, MT, NCH, THREADS, false>), grid, dim3(THREADS), lds, s, L, qp, kp,
                       coarse_scale, top_k, top_p, k_floor, max_kv, kv_idx, kv_cnt, scores);
  return hipGetLastError();
}

// Rows per workgroup and key tiles per lane by n_tiles (LDS: R * n * 4 <= 160 KB);
// sixteen waves where the registers allow (head_dim <= 128, up to 1,536 tiles), else eight.
template <int NCH, int TH>
static hipError_t route_by_n(const DevLayout& L, const float* qp, const float* kp, float coarse_scale,
                             int top_k, float top_p, int k_floor, int max_kv, int32_t* kv_idx,
                             int32_t* kv_cnt, float* scores, hipStream_t s) {
  const int n = L.n_tiles;
  if (n <= 256)
    return launch_route_rm<16, 4, NCH, TH>(L, qp, kp, coarse_scale, top_k, top_p, k_floor, max_kv, kv_idx, kv_cnt, scores, s);
  if (n <= 1536)
    return launch_route_rm<16, 24, NCH, TH>(L, qp, kp, coarse_scale, top_k, top_p, k_floor, max_kv, kv_idx, kv_cnt, scores, s);
  if (n <= 2560)
    return launch_route_rm<16, 48, NCH, 512>(L, qp, kp, coarse_scale, top_k, top_p, k_floor, max_kv, kv_idx, kv_cnt, scores, s);
  return launch_route_rm<8, 64, NCH, 512>(L, qp, kp, coarse_scale, top_k, top_p, k_floor, max_kv, kv_idx, kv_cnt, scores, s);
}

static hipError_t route_from_pooled(const DevLayout& L, const float* qp, const float* kp,
                                    float coarse_scale, int top_k, float top_p, int k_floor,
                                    int max_kv, int32_t* kv_idx, int32_t* kv_cnt, float* scores,
                                    hipStream_t s) {
  if (L.d <= 128)
    return route_by_n<1, 512>(L, qp, kp, coarse_scale, top_k, top_p, k_floor, max_kv, kv_idx, kv_cnt, scores, s);
  return route_by_n<2, 512>(L, qp, kp, coarse_scale, top_k, top_p, k_floor, max_kv, kv_idx, kv_cnt, scores, s);
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
  const dim3 grid(L.n_tiles, L.heads, L.B);
  const uint4* sp = static_cast<const uint4*>(src);
  if (L.C == 64 && L.d == 128)
    hipLaunchKernelGGL((pool_kernel<true, 64, 128>), grid, dim3(kThreads), 0, s, L, sp, nullptr,
                       static_cast<uint4*>(dst), pooled, nullptr);
  else
    hipLaunchKernelGGL((pool_kernel<true>), grid, dim3(kThreads), 0, s, L, sp, nullptr,
                       static_cast<uint4*>(dst), pooled, nullptr);
  return hipGetLastError();
}

}  // namespace vsa
