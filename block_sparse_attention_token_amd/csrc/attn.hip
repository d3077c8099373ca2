// S6: block-sparse attention forward, bf16 MFMA (f32 inputs are rounded to
// bf16 at load). This is the flash-style, FlashAttention-compatible sparse
// attention the pages build on (OSP-Next wiki TL;DR and card "Model
// Summary"; FPSAttention "Approach"; VSA Research Type row; FVAttn summary):
// each query tile visits only the key/value tiles of its list, with an
// online softmax.
//
// gfx950 mapping (one wavefront = one query tile of 32 or 64 rows, in 32-row
// groups):
//   S^T = K . Q^T   v_mfma_f32_32x32x16_bf16, A = K rows (LDS), B = Q^T (registers)
//   O^T += V^T . P^T  same instruction, A = V^T rows (LDS), B = P^T (registers)
// Computing the transposed products leaves every lane holding one query
// row (lane % 32) of S^T, P^T and O^T, so the softmax statistics, the
// rescale and the final normalisation are lane-local; the only cross-lane
// step is one max exchange between the two half-waves per kv tile.
// The PV contraction runs over kv tokens in the order the S^T accumulator
// holds them; V^T is written to LDS in that same token order, so P never
// moves between lanes.
//
// Work shapes:
//   WAVES == 1: one wave per query tile, walking that tile's own list
//               (routed masks, where neighbouring tiles share little);
//   WAVES == 4: four waves = four consecutive query tiles; the workgroup
//               walks the union of their lists once, loading each K/V tile
//               into LDS once for all four (dense, Skiparse-2D and window
//               lists, where neighbours share most of their tiles). A wave
//               whose list lacks the current tile skips its math.
// The softmax uses a lazy rescale: the running maximum a wave subtracts is
// only raised when a new score exceeds it by more than 2^8 (in exp2 units),
// so O^T is rarely rescaled.
#include <float.h>

#include "vsa_internal.h"

namespace vsa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLazyThreshold = 8.0f;   // log2 of the largest unnormalised p kept

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// 8 consecutive elements at element offset `off` as 8 bf16 in a uint4.
template <bool F32IN>
__device__ __forceinline__ uint4 load8(const void* base, long long off) {
  if constexpr (F32IN) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    const float4 x = p[0], y = p[1];
    return make_uint4(pack_bf16(x.x, x.y), pack_bf16(x.z, x.w), pack_bf16(y.x, y.y),
                      pack_bf16(y.z, y.w));
  } else {
    return *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
  }
}
__device__ __forceinline__ uint32_t perm_lo(uint32_t a, uint32_t b) {   // lo16(a) | lo16(b) << 16
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t perm_hi(uint32_t a, uint32_t b) {   // hi16(a) | hi16(b) << 16
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

template <int TILE, int D, int WAVES, bool F32IN>
struct AttnCfg {
  static constexpr int QG = TILE / 32;         // 32-row query groups per wave (one tile)
  static constexpr int MB = TILE / 32;         // 32-token blocks of a kv tile
  static constexpr int KS = D / 16;            // QK^T k-steps over the head dim
  static constexpr int CB = D / 32;            // 32-channel blocks of O^T
  static constexpr int PS = TILE / 16;         // PV k-steps over kv tokens
  static constexpr int CPR_K = D / 8;          // 16-byte chunks per K row (bf16)
  static constexpr int CPR_V = TILE / 8;       // 16-byte chunks per V^T row
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int K_CHUNKS = TILE * CPR_K;
  static constexpr int K_PER_T = K_CHUNKS / THREADS;
  static constexpr int V_HALF = (TILE / 4) * (D / 8);   // 4-token x 8-channel pieces
  static constexpr int V_PER_T = (V_HALF + THREADS - 1) / THREADS;
  static_assert(TILE == 32 || TILE == 64, "tiles of 32 or 64 tokens");
  static_assert(K_CHUNKS % THREADS == 0, "K tile split");
};

// kv-token held in register r of S^T block mb by a lane of half-wave `half`
__device__ __forceinline__ int sacc_token(int mb, int r, int half) {
  return 32 * mb + 8 * (r >> 2) + 4 * half + (r & 3);
}

__device__ __forceinline__ int vt_swizzle(int c, int cpr) { return (c ^ (c >> 3)) & (cpr - 1); }

template <int TILE, int D, int WAVES, bool F32IN>
__global__ __launch_bounds__(64 * WAVES, 1) void attn_bf16_kernel(DevLayout L, AttnArgs a,
                                                                  int n_work, int qtiles_per_wg) {
  using Cfg = AttnCfg<TILE, D, WAVES, F32IN>;
  constexpr int QG = Cfg::QG, MB = Cfg::MB, KS = Cfg::KS, CB = Cfg::CB, PS = Cfg::PS;
  constexpr int CPR_K = Cfg::CPR_K, CPR_V = Cfg::CPR_V, THREADS = Cfg::THREADS;

  __shared__ uint4 k_lds[TILE * CPR_K];
  __shared__ uint4 v_lds[D * CPR_V];
  extern __shared__ int dyn[];                  // WAVES > 1: per-tile wave masks + schedule

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const int w = xcd_remap(blockIdx.x, n_work);
  const int wg_per_bh = (L.n_tiles + qtiles_per_wg - 1) / qtiles_per_wg;
  const int bh = w / wg_per_bh;
  const int qt0 = (w - bh * wg_per_bh) * qtiles_per_wg;
  const int qt = qt0 + wave;
  const bool wave_active = qt < L.n_tiles;
  const long long head_row0 = (long long)bh * L.n_padded;

  // ---- this wave's list
  const int32_t* my_list = nullptr;
  int my_cnt = 0;
  if (wave_active) {
    if (a.kv_idx) {
      const long long row = (a.list_mode ? (long long)bh * L.n_tiles : 0ll) + qt;
      my_list = a.kv_idx + row * a.max_kv;
      my_cnt = min(max(a.kv_cnt[row], 0), a.max_kv);
    } else {
      my_cnt = L.n_tiles;
    }
  }

  // ---- schedule: the ascending union of the waves' lists with a wave mask each
  int sched_len;
  int* sched = dyn + L.n_tiles;
  if constexpr (WAVES > 1) {
    int* marks = dyn;
    for (int t = tid; t < L.n_tiles; t += THREADS) marks[t] = 0;
    __syncthreads();
    for (int i = lane; i < my_cnt; i += 64) {
      const int t = my_list ? min(max(my_list[i], 0), L.n_tiles - 1) : i;
      atomicOr(&marks[t], 1 << wave);
    }
    __syncthreads();
    // compaction in tile order: each thread owns a contiguous run of tiles
    __shared__ int scan[THREADS];
    const int per = (L.n_tiles + THREADS - 1) / THREADS;
    const int lo = tid * per, hi = min(lo + per, L.n_tiles);
    int mine = 0;
    for (int t = lo; t < hi; ++t) mine += marks[t] != 0;
    scan[tid] = mine;
    __syncthreads();
    for (int off = 1; off < THREADS; off <<= 1) {
      const int add = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    int pos = scan[tid] - mine;
    sched_len = scan[THREADS - 1];
    for (int t = lo; t < hi; ++t)
      if (marks[t]) sched[pos++] = t | (marks[t] << 24);
    __syncthreads();
  } else {
    sched_len = my_cnt;
  }

  auto sched_tile = [&](int s) -> int {
    if constexpr (WAVES > 1) return sched[s] & 0xFFFFFF;
    else return my_list ? min(max(my_list[s], 0), L.n_tiles - 1) : s;
  };
  auto sched_mine = [&](int s) -> bool {
    if constexpr (WAVES > 1) return (sched[s] >> (24 + wave)) & 1;
    else return true;
  };

  // ---- Q^T fragments (B operand): lane holds query row 32*qg + l32, 8 channels
  uint4 qf[QG][KS];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const long long row = head_row0 + (long long)min(qt, L.n_tiles - 1) * TILE + 32 * qg + l32;
      qf[qg][ks] = load8<F32IN>(a.q, row * D + ks * 16 + half * 8);
    }

  f32x16_t oacc[CB][QG];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) oacc[cb][qg] = f32x16_t{};
  float m_run[QG], l_run[QG];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    m_run[qg] = -INFINITY;
    l_run[qg] = 0.0f;
  }

  // ---- tile loaders
  uint4 kreg[Cfg::K_PER_T];
  auto load_k = [&](int tile) {
    const long long base = (head_row0 + (long long)tile * TILE) * D;
#pragma unroll
    for (int i = 0; i < Cfg::K_PER_T; ++i) {
      const int c = tid + i * THREADS;
      const int r = c / CPR_K, ch = c % CPR_K;
      kreg[i] = load8<F32IN>(a.k, base + (long long)r * D + ch * 8);
    }
  };
  auto store_k = [&]() {
#pragma unroll
    for (int i = 0; i < Cfg::K_PER_T; ++i) {
      const int c = tid + i * THREADS;
      const int r = c / CPR_K, ch = c % CPR_K;
      k_lds[r * CPR_K + (ch ^ (r % CPR_K))] = kreg[i];
    }
  };
  // V piece u: 4 consecutive kv tokens x 8 channels (channel chunk cc,
  // quarter q4). Its 4 tokens go to V^T positions 4*q4 .. 4*q4+3, i.e. the
  // token order of the S^T accumulator (see sacc_token).
  uint4 vfull[Cfg::V_PER_T][4];
  auto load_v4 = [&](int tile) {
    const long long base = (head_row0 + (long long)tile * TILE) * D;
#pragma unroll
    for (int i = 0; i < Cfg::V_PER_T; ++i) {
      const int u = tid + i * THREADS;
      if (u < Cfg::V_HALF) {
        const int cc = u % (D / 8), q4 = u / (D / 8);
        const int pc = q4 >> 1;
        const int tok0 = 16 * (pc >> 1) + 4 * (pc & 1) + 8 * (q4 & 1);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          vfull[i][j] = load8<F32IN>(a.v, base + (long long)(tok0 + j) * D + cc * 8);
      }
    }
  };
  auto store_v = [&]() {
#pragma unroll
    for (int i = 0; i < Cfg::V_PER_T; ++i) {
      const int u = tid + i * THREADS;
      if (u < Cfg::V_HALF) {
        const int cc = u % (D / 8), q4 = u / (D / 8);
        const int pc = q4 >> 1;
        const uint32_t in[4][4] = {{vfull[i][0].x, vfull[i][0].y, vfull[i][0].z, vfull[i][0].w},
                                   {vfull[i][1].x, vfull[i][1].y, vfull[i][1].z, vfull[i][1].w},
                                   {vfull[i][2].x, vfull[i][2].y, vfull[i][2].z, vfull[i][2].w},
                                   {vfull[i][3].x, vfull[i][3].y, vfull[i][3].z, vfull[i][3].w}};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int c = cc * 8 + e;
          const int dw = e >> 1;
          uint2 o;
          if (e & 1) {
            o.x = perm_hi(in[0][dw], in[1][dw]);
            o.y = perm_hi(in[2][dw], in[3][dw]);
          } else {
            o.x = perm_lo(in[0][dw], in[1][dw]);
            o.y = perm_lo(in[2][dw], in[3][dw]);
          }
          uint2* dst = reinterpret_cast<uint2*>(&v_lds[c * CPR_V + (pc ^ vt_swizzle(c, CPR_V))]);
          dst[q4 & 1] = o;
        }
      }
    }
  };

  const float sl2 = a.scale_log2;

  if (sched_len > 0) {
    load_k(sched_tile(0));
    load_v4(sched_tile(0));
    store_k();
    store_v();
    __syncthreads();
  }

  for (int s = 0; s < sched_len; ++s) {
    const int tile = sched_tile(s);
    const bool mine = sched_mine(s);
    const bool has_next = s + 1 < sched_len;
    const int next = has_next ? sched_tile(s + 1) : 0;
    if (has_next) load_k(next);

    f32x16_t sacc[MB][QG];
    if (mine) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) sacc[mb][qg] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int r = 32 * mb + l32;
          const uint4 av = k_lds[r * CPR_K + ((2 * ks + half) ^ (r % CPR_K))];
#pragma unroll
          for (int qg = 0; qg < QG; ++qg)
            sacc[mb][qg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, qf[qg][ks]),
                sacc[mb][qg], 0, 0, 0);
        }
      }
    }
    __syncthreads();                       // every wave is done reading K(tile)
    if (has_next) {
      store_k();
      load_v4(next);
    }

    if (mine) {
      const TileValid tv = tile_valid(L, tile);
      uint4 pk[QG][PS];
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) {
        float t[MB][16];
        float mx = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float x = sacc[mb][qg][r] * sl2;
            if (!tv.full && !row_is_real(L, tv, sacc_token(mb, r, half))) x = -INFINITY;
            t[mb][r] = x;
            mx = fmaxf(mx, x);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        // lazy rescale: only move the subtracted maximum when it is exceeded by > 2^8
        if (mx > m_run[qg] + kLazyThreshold) {
          const float alpha = exp2f(m_run[qg] - mx);   // 0 on the first tile
          m_run[qg] = mx;
          l_run[qg] *= alpha;
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) oacc[cb][qg] *= alpha;
        }
        const float mref = m_run[qg];
        float psum = 0.0f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = exp2f(t[mb][r] - mref);
            t[mb][r] = p;
            psum += p;
          }
        l_run[qg] += psum;
#pragma unroll
        for (int ps = 0; ps < PS; ++ps) {
          const int mb = ps >> 1, r0 = 8 * (ps & 1);
          pk[qg][ps] = make_uint4(pack_bf16(t[mb][r0 + 0], t[mb][r0 + 1]),
                                  pack_bf16(t[mb][r0 + 2], t[mb][r0 + 3]),
                                  pack_bf16(t[mb][r0 + 4], t[mb][r0 + 5]),
                                  pack_bf16(t[mb][r0 + 6], t[mb][r0 + 7]));
        }
      }
#pragma unroll
      for (int ps = 0; ps < PS; ++ps) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const int c = 32 * cb + l32;
          const uint4 av = v_lds[c * CPR_V + ((2 * ps + half) ^ vt_swizzle(c, CPR_V))];
#pragma unroll
          for (int qg = 0; qg < QG; ++qg)
            oacc[cb][qg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, pk[qg][ps]),
                oacc[cb][qg], 0, 0, 0);
        }
      }
    }
    __syncthreads();                       // every wave is done reading V^T(tile)
    if (has_next) {
      store_v();
      __syncthreads();
    }
  }

  // ---- epilogue: normalise and write O (and lse)
  if (!wave_active) return;
  const TileValid tq = tile_valid(L, qt);
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    const int qrow = 32 * qg + l32;
    const float lt = l_run[qg] + __shfl_xor(l_run[qg], 32);
    const bool real = row_is_real(L, tq, qrow);
    const float inv = (real && lt > 0.0f) ? 1.0f / lt : 0.0f;
    const long long orow = head_row0 + (long long)qt * TILE + qrow;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c0 = 32 * cb + 8 * g + 4 * half;
        const float o0 = oacc[cb][qg][4 * g + 0] * inv, o1 = oacc[cb][qg][4 * g + 1] * inv;
        const float o2 = oacc[cb][qg][4 * g + 2] * inv, o3 = oacc[cb][qg][4 * g + 3] * inv;
        if constexpr (F32IN) {
          *reinterpret_cast<float4*>(static_cast<float*>(a.out) + orow * D + c0) =
              make_float4(o0, o1, o2, o3);
        } else {
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + orow * D + c0) =
              make_uint2(pack_bf16(o0, o1), pack_bf16(o2, o3));
        }
      }
    if (a.lse && half == 0) {
      a.lse[orow] = (real && lt > 0.0f) ? (m_run[qg] + log2f(lt)) * 0.69314718055994531f
                                        : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// fp8 e4m3 variant (FPSAttention, Approach: FP8 on the same tiles as the
// sparsity). Q/K/V are e4m3 codes with one fp32 scale per (b, head, tile).
//   S^T = Kc . Qc^T   v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales),
//                     then times q_scale * k_scale(tile) * sigma * log2(e);
//   O^T += Vc^T . P8^T with P8 = e4m3(p * 112 * v_scale(tile) / max_t v_scale)
// The lazy-rescale threshold is 2 (p <= 4), so p * 112 * (<= 1) stays within
// e4m3's 448. Folding v_scale(tile) / max v_scale into P keeps one O
// accumulator scale for the whole walk; O = acc * max v_scale / 112 / l.
// Both halves of a lane pair hold 32 of the 64 kv tokens of a tile, so one
// K=64 MFMA covers the whole tile in the PV product.
typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr float kLazyFp8 = 2.0f;
constexpr float kP8Scale = 112.0f;          // 448 / 2^kLazyFp8

// kv token of element e (0..31) of a lane in half-wave `half` (e = 16*mb + r)
__device__ __forceinline__ int p8_token(int e, int half) {
  return 32 * (e >> 4) + 8 * ((e & 15) >> 2) + 4 * half + (e & 3);
}
__device__ __forceinline__ int k8_swizzle(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int v8_swizzle(int c) { return ((c >> 1) ^ (c >> 3)) & 3; }

__device__ __forceinline__ i32x8_t cat8(uint4 x, uint4 y) {
  i32x8_t r;
  r[0] = (int)x.x; r[1] = (int)x.y; r[2] = (int)x.z; r[3] = (int)x.w;
  r[4] = (int)y.x; r[5] = (int)y.y; r[6] = (int)y.z; r[7] = (int)y.w;
  return r;
}

template <int WAVES>
__global__ __launch_bounds__(64 * WAVES, 1) void attn_fp8_kernel(DevLayout L, AttnArgs a,
                                                                 int n_work, int qtiles_per_wg) {
  constexpr int TILE = 64, D = 128, QG = 2, MB = 2, CB = 4, KS = 2;
  constexpr int THREADS = 64 * WAVES;
  constexpr int K_CHUNKS = TILE * D / 16;            // 512 chunks of 16 codes
  constexpr int K_PER_T = K_CHUNKS / THREADS;
  constexpr int V_PIECES = (TILE / 4) * (D / 16);    // 4 tokens x 16 channels
  constexpr int V_PER_T = (V_PIECES + THREADS - 1) / THREADS;

  __shared__ uint4 k_lds[TILE * 8];                  // 64 rows x 128 B
  __shared__ uint4 v_lds[D * 4];                     // V^T: 128 rows x 64 B
  extern __shared__ int dyn[];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const int w = xcd_remap(blockIdx.x, n_work);
  const int wg_per_bh = (L.n_tiles + qtiles_per_wg - 1) / qtiles_per_wg;
  const int bh = w / wg_per_bh;
  const int qt0 = (w - bh * wg_per_bh) * qtiles_per_wg;
  const int qt = qt0 + wave;
  const bool wave_active = qt < L.n_tiles;
  const long long head_row0 = (long long)bh * L.n_padded;
  const uint8_t* Q = static_cast<const uint8_t*>(a.q);
  const uint8_t* K = static_cast<const uint8_t*>(a.k);
  const uint8_t* V = static_cast<const uint8_t*>(a.v);
  const float* ksc = a.k_scale + (long long)bh * L.n_tiles;
  const float* vsc = a.v_scale + (long long)bh * L.n_tiles;

  const int32_t* my_list = nullptr;
  int my_cnt = 0;
  if (wave_active) {
    if (a.kv_idx) {
      const long long row = (a.list_mode ? (long long)bh * L.n_tiles : 0ll) + qt;
      my_list = a.kv_idx + row * a.max_kv;
      my_cnt = min(max(a.kv_cnt[row], 0), a.max_kv);
    } else {
      my_cnt = L.n_tiles;
    }
  }

  int sched_len;
  int* sched = dyn + L.n_tiles;
  if constexpr (WAVES > 1) {
    int* marks = dyn;
    for (int t = tid; t < L.n_tiles; t += THREADS) marks[t] = 0;
    __syncthreads();
    for (int i = lane; i < my_cnt; i += 64) {
      const int t = my_list ? min(max(my_list[i], 0), L.n_tiles - 1) : i;
      atomicOr(&marks[t], 1 << wave);
    }
    __syncthreads();
    __shared__ int scan[THREADS];
    const int per = (L.n_tiles + THREADS - 1) / THREADS;
    const int lo = tid * per, hi = min(lo + per, L.n_tiles);
    int mine = 0;
    for (int t = lo; t < hi; ++t) mine += marks[t] != 0;
    scan[tid] = mine;
    __syncthreads();
    for (int off = 1; off < THREADS; off <<= 1) {
      const int add = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    int pos = scan[tid] - mine;
    sched_len = scan[THREADS - 1];
    for (int t = lo; t < hi; ++t)
      if (marks[t]) sched[pos++] = t | (marks[t] << 24);
    __syncthreads();
  } else {
    sched_len = my_cnt;
  }
  auto sched_tile = [&](int s) -> int {
    if constexpr (WAVES > 1) return sched[s] & 0xFFFFFF;
    else return my_list ? min(max(my_list[s], 0), L.n_tiles - 1) : s;
  };
  auto sched_mine = [&](int s) -> bool {
    if constexpr (WAVES > 1) return (sched[s] >> (24 + wave)) & 1;
    else return true;
  };

  // largest v scale of this (b, head): P is scaled by v_scale(tile) / wmax
  float wmax = 0.0f;
  for (int t = lane; t < L.n_tiles; t += 64) wmax = fmaxf(wmax, vsc[t]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) wmax = fmaxf(wmax, __shfl_xor(wmax, off));
  const float inv_wmax = wmax > 0.0f ? 1.0f / wmax : 0.0f;
  const int qt_c = min(qt, L.n_tiles - 1);
  const float qk_base = a.q_scale[(long long)bh * L.n_tiles + qt_c] * a.scale_log2;

  // Q codes as B operands: query row 32*qg + l32, bytes 64*ks + 32*half .. +31
  i32x8_t qf[QG][KS];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4* p = reinterpret_cast<const uint4*>(
          Q + (head_row0 + (long long)qt_c * TILE + 32 * qg + l32) * D + 64 * ks + 32 * half);
      qf[qg][ks] = cat8(p[0], p[1]);
    }

  f32x16_t oacc[CB][QG];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) oacc[cb][qg] = f32x16_t{};
  float m_run[QG], l_run[QG];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    m_run[qg] = -INFINITY;
    l_run[qg] = 0.0f;
  }

  uint4 kreg[K_PER_T];
  auto load_k = [&](int tile) {
    const uint4* base = reinterpret_cast<const uint4*>(K + (head_row0 + (long long)tile * TILE) * D);
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) kreg[i] = base[tid + i * THREADS];
  };
  auto store_k = [&]() {
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int c = tid + i * THREADS;
      const int r = c >> 3, ch = c & 7;
      k_lds[r * 8 + (ch ^ k8_swizzle(r))] = kreg[i];
    }
  };
  // V piece u: tokens tok0 .. tok0+3 (tok0 = 4 * (u / 8)) x channels 16 * (u % 8) ..
  uint4 vreg[V_PER_T][4];
  auto load_v = [&](int tile) {
    const uint4* base = reinterpret_cast<const uint4*>(V + (head_row0 + (long long)tile * TILE) * D);
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int u = tid + i * THREADS;
      if (u < V_PIECES) {
        const int cg = u & 7, tok0 = 4 * (u >> 3);
#pragma unroll
        for (int j = 0; j < 4; ++j) vreg[i][j] = base[(tok0 + j) * 8 + cg];
      }
    }
  };
  auto store_v = [&]() {
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int u = tid + i * THREADS;
      if (u < V_PIECES) {
        const int cg = u & 7, tok0 = 4 * (u >> 3);
        // tokens tok0..tok0+3 sit at V^T byte positions p0..p0+3 (see p8_token)
        const int hh = (tok0 >> 2) & 1, A = tok0 >> 5, B = (tok0 >> 3) & 3;
        const int p0 = 32 * hh + 16 * A + 4 * B;
        const uint32_t in[4][4] = {{vreg[i][0].x, vreg[i][0].y, vreg[i][0].z, vreg[i][0].w},
                                   {vreg[i][1].x, vreg[i][1].y, vreg[i][1].z, vreg[i][1].w},
                                   {vreg[i][2].x, vreg[i][2].y, vreg[i][2].z, vreg[i][2].w},
                                   {vreg[i][3].x, vreg[i][3].y, vreg[i][3].z, vreg[i][3].w}};
#pragma unroll
        for (int dw = 0; dw < 4; ++dw) {
          const uint32_t x01l = __builtin_amdgcn_perm(in[1][dw], in[0][dw], 0x05010400u);
          const uint32_t x01h = __builtin_amdgcn_perm(in[1][dw], in[0][dw], 0x07030602u);
          const uint32_t x23l = __builtin_amdgcn_perm(in[3][dw], in[2][dw], 0x05010400u);
          const uint32_t x23h = __builtin_amdgcn_perm(in[3][dw], in[2][dw], 0x07030602u);
          const uint32_t o[4] = {__builtin_amdgcn_perm(x23l, x01l, 0x05040100u),
                                 __builtin_amdgcn_perm(x23l, x01l, 0x07060302u),
                                 __builtin_amdgcn_perm(x23h, x01h, 0x05040100u),
                                 __builtin_amdgcn_perm(x23h, x01h, 0x07060302u)};
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) {
            const int c = 16 * cg + 4 * dw + bb;
            uint32_t* row = reinterpret_cast<uint32_t*>(&v_lds[c * 4]);
            const int chunk = (p0 >> 4) ^ v8_swizzle(c);
            row[chunk * 4 + ((p0 & 15) >> 2)] = o[bb];
          }
        }
      }
    }
  };

  if (sched_len > 0) {
    load_k(sched_tile(0));
    load_v(sched_tile(0));
    store_k();
    store_v();
    __syncthreads();
  }

  for (int s = 0; s < sched_len; ++s) {
    const int tile = sched_tile(s);
    const bool mine = sched_mine(s);
    const bool has_next = s + 1 < sched_len;
    const int next = has_next ? sched_tile(s + 1) : 0;
    if (has_next) load_k(next);

    f32x16_t sacc[MB][QG];
    if (mine) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) sacc[mb][qg] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int r = 32 * mb + l32;
          const int sw = k8_swizzle(r);
          const i32x8_t av = cat8(k_lds[r * 8 + ((4 * ks + 2 * half) ^ sw)],
                                  k_lds[r * 8 + ((4 * ks + 2 * half + 1) ^ sw)]);
#pragma unroll
          for (int qg = 0; qg < QG; ++qg)
            sacc[mb][qg] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                av, qf[qg][ks], sacc[mb][qg], 0, 0, 0, 127, 0, 127);
        }
      }
    }
    __syncthreads();
    if (has_next) {
      store_k();
      load_v(next);
    }

    if (mine) {
      const TileValid tv = tile_valid(L, tile);
      const float cs = qk_base * ksc[tile];
      const float pscale = kP8Scale * vsc[tile] * inv_wmax;
      i32x8_t pk[QG];
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) {
        float t[MB][16];
        float mx = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float x = sacc[mb][qg][r] * cs;
            if (!tv.full && !row_is_real(L, tv, sacc_token(mb, r, half))) x = -INFINITY;
            t[mb][r] = x;
            mx = fmaxf(mx, x);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (mx > m_run[qg] + kLazyFp8) {
          const float alpha = exp2f(m_run[qg] - mx);
          m_run[qg] = mx;
          l_run[qg] *= alpha;
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) oacc[cb][qg] *= alpha;
        }
        const float mref = m_run[qg];
        float psum = 0.0f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = exp2f(t[mb][r] - mref);
            psum += p;
            t[mb][r] = p * pscale;
          }
        l_run[qg] += psum;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int mb = i >> 2, r0 = 4 * (i & 3);
          int wv = __builtin_amdgcn_cvt_pk_fp8_f32(t[mb][r0], t[mb][r0 + 1], 0, false);
          wv = __builtin_amdgcn_cvt_pk_fp8_f32(t[mb][r0 + 2], t[mb][r0 + 3], wv, true);
          pk[qg][i] = wv;
        }
      }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int c = 32 * cb + l32;
        const int sw = v8_swizzle(c);
        const i32x8_t av = cat8(v_lds[c * 4 + ((2 * half) ^ sw)], v_lds[c * 4 + ((2 * half + 1) ^ sw)]);
#pragma unroll
        for (int qg = 0; qg < QG; ++qg)
          oacc[cb][qg] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              av, pk[qg], oacc[cb][qg], 0, 0, 0, 127, 0, 127);
      }
    }
    __syncthreads();
    if (has_next) {
      store_v();
      __syncthreads();
    }
  }

  if (!wave_active) return;
  const TileValid tq = tile_valid(L, qt);
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    const int qrow = 32 * qg + l32;
    const float lt = l_run[qg] + __shfl_xor(l_run[qg], 32);
    const bool real = row_is_real(L, tq, qrow);
    const float inv = (real && lt > 0.0f) ? wmax / (kP8Scale * lt) : 0.0f;
    const long long orow = head_row0 + (long long)qt * TILE + qrow;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c0 = 32 * cb + 8 * g + 4 * half;
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + orow * D + c0) =
            make_uint2(pack_bf16(oacc[cb][qg][4 * g] * inv, oacc[cb][qg][4 * g + 1] * inv),
                       pack_bf16(oacc[cb][qg][4 * g + 2] * inv, oacc[cb][qg][4 * g + 3] * inv));
      }
    if (a.lse && half == 0) {
      a.lse[orow] = (real && lt > 0.0f) ? (m_run[qg] + log2f(lt)) * 0.69314718055994531f
                                        : -INFINITY;
    }
  }
}

template <int TILE, int D, int WAVES, bool F32IN>
hipError_t launch_one(const DevLayout& L, const AttnArgs& a, hipStream_t s) {
  const int qpw = WAVES;
  const int wg_per_bh = (L.n_tiles + qpw - 1) / qpw;
  const int n_work = L.B * L.heads * wg_per_bh;
  const size_t dyn = WAVES > 1 ? (size_t)2 * L.n_tiles * sizeof(int) : 0;
  hipLaunchKernelGGL((attn_bf16_kernel<TILE, D, WAVES, F32IN>), dim3(n_work), dim3(64 * WAVES), dyn,
                     s, L, a, n_work, qpw);
  return hipGetLastError();
}

template <int WAVES>
hipError_t launch_fp8(const DevLayout& L, const AttnArgs& a, hipStream_t s) {
  const int wg_per_bh = (L.n_tiles + WAVES - 1) / WAVES;
  const int n_work = L.B * L.heads * wg_per_bh;
  const size_t dyn = WAVES > 1 ? (size_t)2 * L.n_tiles * sizeof(int) : 0;
  hipLaunchKernelGGL((attn_fp8_kernel<WAVES>), dim3(n_work), dim3(64 * WAVES), dyn, s, L, a,
                     n_work, WAVES);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const DevLayout& L, int dtype, const AttnArgs& a, hipStream_t s) {
  // shared (head-invariant) or dense lists: neighbouring query tiles share key
  // tiles, so four query tiles walk their union together; routed lists: one
  // wave per query tile.
  const bool grouped = (a.kv_idx == nullptr || a.list_mode == 0) && L.n_tiles <= 4096;
  if (dtype == 2) {
    if (L.C != 64 || L.d != 128) return hipErrorInvalidValue;
    return grouped ? launch_fp8<4>(L, a, s) : launch_fp8<1>(L, a, s);
  }
  const bool f32 = dtype == 0;
  if (L.C == 64 && L.d == 128) {
    if (f32) return grouped ? launch_one<64, 128, 4, true>(L, a, s) : launch_one<64, 128, 1, true>(L, a, s);
    return grouped ? launch_one<64, 128, 4, false>(L, a, s) : launch_one<64, 128, 1, false>(L, a, s);
  }
  if (L.C == 64 && L.d == 64) {
    if (f32) return grouped ? launch_one<64, 64, 4, true>(L, a, s) : launch_one<64, 64, 1, true>(L, a, s);
    return grouped ? launch_one<64, 64, 4, false>(L, a, s) : launch_one<64, 64, 1, false>(L, a, s);
  }
  if (L.C == 32 && L.d == 128) {
    if (f32) return grouped ? launch_one<32, 128, 4, true>(L, a, s) : launch_one<32, 128, 1, true>(L, a, s);
    return grouped ? launch_one<32, 128, 4, false>(L, a, s) : launch_one<32, 128, 1, false>(L, a, s);
  }
  if (L.C == 32 && L.d == 64) {
    if (f32) return grouped ? launch_one<32, 64, 4, true>(L, a, s) : launch_one<32, 64, 1, true>(L, a, s);
    return grouped ? launch_one<32, 64, 4, false>(L, a, s) : launch_one<32, 64, 1, false>(L, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace vsa
