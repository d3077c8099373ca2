// S6: block-sparse attention forward on gfx950 MFMA. This is the flash-style,
// FlashAttention-compatible sparse attention the pages build on (OSP-Next
// wiki TL;DR and card "Model Summary"; FPSAttention "Approach"; VSA Research
// Type row; FVAttn summary): each query tile visits only the key/value tiles
// of its list, with an online softmax.
//
// A wavefront owns 32 query rows (bf16) or one 64-row query tile (fp8) and
// computes the transposed products
//   S^T  = K . Q^T     A = K rows (LDS), B = Q^T (registers)
//   O^T += V^T . P^T   A = V^T rows (LDS), B = P^T (registers)
// so every lane holds one query row (lane % 32) of S^T, P^T and O^T: the
// softmax statistics, the rescale and the normalisation are lane-local, and
// the only cross-lane step is one max exchange between the half-waves per
// kv tile. The PV contraction runs over kv tokens in the order the S^T
// accumulator holds them and V^T is written to LDS in that same order, so P
// never moves between lanes.
//
// Work shapes (QPW = query tiles per workgroup):
//   QPW == 1: one query tile per workgroup, walking its own list (routed
//             masks, where neighbouring tiles share few key tiles);
//   QPW == 4: four consecutive query tiles walk the ascending union of their
//             lists once, each K/V tile loaded into LDS once for all of them
//             (dense, Skiparse-2D and window lists); waves whose list lacks
//             a tile skip its math. The LDS tiles are double-buffered: tile
//             s+1 is fetched while tile s is computed, one barrier per tile.
// The softmax subtracts a lazily raised running maximum: it only moves when
// a score exceeds it by more than 2^kLazy (exp2 units), so O^T is rarely
// rescaled. Pad keys are masked from one ballot per padded tile.
#include <float.h>

#include "vsa_internal.h"

namespace vsa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

// two floats -> two bf16 (round to nearest even) in one dword, lo first
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// 8 consecutive elements at element offset `off` as 8 bf16 in a uint4.
template <bool F32IN>
__device__ __forceinline__ uint4 load8(const void* base, long long off) {
  if constexpr (F32IN) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    const float4 x = p[0], y = p[1];
    return make_uint4(pack2(x.x, x.y), pack2(x.z, x.w), pack2(y.x, y.y), pack2(y.z, y.w));
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

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Work assignment and the per-workgroup schedule (shared by both kernels).
struct WaveWork {
  long long head_row0;     // first row of this (b, head) in the tiled tensors
  int bh;                  // b * heads + head
  int slot;                // which of the workgroup's query tiles this wave works on
  int qt;                  // that query tile
  bool active;             // qt < n_tiles
  const int32_t* list;     // null: dense
  int cnt;
};

// QPW query tiles per workgroup, WPQ waves per query tile.
template <int QPW, int WPQ>
__device__ __forceinline__ WaveWork wave_work(const DevLayout& L, const AttnArgs& a, int n_work,
                                              int wave) {
  WaveWork w;
  const int item = xcd_remap(blockIdx.x, n_work);
  const int wg_per_bh = (L.n_tiles + QPW - 1) / QPW;
  w.bh = item / wg_per_bh;
  w.slot = wave / WPQ;
  w.qt = (item - w.bh * wg_per_bh) * QPW + w.slot;
  w.active = w.qt < L.n_tiles;
  w.head_row0 = (long long)w.bh * L.n_padded;
  w.list = nullptr;
  w.cnt = 0;
  if (w.active) {
    if (a.kv_idx) {
      const long long row = (a.list_mode ? (long long)w.bh * L.n_tiles : 0ll) + w.qt;
      w.list = a.kv_idx + row * a.max_kv;
      w.cnt = min(max(a.kv_cnt[row], 0), a.max_kv);
    } else {
      w.cnt = L.n_tiles;
    }
  }
  return w;
}

// QPW > 1: write the ascending union of the query tiles' lists into sched[],
// each entry = tile | (mask of query-tile slots listing it) << 24; returns
// its length.
template <int QPW, int WPQ>
__device__ int build_schedule(const DevLayout& L, const WaveWork& w, int* dyn, int* scan,
                              int tid, int lane) {
  constexpr int THREADS = 64 * QPW * WPQ;
  int* marks = dyn;
  int* sched = dyn + L.n_tiles;
  for (int t = tid; t < L.n_tiles; t += THREADS) marks[t] = 0;
  __syncthreads();
  if ((tid >> 6) % WPQ == 0) {
    for (int i = lane; i < w.cnt; i += 64) {
      const int t = w.list ? min(max(w.list[i], 0), L.n_tiles - 1) : i;
      atomicOr(&marks[t], 1 << w.slot);
    }
  }
  __syncthreads();
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
  const int len = scan[THREADS - 1];
  for (int t = lo; t < hi; ++t)
    if (marks[t]) sched[pos++] = t | (marks[t] << 24);
  __syncthreads();
  return len;
}

template <int QPW>
__device__ __forceinline__ int sched_tile(const int* sched, const WaveWork& w, int s, int n_tiles) {
  if constexpr (QPW > 1) return sched[s] & 0xFFFFFF;
  else return w.list ? min(max(w.list[s], 0), n_tiles - 1) : s;
}
template <int QPW>
__device__ __forceinline__ bool sched_mine(const int* sched, int s, int slot) {
  if constexpr (QPW > 1) return (sched[s] >> (24 + slot)) & 1;
  else return true;
}

// Bit (16*mb + r) set iff the kv token this lane holds in register r of S^T
// block mb is a real token. Wave-uniform `full` short-cuts the common case.
template <int MB>
__device__ __forceinline__ uint32_t kv_valid_bits(const DevLayout& L, int tile, int lane, int half,
                                                  bool& full) {
  const TileValid tv = tile_valid(L, tile);
  full = tv.full;
  if (full) return 0xFFFFFFFFu;
  const bool v = lane < 32 * MB && row_is_real(L, tv, lane);
  const unsigned long long vm = __ballot(v);
  uint32_t m = 0;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      m |= (uint32_t)((vm >> (32 * mb + 8 * g + 4 * half)) & 0xFull) << (16 * mb + 4 * g);
  return m;
}

// Online-softmax step on one 32-row query group: scores s (raw dot products,
// MB blocks of 16 per lane) become p = exp2(s * sl2 - m_run), in place.
// Returns the factor O must be multiplied by (1 when m_run did not move).
template <int MB>
__device__ __forceinline__ float softmax_step(f32x16_t (&s)[MB], bool full, uint32_t bits,
                                              float sl2, float lazy, float& m_run, float& l_run) {
  float hi = -INFINITY, lo = INFINITY;
  if (full) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        hi = fmaxf(hi, s[mb][r]);
        lo = fminf(lo, s[mb][r]);
      }
  } else {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool ok = (bits >> (16 * mb + r)) & 1u;
        hi = fmaxf(hi, ok ? s[mb][r] : -INFINITY);
        lo = fminf(lo, ok ? s[mb][r] : INFINITY);
      }
  }
  hi = fmaxf(hi, __shfl_xor(hi, 32));
  lo = fminf(lo, __shfl_xor(lo, 32));
  const float mx = sl2 >= 0.0f ? hi * sl2 : lo * sl2;    // max over the tile of s * sl2
  float alpha = 1.0f;
  if (mx > m_run + lazy) {
    alpha = fast_exp2(m_run - mx);                       // 0 on the first tile
    m_run = mx;
    l_run *= alpha;
  }
  const float nm = -m_run;
  float psum = 0.0f;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float p = fast_exp2(fmaf(s[mb][r], sl2, nm));
      if (!full) p = ((bits >> (16 * mb + r)) & 1u) ? p : 0.0f;
      s[mb][r] = p;
      psum += p;
    }
  l_run += psum;
  return alpha;
}

__device__ __forceinline__ int vt_swizzle(int c, int cpr) { return (c ^ (c >> 3)) & (cpr - 1); }

// ---------------------------------------------------------------------------
// bf16 kernel: one wave = 32 query rows (a query tile of 64 rows takes two
// waves, which share the K/V tiles in LDS). About 200 registers per wave let
// two waves share each SIMD, so one wave's softmax runs while the other's
// MFMAs do. QPW query tiles per workgroup: 4 for shared lists (union walk,
// LDS double-buffered), 1 for routed lists.
template <int TILE, int D, int QPW, bool F32IN>
__global__ __launch_bounds__(64 * QPW * (TILE / 32)) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bf16_kernel(DevLayout L, AttnArgs a, int n_work) {
  constexpr int WPQ = TILE / 32;         // waves per query tile
  constexpr int MB = TILE / 32;          // 32-token blocks of a kv tile
  constexpr int KS = D / 16;             // QK^T k-steps over the head dim
  constexpr int CB = D / 32;             // 32-channel blocks of O^T
  constexpr int PS = TILE / 16;          // PV k-steps over kv tokens
  constexpr int CPR_K = D / 8;           // 16-byte chunks per K row
  constexpr int CPR_V = TILE / 8;        // 16-byte chunks per V^T row
  constexpr int THREADS = 64 * QPW * WPQ;
  constexpr int K_PER_T = TILE * CPR_K / THREADS;
  constexpr int V_PIECES = (TILE / 4) * (D / 8);         // 4 tokens x 8 channels
  constexpr int V_PER_T = (V_PIECES + THREADS - 1) / THREADS;
  constexpr int NBUF = QPW > 1 ? 2 : 1;
  constexpr float kLazy = 8.0f;
  static_assert(TILE == 32 || TILE == 64, "tiles of 32 or 64 tokens");
  static_assert((TILE * CPR_K) % THREADS == 0, "K tile split");

  __shared__ uint4 k_lds[NBUF][TILE * CPR_K];
  __shared__ uint4 v_lds[NBUF][D * CPR_V];
  __shared__ int scan[THREADS];
  extern __shared__ int dyn[];           // QPW > 1: marks + schedule

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int rg = wave % WPQ;             // which 32 rows of the query tile

  const WaveWork ww = wave_work<QPW, WPQ>(L, a, n_work, wave);
  const int* sched = dyn + L.n_tiles;
  int len;
  if constexpr (QPW > 1) len = build_schedule<QPW, WPQ>(L, ww, dyn, scan, tid, lane);
  else len = ww.cnt;

  // Q^T fragments (B operand): query row 32*rg + l32, channels 16*ks + 8*half ..
  const int qt_c = min(ww.qt, L.n_tiles - 1);
  uint4 qf[KS];
  {
    const long long row = ww.head_row0 + (long long)qt_c * TILE + 32 * rg + l32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = load8<F32IN>(a.q, row * D + ks * 16 + half * 8);
  }

  f32x16_t oacc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) oacc[cb] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.0f;

  uint4 kreg[K_PER_T];
  uint4 vreg[V_PER_T][4];
  auto load_k = [&](int tile) {
    const long long base = (ww.head_row0 + (long long)tile * TILE) * D;
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int c = tid + i * THREADS;
      kreg[i] = load8<F32IN>(a.k, base + (long long)(c / CPR_K) * D + (c % CPR_K) * 8);
    }
  };
  auto store_k = [&](int buf) {
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int c = tid + i * THREADS;
      const int r = c / CPR_K, ch = c % CPR_K;
      k_lds[buf][r * CPR_K + (ch ^ (r % CPR_K))] = kreg[i];
    }
  };
  // V piece u = 4 consecutive kv tokens x 8 channels (channel chunk cc,
  // quarter q4); its tokens go to V^T positions 4*q4 .. 4*q4+3, which is the
  // token order of the S^T accumulator: register r of block mb in half-wave
  // h holds token 32*mb + 8*(r/4) + 4*h + r%4.
  auto load_v = [&](int tile) {
    const long long base = (ww.head_row0 + (long long)tile * TILE) * D;
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int u = tid + i * THREADS;
      if (u < V_PIECES) {
        const int cc = u % (D / 8), q4 = u / (D / 8);
        const int pc = q4 >> 1;
        const int tok0 = 16 * (pc >> 1) + 4 * (pc & 1) + 8 * (q4 & 1);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          vreg[i][j] = load8<F32IN>(a.v, base + (long long)(tok0 + j) * D + cc * 8);
      }
    }
  };
  auto store_v = [&](int buf) {
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int u = tid + i * THREADS;
      if (u < V_PIECES) {
        const int cc = u % (D / 8), q4 = u / (D / 8);
        const int pc = q4 >> 1;
        const uint32_t in[4][4] = {{vreg[i][0].x, vreg[i][0].y, vreg[i][0].z, vreg[i][0].w},
                                   {vreg[i][1].x, vreg[i][1].y, vreg[i][1].z, vreg[i][1].w},
                                   {vreg[i][2].x, vreg[i][2].y, vreg[i][2].z, vreg[i][2].w},
                                   {vreg[i][3].x, vreg[i][3].y, vreg[i][3].z, vreg[i][3].w}};
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
          uint2* dst =
              reinterpret_cast<uint2*>(&v_lds[buf][c * CPR_V + (pc ^ vt_swizzle(c, CPR_V))]);
          dst[q4 & 1] = o;
        }
      }
    }
  };

  const float sl2 = a.scale_log2;
  if (len > 0) {
    const int t0 = sched_tile<QPW>(sched, ww, 0, L.n_tiles);
    load_k(t0);
    load_v(t0);
    store_k(0);
    store_v(0);
    __syncthreads();
  }

  for (int s = 0; s < len; ++s) {
    const int cur = NBUF == 2 ? (s & 1) : 0;
    const int tile = sched_tile<QPW>(sched, ww, s, L.n_tiles);
    const bool mine = sched_mine<QPW>(sched, s, ww.slot);
    const bool has_next = s + 1 < len;
    const int next = has_next ? sched_tile<QPW>(sched, ww, s + 1, L.n_tiles) : 0;
    if (has_next) {
      load_k(next);
      if constexpr (NBUF == 2) load_v(next);
    }
    f32x16_t sacc[MB];
    if (mine) {
      // ---- S^T = K . Q^T
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) sacc[mb] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int r = 32 * mb + l32;
          const uint4 av = k_lds[cur][r * CPR_K + ((2 * ks + half) ^ (r % CPR_K))];
          sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, qf[ks]), sacc[mb],
              0, 0, 0);
        }
    }
    if constexpr (NBUF == 1) {
      __syncthreads();                            // done reading K(tile)
      if (has_next) {
        store_k(0);
        load_v(next);
      }
    }
    if (mine) {
      bool full;
      const uint32_t bits = kv_valid_bits<MB>(L, tile, lane, half, full);
      const float alpha = softmax_step<MB>(sacc, full, bits, sl2, kLazy, m_run, l_run);
      if (alpha != 1.0f) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) oacc[cb] *= alpha;
      }
      uint4 pk[PS];
#pragma unroll
      for (int ps = 0; ps < PS; ++ps) {
        const int mb = ps >> 1, r0 = 8 * (ps & 1);
        pk[ps] = make_uint4(pack2(sacc[mb][r0 + 0], sacc[mb][r0 + 1]),
                            pack2(sacc[mb][r0 + 2], sacc[mb][r0 + 3]),
                            pack2(sacc[mb][r0 + 4], sacc[mb][r0 + 5]),
                            pack2(sacc[mb][r0 + 6], sacc[mb][r0 + 7]));
      }
      // ---- O^T += V^T . P^T
#pragma unroll
      for (int ps = 0; ps < PS; ++ps)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const int c = 32 * cb + l32;
          const uint4 av = v_lds[cur][c * CPR_V + ((2 * ps + half) ^ vt_swizzle(c, CPR_V))];
          oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, pk[ps]), oacc[cb],
              0, 0, 0);
        }
    }
    if constexpr (NBUF == 2) {
      if (has_next) {
        store_k(cur ^ 1);
        store_v(cur ^ 1);
      }
      __syncthreads();
    } else {
      __syncthreads();                            // done reading V^T(tile)
      if (has_next) {
        store_v(0);
        __syncthreads();
      }
    }
  }

  // ---- epilogue: normalise and write O (and lse)
  if (!ww.active) return;
  const TileValid tq = tile_valid(L, ww.qt);
  const int qrow = 32 * rg + l32;
  const float lt = l_run + __shfl_xor(l_run, 32);
  const bool real = row_is_real(L, tq, qrow);
  const float inv = (real && lt > 0.0f) ? 1.0f / lt : 0.0f;
  const long long orow = ww.head_row0 + (long long)ww.qt * TILE + qrow;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c0 = 32 * cb + 8 * g + 4 * half;
      const float o0 = oacc[cb][4 * g + 0] * inv, o1 = oacc[cb][4 * g + 1] * inv;
      const float o2 = oacc[cb][4 * g + 2] * inv, o3 = oacc[cb][4 * g + 3] * inv;
      if constexpr (F32IN) {
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + orow * D + c0) =
            make_float4(o0, o1, o2, o3);
      } else {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + orow * D + c0) =
            make_uint2(pack2(o0, o1), pack2(o2, o3));
      }
    }
  if (a.lse && half == 0) {
    a.lse[orow] = (real && lt > 0.0f) ? (m_run + __log2f(lt)) * 0.69314718055994531f : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// fp8 e4m3 variant (FPSAttention, Approach: FP8 on the same tiles as the
// sparsity). Q/K/V are e4m3 codes with one fp32 scale per (b, head, tile).
//   S^T = Kc . Qc^T   v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales),
//                     times q_scale * k_scale(tile) * sigma * log2(e);
//   O^T += Vc^T . P8^T with P8 = e4m3(p * 112 * v_scale(tile) / max_t v_scale)
// The lazy-rescale threshold is 2 (p <= 4), so p * 112 * (<= 1) stays within
// e4m3's 448. Folding v_scale(tile) / max v_scale into P keeps one O
// accumulator scale for the whole walk; O = acc * max v_scale / 112 / l.
// The two half-waves each hold 32 of a tile's 64 kv tokens, so one K=64 MFMA
// covers the whole tile in the PV product. Tiles are 64 tokens, d = 128; LDS
// holds two K/V tile buffers in both work shapes.
constexpr float kP8Scale = 112.0f;          // 448 / 2^2

__device__ __forceinline__ int k8_swizzle(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int v8_swizzle(int c) { return ((c >> 1) ^ (c >> 3)) & 3; }

__device__ __forceinline__ i32x8_t cat8(uint4 x, uint4 y) {
  i32x8_t r;
  r[0] = (int)x.x; r[1] = (int)x.y; r[2] = (int)x.z; r[3] = (int)x.w;
  r[4] = (int)y.x; r[5] = (int)y.y; r[6] = (int)y.z; r[7] = (int)y.w;
  return r;
}

template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_fp8_kernel(DevLayout L, AttnArgs a, int n_work) {
  constexpr int TILE = 64, D = 128, QG = 2, MB = 2, CB = 4, KS = 2;
  constexpr int THREADS = 64 * WAVES;
  constexpr int K_PER_T = TILE * D / 16 / THREADS;   // 512 chunks of 16 codes
  constexpr int V_PIECES = (TILE / 4) * (D / 16);    // 4 tokens x 16 channels
  constexpr int V_PER_T = (V_PIECES + THREADS - 1) / THREADS;
  constexpr float kLazy = 2.0f;

  __shared__ uint4 k_lds[2][TILE * 8];               // 64 rows x 128 B
  __shared__ uint4 v_lds[2][D * 4];                  // V^T: 128 rows x 64 B
  __shared__ int scan[THREADS];
  extern __shared__ int dyn[];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const WaveWork ww = wave_work<WAVES, 1>(L, a, n_work, wave);
  const int* sched = dyn + L.n_tiles;
  int len;
  if constexpr (WAVES > 1) len = build_schedule<WAVES, 1>(L, ww, dyn, scan, tid, lane);
  else len = ww.cnt;

  const uint8_t* Q = static_cast<const uint8_t*>(a.q);
  const uint8_t* K = static_cast<const uint8_t*>(a.k);
  const uint8_t* V = static_cast<const uint8_t*>(a.v);
  const float* ksc = a.k_scale + (long long)ww.bh * L.n_tiles;
  const float* vsc = a.v_scale + (long long)ww.bh * L.n_tiles;

  // largest v scale of this (b, head): P is scaled by v_scale(tile) / wmax
  float wmax = 0.0f;
  for (int t = lane; t < L.n_tiles; t += 64) wmax = fmaxf(wmax, vsc[t]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) wmax = fmaxf(wmax, __shfl_xor(wmax, off));
  const float inv_wmax = wmax > 0.0f ? 1.0f / wmax : 0.0f;
  const int qt_c = min(ww.qt, L.n_tiles - 1);
  const float qk_base = a.q_scale[(long long)ww.bh * L.n_tiles + qt_c] * a.scale_log2;

  // Q codes as B operands: query row 32*qg + l32, bytes 64*ks + 32*half .. +31
  i32x8_t qf[QG][KS];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4* p = reinterpret_cast<const uint4*>(
          Q + (ww.head_row0 + (long long)qt_c * TILE + 32 * qg + l32) * D + 64 * ks + 32 * half);
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
  uint4 vreg[V_PER_T][4];
  auto load_k = [&](int tile) {
    const uint4* base =
        reinterpret_cast<const uint4*>(K + (ww.head_row0 + (long long)tile * TILE) * D);
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) kreg[i] = base[tid + i * THREADS];
  };
  auto store_k = [&](int buf) {
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int c = tid + i * THREADS;
      const int r = c >> 3, ch = c & 7;
      k_lds[buf][r * 8 + (ch ^ k8_swizzle(r))] = kreg[i];
    }
  };
  // V piece u: tokens tok0 .. tok0+3 (tok0 = 4 * (u / 8)) x channels 16 * (u % 8) ..
  auto load_v = [&](int tile) {
    const uint4* base =
        reinterpret_cast<const uint4*>(V + (ww.head_row0 + (long long)tile * TILE) * D);
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
  // kv token of element e (0..31) of a lane in half-wave h: 32*(e/16) +
  // 8*((e%16)/4) + 4*h + e%4; tokens tok0..tok0+3 therefore sit at V^T byte
  // positions p0..p0+3 with p0 = 32*h + 16*(tok0/32) + 4*((tok0/8)%4).
  auto store_v = [&](int buf) {
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int u = tid + i * THREADS;
      if (u < V_PIECES) {
        const int cg = u & 7, tok0 = 4 * (u >> 3);
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
            uint32_t* row = reinterpret_cast<uint32_t*>(&v_lds[buf][c * 4]);
            row[((p0 >> 4) ^ v8_swizzle(c)) * 4 + ((p0 & 15) >> 2)] = o[bb];
          }
        }
      }
    }
  };

  if (len > 0) {
    const int t0 = sched_tile<WAVES>(sched, ww, 0, L.n_tiles);
    load_k(t0);
    load_v(t0);
    store_k(0);
    store_v(0);
    __syncthreads();
  }

  for (int s = 0; s < len; ++s) {
    const int cur = s & 1;
    const int tile = sched_tile<WAVES>(sched, ww, s, L.n_tiles);
    const bool mine = sched_mine<WAVES>(sched, s, ww.slot);
    const bool has_next = s + 1 < len;
    if (has_next) {
      const int next = sched_tile<WAVES>(sched, ww, s + 1, L.n_tiles);
      load_k(next);
      load_v(next);
    }
    if (mine) {
      f32x16_t sacc[QG][MB];
#pragma unroll
      for (int qg = 0; qg < QG; ++qg)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) sacc[qg][mb] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int r = 32 * mb + l32;
          const int sw = k8_swizzle(r);
          const i32x8_t av = cat8(k_lds[cur][r * 8 + ((4 * ks + 2 * half) ^ sw)],
                                  k_lds[cur][r * 8 + ((4 * ks + 2 * half + 1) ^ sw)]);
#pragma unroll
          for (int qg = 0; qg < QG; ++qg)
            sacc[qg][mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                av, qf[qg][ks], sacc[qg][mb], 0, 0, 0, 127, 0, 127);
        }
      bool full;
      const uint32_t bits = kv_valid_bits<MB>(L, tile, lane, half, full);
      const float cs = qk_base * ksc[tile];
      const float pscale = kP8Scale * vsc[tile] * inv_wmax;
      i32x8_t pk[QG];
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) {
        const float alpha = softmax_step<MB>(sacc[qg], full, bits, cs, kLazy, m_run[qg], l_run[qg]);
        if (alpha != 1.0f) {
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) oacc[cb][qg] *= alpha;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int mb = i >> 2, r0 = 4 * (i & 3);
          int wv = __builtin_amdgcn_cvt_pk_fp8_f32(sacc[qg][mb][r0] * pscale,
                                                   sacc[qg][mb][r0 + 1] * pscale, 0, false);
          wv = __builtin_amdgcn_cvt_pk_fp8_f32(sacc[qg][mb][r0 + 2] * pscale,
                                               sacc[qg][mb][r0 + 3] * pscale, wv, true);
          pk[qg][i] = wv;
        }
      }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int c = 32 * cb + l32;
        const int sw = v8_swizzle(c);
        const i32x8_t av = cat8(v_lds[cur][c * 4 + ((2 * half) ^ sw)],
                                v_lds[cur][c * 4 + ((2 * half + 1) ^ sw)]);
#pragma unroll
        for (int qg = 0; qg < QG; ++qg)
          oacc[cb][qg] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              av, pk[qg], oacc[cb][qg], 0, 0, 0, 127, 0, 127);
      }
    }
    if (has_next) {
      store_k(cur ^ 1);
      store_v(cur ^ 1);
    }
    __syncthreads();
  }

  if (!ww.active) return;
  const TileValid tq = tile_valid(L, ww.qt);
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    const int qrow = 32 * qg + l32;
    const float lt = l_run[qg] + __shfl_xor(l_run[qg], 32);
    const bool real = row_is_real(L, tq, qrow);
    const float inv = (real && lt > 0.0f) ? wmax / (kP8Scale * lt) : 0.0f;
    const long long orow = ww.head_row0 + (long long)ww.qt * TILE + qrow;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c0 = 32 * cb + 8 * g + 4 * half;
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + orow * D + c0) =
            make_uint2(pack2(oacc[cb][qg][4 * g] * inv, oacc[cb][qg][4 * g + 1] * inv),
                       pack2(oacc[cb][qg][4 * g + 2] * inv, oacc[cb][qg][4 * g + 3] * inv));
      }
    if (a.lse && half == 0) {
      a.lse[orow] = (real && lt > 0.0f) ? (m_run[qg] + __log2f(lt)) * 0.69314718055994531f
                                        : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
template <int TILE, int D, int QPW, bool F32IN>
hipError_t launch_bf16(const DevLayout& L, const AttnArgs& a, hipStream_t s) {
  const int n_work = L.B * L.heads * ((L.n_tiles + QPW - 1) / QPW);
  const size_t dyn = QPW > 1 ? (size_t)2 * L.n_tiles * sizeof(int) : 0;
  hipLaunchKernelGGL((attn_bf16_kernel<TILE, D, QPW, F32IN>), dim3(n_work),
                     dim3(64 * QPW * (TILE / 32)), dyn, s, L, a, n_work);
  return hipGetLastError();
}

template <int WAVES>
hipError_t launch_fp8(const DevLayout& L, const AttnArgs& a, hipStream_t s) {
  const int n_work = L.B * L.heads * ((L.n_tiles + WAVES - 1) / WAVES);
  const size_t dyn = WAVES > 1 ? (size_t)2 * L.n_tiles * sizeof(int) : 0;
  hipLaunchKernelGGL((attn_fp8_kernel<WAVES>), dim3(n_work), dim3(64 * WAVES), dyn, s, L, a,
                     n_work);
  return hipGetLastError();
}

template <int TILE, int D, bool F32IN>
hipError_t launch_bf16_shape(const DevLayout& L, const AttnArgs& a, bool grouped, hipStream_t s) {
  return grouped ? launch_bf16<TILE, D, 4, F32IN>(L, a, s) : launch_bf16<TILE, D, 1, F32IN>(L, a, s);
}

}  // namespace

hipError_t launch_attn(const DevLayout& L, int dtype, const AttnArgs& a, hipStream_t s) {
  // Shared (head-invariant) or dense lists: neighbouring query tiles share key
  // tiles, so four query tiles walk their union together. Routed lists: one
  // wave per query tile.
  const bool grouped = (a.kv_idx == nullptr || a.list_mode == 0) && L.n_tiles <= 4096;
  if (dtype == 2) {
    if (L.C != 64 || L.d != 128) return hipErrorInvalidValue;
    return grouped ? launch_fp8<4>(L, a, s) : launch_fp8<1>(L, a, s);
  }
  const bool f32 = dtype == 0;
  if (L.C == 64 && L.d == 128)
    return f32 ? launch_bf16_shape<64, 128, true>(L, a, grouped, s)
               : launch_bf16_shape<64, 128, false>(L, a, grouped, s);
  if (L.C == 64 && L.d == 64)
    return f32 ? launch_bf16_shape<64, 64, true>(L, a, grouped, s)
               : launch_bf16_shape<64, 64, false>(L, a, grouped, s);
  if (L.C == 32 && L.d == 128)
    return f32 ? launch_bf16_shape<32, 128, true>(L, a, grouped, s)
               : launch_bf16_shape<32, 128, false>(L, a, grouped, s);
  if (L.C == 32 && L.d == 64)
    return f32 ? launch_bf16_shape<32, 64, true>(L, a, grouped, s)
               : launch_bf16_shape<32, 64, false>(L, a, grouped, s);
  return hipErrorInvalidValue;
}

}  // namespace vsa
