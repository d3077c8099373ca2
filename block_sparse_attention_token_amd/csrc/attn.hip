// S6: block-sparse attention forward on gfx950 MFMA. This is the flash-style,
// FlashAttention-compatible sparse attention the pages build on (OSP-Next
// wiki TL;DR and card "Model Summary"; FPSAttention "Approach"; VSA Research
// Type row; FVAttn summary): each query tile visits only the key/value tiles
// of its list, with an online softmax.
//
// A wavefront owns 32 query rows and computes the transposed products
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

#include <type_traits>

#include "vsa_internal.h"

namespace vsa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// two floats -> two bf16 (round to nearest even) in one dword, lo first
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t perm_lo(uint32_t a, uint32_t b) {   // lo16(a) | lo16(b) << 16
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t perm_hi(uint32_t a, uint32_t b) {   // hi16(a) | hi16(b) << 16
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Buffer-resource loads: the base of one (b, head) slice of a tensor sits in
// SGPRs and each load takes a 32-bit byte offset (VGPR part + SGPR part), so
// tile loads need no 64-bit address registers; offsets past num_records read
// as zero instead of faulting.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, long long bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)(bytes < 0x7FFFFFFFll ? bytes : 0x7FFFFFFFll),
                                           0x00020000);
}
__device__ __forceinline__ uint4 bload(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
// 8 consecutive elements at byte offset voff + soff as 8 bf16 (f32 input: 32 bytes, rounded)
template <bool F32IN>
__device__ __forceinline__ uint4 bload8(rsrc_t r, uint32_t voff, uint32_t soff) {
  if constexpr (F32IN) {
    const uint4 x = bload(r, voff, soff), y = bload(r, voff + 16, soff);
    return make_uint4(pack2(__uint_as_float(x.x), __uint_as_float(x.y)),
                      pack2(__uint_as_float(x.z), __uint_as_float(x.w)),
                      pack2(__uint_as_float(y.x), __uint_as_float(y.y)),
                      pack2(__uint_as_float(y.z), __uint_as_float(y.w)));
  } else {
    return bload(r, voff, soff);
  }
}

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
  // shared lists: contiguous ranges (query tiles sharing K/V share an L2);
  // per-head lists: chunks dealt round the XCDs (per-head work differs)
  int item = a.kv_idx && a.list_mode == 1 ? xcd_chunked(blockIdx.x, n_work, 64)
                                           : xcd_remap(blockIdx.x, n_work);
  // a work order deals the items heavy-first (per-head lists, one query tile
  // per workgroup); entries are clamped so that a bad order cannot address
  // outside the tensors
  if (QPW == 1 && a.work_order) item = min(max(a.work_order[item], 0), n_work - 1);
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
      const long long row = (a.list_mode == 1 ? (long long)w.bh * L.n_tiles : 0ll) + w.qt;
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
// its length. `shared` is set when every entry lists every active slot (the
// query tiles share one list), so every wave owns every step of the walk.
// `marks` (one byte per tile) and `scan` (one int per thread) are scratch
// that the caller may alias onto LDS it only uses afterwards.
template <int QPW, int WPQ>
__device__ int build_schedule(const DevLayout& L, const WaveWork& w, uint32_t* marks, int* scan,
                              int* sched, int tid, int lane, bool& shared) {
  static_assert(QPW <= 8, "slot masks are one byte");
  constexpr int THREADS = 64 * QPW * WPQ;
  const int words = (L.n_tiles + 3) >> 2;
  for (int t = tid; t < words; t += THREADS) marks[t] = 0;
  __syncthreads();
  if ((tid >> 6) % WPQ == 0) {
    for (int i = lane; i < w.cnt; i += 64) {
      const int t = w.list ? min(max(w.list[i], 0), L.n_tiles - 1) : i;
      atomicOr(&marks[t >> 2], 1u << (8 * (t & 3) + w.slot));
    }
  }
  __syncthreads();
  auto mark = [&](int t) -> int { return (marks[t >> 2] >> (8 * (t & 3))) & 0xFF; };
  const int per = (L.n_tiles + THREADS - 1) / THREADS;
  const int lo = tid * per, hi = min(lo + per, L.n_tiles);
  int mine = 0;
  for (int t = lo; t < hi; ++t) mine += mark(t) != 0;
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
  const int qt0 = w.qt - w.slot;
  const int active = (1 << min(max(L.n_tiles - qt0, 0), QPW)) - 1;
  bool same = true;
  for (int t = lo; t < hi; ++t) {
    const int m = mark(t);
    if (m) sched[pos++] = t | (m << 24);
    same = same && (m == 0 || m == active);
  }
  shared = __syncthreads_and(same) != 0;
  return len;
}

// Bit t set iff token tok0 + t (t < 32 * MB) of the tile is a real token,
// for a block known to hold padding; the same value in every lane.
template <int MB>
__device__ __forceinline__ unsigned long long kv_pad_ballot(const DevLayout& L, int tile, int tok0,
                                                            int lane) {
  const TileValid tv = tile_valid(L, tile);
  return __ballot(lane < 32 * MB && row_is_real(L, tv, tok0 + lane));
}

// A window of 64 schedule entries held in two registers: lane i holds entry
// base + i, its key tile and flags (bit j: kv block j of the tile holds
// padding; bits 8..15: the query-tile slots that list it). Each step reads
// its entry with v_readlane instead of a memory round trip; the window is
// refilled once per 64 entries.
template <int QPW, int SUB, int KVH>
struct SchedWindow {
  int base = 0, tile_v = 0, flags_v = 0;

  __device__ __forceinline__ void fill(const DevLayout& L, const WaveWork& w, const int* sched,
                                       int len, int b, int lane) {
    base = b;
    const int e = b + lane;
    int tile = 0, flags = 0;
    if (e < len) {
      if constexpr (QPW > 1) {
        const int ent = sched[e];
        tile = ent & 0xFFFFFF;
        flags = (ent >> 24) << 8;
      } else {
        tile = w.list ? min(max(w.list[e], 0), L.n_tiles - 1) : e;
        flags = 1 << 8;
      }
      const TileValid tv = tile_valid(L, tile);
#pragma unroll
      for (int j = 0; j < SUB; ++j) {
        const bool full = tv.full || (L.kind == 1 && (j + 1) * KVH <= tv.vlen);  // Skiparse: pads at the tail
        flags |= full ? 0 : 1 << j;
      }
    }
    tile_v = tile;
    flags_v = flags;
  }
  // entries lo .. hi must lie in the window (hi - lo < 64)
  __device__ __forceinline__ void cover(const DevLayout& L, const WaveWork& w, const int* sched,
                                        int len, int lo, int hi, int lane) {
    if (hi - base >= 64) fill(L, w, sched, len, lo, lane);
  }
  __device__ __forceinline__ int tile(int e) const {
    return __builtin_amdgcn_readlane(tile_v, e - base);
  }
  __device__ __forceinline__ int flags(int e) const {
    return __builtin_amdgcn_readlane(flags_v, e - base);
  }
};

// ---------------------------------------------------------------------------
// bf16 kernels. One wave owns 32 query rows (a 64-row query tile takes two
// waves) and at most 256 registers, so two waves share each SIMD.
//
// The walk over kv blocks is software-pipelined inside each wave, because
// gfx950 only overlaps MFMA and VALU work that is interleaved in the
// instruction stream. Step s runs two scheduling regions:
//   A: the 16 score MFMAs of block s+1, interleaved with the row maximum,
//      the running-max update and the first half of exp2/pack of block s;
//   B: the PV MFMAs of block s, interleaved with the second half of its
//      exp2/pack (each 16-key group of P feeds its MFMAs as soon as it is
//      packed).
// K blocks are staged two steps ahead and V blocks one step ahead, each
// double-buffered in LDS, with one barrier per step.

// Register staging of K and V blocks (KVH tokens x D channels) and their
// stores into LDS: K row-major, V transposed to V^T rows (one per channel)
// in the token order of the S^T accumulator (register r of block mb in
// half-wave h holds token 32*mb + 8*(r/4) + 4*h + r%4), built from 2-token x
// 8-channel pieces (two consecutive tokens land on two adjacent positions).
// Every LDS row is padded by 16 bytes: the 16 rows a half-wave reads at one
// column then start 16 bytes apart, which spreads them over all banks, and
// each fragment address is one base register plus an immediate offset.
// VOP: bf16 V already stored in that order (each 32-token block channel-major,
// positions in the order above), so V^T rows are filled by whole 16-byte
// chunks copied from contiguous loads.
template <int KVH, int D, int THREADS, bool F32IN, bool VOP = false>
struct BfTile {
  static_assert(!(VOP && F32IN), "the V operand layout is bf16");
  static constexpr int ES = F32IN ? 4 : 2;
  static constexpr int CPR_K = D / 8;               // 16-byte chunks per K row
  static constexpr int CPR_V = KVH / 8;             // 16-byte chunks per V^T row
  static constexpr int KS_ = CPR_K + 1;             // padded row strides, in uint4
  static constexpr int VS_ = CPR_V + 1;
  static constexpr int K_CHUNKS = KVH * CPR_K;
  static constexpr int K_PER_T = (K_CHUNKS + THREADS - 1) / THREADS;
  static constexpr int PAIRS = KVH / 2;
  static constexpr int V_PIECES = PAIRS * (D / 8);
  static constexpr int V_PER_T = (V_PIECES + THREADS - 1) / THREADS;
  static constexpr int V_CHUNKS = KVH * D / 8;      // VOP: 16-byte chunks per block
  static constexpr int V_CH_PER_T = (V_CHUNKS + THREADS - 1) / THREADS;
  static_assert(!VOP || V_CH_PER_T <= 2 * V_PER_T, "VOP chunks fit the staging registers");
  static constexpr int K_LDS = KVH * KS_;           // uint4 per K buffer
  static constexpr int V_LDS = D * VS_;             // uint4 per V^T buffer
  uint4 kreg[K_PER_T];
  uint4 vreg[V_PER_T][2];

  // first token of V^T position pair q2 (positions 2*q2, 2*q2 + 1 hold
  // tokens t0, t0 + 1): position 16*ps + 8*h + i of key group ps holds token
  // 16*ps + 8*(i / 4) + 4*h + i % 4
  static __device__ __forceinline__ int v_pair_token(int q2) {
    const int pos = 2 * q2;
    return 16 * (pos >> 4) + 8 * ((pos >> 2) & 1) + 4 * ((pos >> 3) & 1) + (pos & 3);
  }

  // block_off: byte offset of the kv block inside this (b, head) slice
  __device__ __forceinline__ void load_k(rsrc_t rk, uint32_t block_off, int tid) {
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int c = tid + i * THREADS;            // chunk c = 8 elements at element 8*c
      if (K_CHUNKS % THREADS == 0 || c < K_CHUNKS)
        kreg[i] = bload8<F32IN>(rk, tid * 8 * ES, block_off + i * THREADS * 8 * ES);
    }
  }
  __device__ __forceinline__ void load_v(rsrc_t rv, uint32_t block_off, int tid) {
    if constexpr (VOP) {
#pragma unroll
      for (int k = 0; k < V_CH_PER_T; ++k) {
        const int c = tid + k * THREADS;
        if (V_CHUNKS % THREADS == 0 || c < V_CHUNKS)
          vreg[k >> 1][k & 1] = bload8<false>(rv, tid * 16, block_off + k * THREADS * 16);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int u = tid + i * THREADS;
      if (V_PIECES % THREADS == 0 || u < V_PIECES) {
        const int q2 = u % PAIRS, cc = u / PAIRS;
        const uint32_t voff = (uint32_t)((v_pair_token(q2) * D + cc * 8) * ES);
        vreg[i][0] = bload8<F32IN>(rv, voff, block_off);
        vreg[i][1] = bload8<F32IN>(rv, voff, block_off + D * ES);
      }
    }
  }
  __device__ __forceinline__ void store_k(uint4* k_lds, int tid) const {
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int c = tid + i * THREADS;
      if (K_CHUNKS % THREADS == 0 || c < K_CHUNKS) k_lds[(c / CPR_K) * KS_ + c % CPR_K] = kreg[i];
    }
  }
  __device__ __forceinline__ void store_v(uint4* v_lds, int tid) const {
    if constexpr (VOP) {
      // chunk c of the block: 32-token block c / (4 D), channel (c / 4) % D,
      // positions 8 (c % 4) .. + 7 of that block
#pragma unroll
      for (int k = 0; k < V_CH_PER_T; ++k) {
        const int c = tid + k * THREADS;
        if (V_CHUNKS % THREADS == 0 || c < V_CHUNKS) {
          const int kb = c / (4 * D), ch = (c >> 2) - kb * D;
          v_lds[ch * VS_ + 4 * kb + (c & 3)] = vreg[k >> 1][k & 1];
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int u = tid + i * THREADS;
      if (V_PIECES % THREADS == 0 || u < V_PIECES) {
        const int q2 = u % PAIRS, cc = u / PAIRS;
        // positions 2*q2, 2*q2 + 1 of channel rows cc*8 .. cc*8+7
        uint32_t* dst = reinterpret_cast<uint32_t*>(v_lds + (cc * 8) * VS_) + q2;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int dw = e >> 1;
          dst[e * VS_ * 4] = (e & 1) ? perm_hi(vreg[i][0][dw], vreg[i][1][dw])
                                     : perm_lo(vreg[i][0][dw], vreg[i][1][dw]);
        }
      }
    }
  }
};

// max / sum of a value over the two half-waves (lanes l and l ^ 32)
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// S^T block (KVH kv tokens x 32 query rows) = K . Q^T; kb = K buffer + lane base
template <int KVH, int D>
__device__ __forceinline__ void bf_scores(const uint4* kb, const uint4 (&qf)[D / 16],
                                          f32x16_t (&sacc)[KVH / 32]) {
  constexpr int KS_ = D / 8 + 1;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
    for (int mb = 0; mb < KVH / 32; ++mb) {
      const uint4 kf = kb[mb * 32 * KS_ + 2 * ks];
      sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kf),
                                                         __builtin_bit_cast(bf16x8_t, qf[ks]),
                                                         ks == 0 ? f32x16_t{} : sacc[mb], 0, 0, 0);
    }
}

// Padded keys of a block (bit t of `real` clear for key t) get score -inf,
// so the softmax below needs no mask: they add nothing to the maximum and
// exp2 turns them into p = 0. The running maximum starts at -FLT_MAX rather
// than -inf, so even a block whose keys are all padding yields p = 0, not NaN.
// Register r of S^T block mb holds key 32*mb + 8*(r/4) + 4*half + r%4, so
// the lane mask of each select comes straight from `real` (half-wave 0 tests
// one bit, half-wave 1 the bit four above it): scalar bit extracts and one
// vector select per register.
template <int MB>
__device__ __forceinline__ void mask_scores(f32x16_t (&s)[MB], unsigned long long real) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = 32 * mb + 8 * (r >> 2) + (r & 3);
      const unsigned long long lo = ((real >> j) & 1ull) ? 0xFFFFFFFFull : 0ull;
      const unsigned long long hi = ((real >> (j + 4)) & 1ull) ? 0xFFFFFFFF00000000ull : 0ull;
      s[mb][r] = __builtin_amdgcn_inverse_ballot_w64(lo | hi) ? s[mb][r] : -INFINITY;
    }
}

// Row maximum of the raw scores (this lane's query row, both half-waves)
template <int MB>
__device__ __forceinline__ float bf_row_max(const f32x16_t (&s)[MB]) {
  float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) m4[r & 3] = fmaxf(m4[r & 3], s[mb][r]);
  return halves_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
}

// Lazy running-max update from the block's row maximum `hi` (raw score
// units, sl2 >= 0): m_run only moves when the block's scaled maximum exceeds
// it by more than `lazy`. Returns the factor O must be multiplied by.
__device__ __forceinline__ float bf_update_max(float hi, float sl2, float lazy, float& m_run,
                                               float& l_run) {
  const float mx = hi * sl2;
  float alpha = 1.0f;
  if (mx > m_run + lazy) {
    alpha = fast_exp2(m_run - mx);                       // 0 on the first block
    m_run = mx;
    l_run *= alpha;
  }
  return alpha;
}

// p = exp2(s * sl2 - m_run) for the 16-key groups PS0 .. PS1-1 of the block,
// packed to bf16 P^T operands; the packed (rounded) values are summed into
// l_run, so numerator and denominator use the same weights.
template <int MB, int PS0, int PS1>
__device__ __forceinline__ void bf_exp_pack(const f32x16_t (&s)[MB], float sl2, float m_run,
                                            float& l_run, uint4 (&pk)[2 * MB]) {
  const float nm = -m_run;
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
  float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
  for (int ps = PS0; ps < PS1; ++ps) {
    const int mb = ps >> 1, r0 = 8 * (ps & 1);
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = fast_exp2(fmaf(s[mb][r0 + i], sl2, nm));
    pk[ps] = make_uint4(pack2(p[0], p[1]), pack2(p[2], p[3]), pack2(p[4], p[5]), pack2(p[6], p[7]));
    acc0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[ps].x), ones, acc0, false);
    acc1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[ps].y), ones, acc1, false);
    acc0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[ps].z), ones, acc0, false);
    acc1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[ps].w), ones, acc1, false);
  }
  l_run += acc0 + acc1;
}

// O^T += V^T . P^T for the 16-key groups PS0 .. PS1-1; vb = V^T buffer + lane base
template <int KVH, int D, int PS0, int PS1>
__device__ __forceinline__ void bf_pv(const uint4* vb, const uint4 (&pk)[KVH / 16],
                                      f32x16_t (&oacc)[D / 32]) {
  constexpr int VS_ = KVH / 8 + 1;
#pragma unroll
  for (int ps = PS0; ps < PS1; ++ps)
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) {
      const uint4 vf = vb[cb * 32 * VS_ + 2 * ps];
      oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vf),
                                                         __builtin_bit_cast(bf16x8_t, pk[ps]),
                                                         oacc[cb], 0, 0, 0);
    }
}

// Scheduling hint for a region of NM MFMAs, each fed by one LDS read issued
// PRE MFMAs ahead, with up to NV VALU instructions placed after each MFMA.
template <int NM, int PRE, int NV>
__device__ __forceinline__ void interleave_hint() {
  __builtin_amdgcn_sched_group_barrier(0x100, PRE, 0);          // DS reads
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // one MFMA
    if (i < NM - PRE) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);         // VALU
  }
}

// exp2/pack and PV products of the current block, each 16-key group of P
// feeding its MFMAs as soon as it is packed
template <int KVH, int D>
__device__ __forceinline__ void bf_block_pv(const uint4* vb, const f32x16_t (&scur)[KVH / 32],
                                            float sl2, float m_run, float& l_run,
                                            f32x16_t (&oacc)[D / 32]) {
  constexpr int MB = KVH / 32, NPS = KVH / 16;
  uint4 pk[NPS];
  bf_exp_pack<MB, 0, NPS / 2>(scur, sl2, m_run, l_run, pk);
  bf_pv<KVH, D, 0, NPS / 2>(vb, pk, oacc);
  bf_exp_pack<MB, NPS / 2, NPS>(scur, sl2, m_run, l_run, pk);
  bf_pv<KVH, D, NPS / 2, NPS>(vb, pk, oacc);
}

// One pipelined step with the PV product one block behind: the score MFMAs
// of block s+1 and the PV MFMAs of block s-1 (whose P^T operands were packed
// during the previous step) around the exp2/pack work of block s, so no
// MFMA of the step waits on the step's own VALU work. Returns the row
// maximum of block s+1 (taken without its pad mask).
template <int KVH, int D>
__device__ __forceinline__ float bf_step_lag(const uint4* kb, const uint4* vb,
                                             const uint4 (&qf)[D / 16],
                                             f32x16_t (&snext)[KVH / 32],
                                             const f32x16_t (&scur)[KVH / 32], float sl2,
                                             float m_run, float& l_run,
                                             const uint4 (&pprev)[KVH / 16],
                                             uint4 (&pcur)[KVH / 16], f32x16_t (&oacc)[D / 32]) {
  constexpr int MB = KVH / 32, NPS = KVH / 16;
  bf_scores<KVH, D>(kb, qf, snext);
  bf_exp_pack<MB, 0, NPS>(scur, sl2, m_run, l_run, pcur);
  bf_pv<KVH, D, 0, NPS>(vb, pprev, oacc);
  const float hi = bf_row_max<MB>(snext);
  interleave_hint<(D / 16) * MB + NPS * (D / 32), 3, 4>();
  return hi;
}

// Q^T fragments for query row 32*rg + l32 of tile qt; a negative softmax
// scale is folded into Q (sign flip) so the softmax only needs a maximum.
// row_off: byte offset of the row in rq (past its end for a row that does
// not exist, which then reads as zeros).
template <int D, bool F32IN>
__device__ __forceinline__ void bf_load_q(rsrc_t rq, uint32_t row_off, int half,
                                          uint32_t qsign, uint4 (&qf)[D / 16]) {
  constexpr int ES = F32IN ? 4 : 2;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const uint4 x = bload8<F32IN>(rq, row_off + (ks * 16 + half * 8) * ES, 0);
    qf[ks] = make_uint4(x.x ^ qsign, x.y ^ qsign, x.z ^ qsign, x.w ^ qsign);
  }
}

// Normalise and write this wave's 32 output rows (and lse). NAT: the rows go
// to their natural positions in out [B, T*H*W, heads, d] (pad rows have none
// and are not written); lse stays in the tiled order.
template <int TILE, int D, bool F32IN, bool NAT = false>
__device__ __forceinline__ void bf_epilogue(const DevLayout& L, const AttnArgs& a, const WaveWork& ww,
                                            int rg, int l32, int half, const f32x16_t (&oacc)[D / 32],
                                            float m_run, float l_run) {
  const TileValid tq = tile_valid(L, ww.qt);
  const int qrow = 32 * rg + l32;
  const float lt = halves_sum(l_run);
  const bool real = row_is_real(L, tq, qrow);
  const float inv = (real && lt > 0.0f) ? 1.0f / lt : 0.0f;
  const long long orow = ww.head_row0 + (long long)ww.qt * TILE + qrow;
  long long obase = orow;
  bool store = true;
  if constexpr (NAT) {
    const int n = natural_index(L, ww.qt, qrow);
    const int b = ww.bh / L.heads, h = ww.bh - b * L.heads;
    store = n >= 0;
    obase = ((long long)b * L.n_tokens + max(n, 0)) * L.heads + h;
  }
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (!store) break;
      const int c0 = 32 * cb + 8 * g + 4 * half;
      const float o0 = oacc[cb][4 * g + 0] * inv, o1 = oacc[cb][4 * g + 1] * inv;
      const float o2 = oacc[cb][4 * g + 2] * inv, o3 = oacc[cb][4 * g + 3] * inv;
      if constexpr (F32IN) {
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + obase * D + c0) =
            make_float4(o0, o1, o2, o3);
      } else {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + obase * D + c0) =
            make_uint2(pack2(o0, o1), pack2(o2, o3));
      }
    }
  if (a.lse && half == 0) {
    a.lse[orow] = (real && lt > 0.0f) ? (m_run + __log2f(lt)) * 0.69314718055994531f : -INFINITY;
  }
}

constexpr float kLazyBf16 = 8.0f;

// One kernel for every bf16 / f32-input shape. Each schedule entry (a key
// tile) is walked as TILE/KVH kv blocks of KVH tokens. KVH = 32 for routed
// lists over 64-token tiles keeps the LDS buffers within 36 KB, so four
// workgroups (eight waves) fit a CU.
//
// Two walks: the pipelined one when every wave owns every block (routed
// lists, dense lists, query tiles sharing one list), and a plain
// double-buffered one for unions whose blocks some waves skip.
// NAT: Q is read from and O written to the natural order [B, T*H*W, heads, d]
// (the tile permute of Q and the inverse permute of O fused into the
// kernel's first load and last store); K and V stay tiled.
// VOP: bf16 V in the P.V operand layout (whole-chunk staging).
template <int TILE, int KVH, int D, int QPW, bool F32IN, int NBUF, bool NAT, bool VOP>
__global__ __launch_bounds__(64 * QPW * (TILE / 32)) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bf16_kernel(DevLayout L, AttnArgs a, int n_work) {
  constexpr int WPQ = TILE / 32;         // waves per query tile
  constexpr int SUB = TILE / KVH;        // kv blocks per tile
  constexpr int MB = KVH / 32;
  constexpr int NPS = KVH / 16;
  constexpr int THREADS = 64 * QPW * WPQ;
  using IO = BfTile<KVH, D, THREADS, F32IN, VOP>;
  static_assert(TILE == 32 || TILE == 64, "tiles of 32 or 64 tokens");
  static_assert(!VOP || TILE == 64, "the V operand layout has 64-token tiles");

  static_assert(NBUF == 2 || NBUF == 4, "two or four K/V buffers");
  __shared__ uint4 k_lds[NBUF][IO::K_LDS];
  __shared__ uint4 v_lds[NBUF][IO::V_LDS];
  extern __shared__ int sched[];         // QPW > 1: the schedule (n_tiles entries)
  static_assert(THREADS * 4 <= IO::K_LDS * 16, "scan scratch fits one K buffer");
  static_assert(4096 <= IO::V_LDS * 16, "marks of 4096 tiles fit one V buffer");

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int rg = wave % WPQ;

  const WaveWork ww = wave_work<QPW, WPQ>(L, a, n_work, wave);
  // the marks (n_tiles bytes, n_tiles <= 4096 on this path) and the scan
  // borrow the second K/V buffers, which the walk first writes after the
  // schedule's closing barrier
  int len;
  bool shared = true;
  if constexpr (QPW > 1)
    len = build_schedule<QPW, WPQ>(L, ww, reinterpret_cast<uint32_t*>(v_lds[1]),
                                   reinterpret_cast<int*>(k_lds[1]), sched, tid, lane, shared);
  else len = ww.cnt;

  const long long head_bytes = L.n_padded * D * IO::ES;
  rsrc_t rq;
  uint32_t q_row_off;
  {
    const int qrow = 32 * rg + l32, qt = min(ww.qt, L.n_tiles - 1);
    if constexpr (NAT) {
      // one (b, head) of natural Q: rows n at stride heads * d elements
      const int b = ww.bh / L.heads, h = ww.bh - b * L.heads;
      const long long first = ((long long)b * L.n_tokens * L.heads + h) * D * IO::ES;
      rq = make_rsrc(static_cast<const char*>(a.q) + first,
                     ((long long)L.n_tokens * L.heads - h) * D * IO::ES);
      const int n = natural_index(L, qt, qrow);
      q_row_off = n < 0 ? 0x7FFFFF00u : (uint32_t)((long long)n * L.heads * D * IO::ES);
    } else {
      rq = make_rsrc(static_cast<const char*>(a.q) + ww.head_row0 * D * IO::ES, head_bytes);
      q_row_off = (uint32_t)((qt * TILE + qrow) * D * IO::ES);
    }
  }
  const rsrc_t rk = make_rsrc(static_cast<const char*>(a.k) + ww.head_row0 * D * IO::ES, head_bytes);
  const rsrc_t rv = make_rsrc(static_cast<const char*>(a.v) + ww.head_row0 * D * IO::ES, head_bytes);

  // kept > 0 (a zero scale gives uniform weights) so a masked -inf stays -inf
  const float sl2 = fmaxf(fabsf(a.scale_log2), FLT_MIN);
  uint4 qf[D / 16];
  bf_load_q<D, F32IN>(rq, q_row_off, half, a.scale_log2 < 0.0f ? 0x80008000u : 0u, qf);
  f32x16_t oacc[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) oacc[cb] = f32x16_t{};
  float m_run = -FLT_MAX, l_run = 0.0f;

  const int steps = len * SUB;
  IO io;
  SchedWindow<QPW, SUB, KVH> win;
  win.fill(L, ww, sched, len, 0, lane);
  // the window must hold the entries of steps s .. s+2 before step s
  auto cover = [&](int s) {
    win.cover(L, ww, sched, len, s / SUB, min(s + 2, max(steps - 1, 0)) / SUB, lane);
  };
  // byte offset of kv block `step`; steps past the end reload the last
  // block into a buffer nobody reads again
  auto block_off = [&](int step) -> uint32_t {
    step = min(step, steps - 1);
    return (uint32_t)((win.tile(step / SUB) * TILE + (step % SUB) * KVH) * D * IO::ES);
  };
  const int k_lane = l32 * IO::KS_ + half;
  const int v_lane = l32 * IO::VS_ + half;
  // pad mask of block s: bit t set for real key t, `full` when all are
  auto block_bits = [&](int s, bool& full) -> unsigned long long {
    full = ((win.flags(s / SUB) >> (s % SUB)) & 1) == 0;
    if (full) return ~0ull;
    return kv_pad_ballot<MB>(L, win.tile(s / SUB), (s % SUB) * KVH, lane);
  };
  // running-max update from a block's row maximum and the (rare) rescale of O
  auto update_max = [&](float hi) __attribute__((always_inline)) {
    const float alpha = bf_update_max(hi, sl2, kLazyBf16, m_run, l_run);
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {   // lanes whose max did not move multiply by 1
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) oacc[cb] *= alpha;
    }
  };

  if (shared) {
    // Pipelined walk with the PV product one block behind, over a ring of
    // NBUF K and NBUF V buffers (block j in buffer j % NBUF). Step s takes
    // K(s+1) and V(s-1) from their buffers, and stages K(s+LK) and V(s+LV),
    // loaded at the step's start, at its end. With NBUF = 2 (LK = 2, LV = 0)
    // every step ends in a barrier; with NBUF = 4 (LK = 3, LV = 1) only odd
    // steps do, which still puts a barrier between each store and the first
    // read of that block, and between the last read of a buffer and the
    // store that refills it. The row maximum of block s+1 is taken during
    // step s; at the last steps the scores of a clamped block are computed
    // and never used. Before the first step the V buffer of "block -1" and
    // its P operands are zero, so the first step's PV product adds nothing.
    constexpr int LK = NBUF == 4 ? 3 : 2, LV = NBUF == 4 ? 1 : 0;
    f32x16_t s_a[MB], s_b[MB];
    uint4 pk_a[NPS], pk_b[NPS];
#pragma unroll
    for (int i = 0; i < NPS; ++i) pk_b[i] = make_uint4(0u, 0u, 0u, 0u);
    float hi = 0.0f;
    if (steps > 0) {
#pragma unroll
      for (int j = 0; j < LK; ++j) {
        io.load_k(rk, block_off(j), tid);
        io.store_k(k_lds[j], tid);
      }
#pragma unroll
      for (int j = 0; j < LV; ++j) {
        io.load_v(rv, block_off(j), tid);
        io.store_v(v_lds[j], tid);
      }
      for (int i = tid; i < IO::V_LDS; i += THREADS) v_lds[NBUF - 1][i] = make_uint4(0u, 0u, 0u, 0u);
      __syncthreads();
      bf_scores<KVH, D>(k_lds[0] + k_lane, qf, s_a);
      hi = bf_row_max<MB>(s_a);
      __syncthreads();                   // K buffer 0 is refilled before the next barrier
    }
    // `hi` is block s's row maximum taken without its pad mask; a padded
    // block (rare) is masked and its maximum retaken at the step's start.
    // Entering step s, O holds the products of blocks up to s-2 on the scale
    // of the running maximum before step s-1's update, and P(s-1) is on the
    // scale after it; step s-1's rescale factor `alpha` is applied to O
    // first, then the running maximum takes block s.
    float alpha = 1.0f;
    bool pending = false;
    auto rescale_o = [&]() __attribute__((always_inline)) {
      if (pending) {                     // lanes whose max did not move multiply by 1
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb) oacc[cb] *= alpha;
      }
    };
    // I = s % NBUF; even steps take (s_a, s_b, pk_b, pk_a), odd ones the reverse
    auto step = [&](auto phase, int s, f32x16_t (&scur)[MB], f32x16_t (&snext)[MB],
                    const uint4 (&pprev)[NPS], uint4 (&pcur)[NPS]) __attribute__((always_inline)) {
      constexpr int I = decltype(phase)::value;
      win.cover(L, ww, sched, len, s / SUB, min(s + LK, steps - 1) / SUB, lane);
      io.load_k(rk, block_off(s + LK), tid);
      io.load_v(rv, block_off(s + LV), tid);
      rescale_o();
      bool full;
      const unsigned long long bits = block_bits(s, full);
      if (!full) {
        mask_scores<MB>(scur, bits);
        hi = bf_row_max<MB>(scur);
      }
      alpha = bf_update_max(hi, sl2, kLazyBf16, m_run, l_run);
      pending = __builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0;
      hi = bf_step_lag<KVH, D>(k_lds[(I + 1) % NBUF] + k_lane, v_lds[(I + NBUF - 1) % NBUF] + v_lane,
                               qf, snext, scur, sl2, m_run, l_run, pprev, pcur, oacc);
      __builtin_amdgcn_sched_barrier(0);  // the staging stores wait for their loads here
      io.store_k(k_lds[(I + LK) % NBUF], tid);
      io.store_v(v_lds[(I + LV) % NBUF], tid);
      if (NBUF == 2 || (I & 1)) __syncthreads();
    };
    // after the last step its rescale and its block's PV product remain;
    // the last P operands are left in pk_b
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    using C3 = std::integral_constant<int, 3>;
    for (int s = 0; s < steps; s += NBUF) {
      step(C0{}, s, s_a, s_b, pk_b, pk_a);
      if (s + 1 >= steps) {
#pragma unroll
        for (int i = 0; i < NPS; ++i) pk_b[i] = pk_a[i];
        break;
      }
      step(C1{}, s + 1, s_b, s_a, pk_a, pk_b);
      if constexpr (NBUF == 4) {
        if (s + 2 >= steps) break;
        step(C2{}, s + 2, s_a, s_b, pk_b, pk_a);
        if (s + 3 >= steps) {
#pragma unroll
          for (int i = 0; i < NPS; ++i) pk_b[i] = pk_a[i];
          break;
        }
        step(C3{}, s + 3, s_b, s_a, pk_a, pk_b);
      }
    }
    if (steps > 0) {
      __syncthreads();                   // the last V block is visible to every wave
      rescale_o();
      bf_pv<KVH, D, 0, NPS>(v_lds[(steps - 1) % NBUF] + v_lane, pk_b, oacc);
    }
  } else {
    // Plain double-buffered walk over a union: block s+1 is staged while
    // block s is computed by the waves whose list holds it.
    if (steps > 0) {
      io.load_k(rk, block_off(0), tid);
      io.load_v(rv, block_off(0), tid);
      io.store_k(k_lds[0], tid);
      io.store_v(v_lds[0], tid);
      __syncthreads();
    }
    for (int s = 0; s < steps; ++s) {
      const int P = s & 1;
      const bool has_next = s + 1 < steps;
      cover(s);
      if (has_next) {
        io.load_k(rk, block_off(s + 1), tid);
        io.load_v(rv, block_off(s + 1), tid);
      }
      if ((win.flags(s / SUB) >> (8 + ww.slot)) & 1) {
        f32x16_t sc[MB];
        bf_scores<KVH, D>(k_lds[P] + k_lane, qf, sc);
        bool full;
        const unsigned long long bits = block_bits(s, full);
        if (!full) mask_scores<MB>(sc, bits);
        update_max(bf_row_max<MB>(sc));
        bf_block_pv<KVH, D>(v_lds[P] + v_lane, sc, sl2, m_run, l_run, oacc);
        interleave_hint<(KVH / 16) * (D / 32), 3, 4>();
      }
      if (has_next) {
        io.store_k(k_lds[P ^ 1], tid);
        io.store_v(v_lds[P ^ 1], tid);
      }
      __syncthreads();
    }
  }
  if (!ww.active) return;
  bf_epilogue<TILE, D, F32IN, NAT>(L, a, ww, rg, l32, half, oacc, m_run, l_run);
}

// ---------------------------------------------------------------------------
// fp8 e4m3 variant (FPSAttention, Approach: FP8 on the same tiles as the
// sparsity). Q/K/V are e4m3 codes with one fp32 scale per (b, head, tile);
// tiles are 64 tokens, d = 128, and one wave owns 32 query rows (two waves
// per query tile, two waves per SIMD), as in the bf16 kernel.
//   S^T = Kc . Qc^T   v_mfma_scale_f32_32x32x64_f8f6f4 with unit block
//                     scales; the exponent of p is S * cs(tile) with
//                     cs = q_scale * k_scale(tile) * sigma * log2(e);
//   O^T += Vc^T . P8^T, P8 = e4m3(p * ps(tile)), ps = 112 * v_scale(tile) /
//                     max_t v_scale (112 for an all-zero V tile, whose codes
//                     are all zero).
// ps is folded into the exponent (p * ps = exp2(S * cs - m + log2 ps)) and
// the running sum adds the tile's sum of p * ps times 1/ps (the four-tile
// walk sums the rounded P8 on the matrix core, the one-tile walk the
// unrounded values on the VALU). The lazy-rescale
// threshold is 2 (p <= 4), so p * ps <= 448 fits e4m3, and one O accumulator
// scale serves the whole walk: O = acc * max v_scale / 112 / l.
// The two half-waves each hold 32 of a tile's 64 kv tokens (element e of a
// lane in half-wave h is token 32*(e/16) + 8*((e%16)/4) + 4*h + e%4), so one
// K=64 MFMA covers the whole tile in the PV product. The walks are those of
// the bf16 kernel: pipelined when every wave owns every tile, a plain
// double-buffered union walk otherwise; LDS rows are padded by 16 bytes. The
// one-tile walk over V in the operand layout copies K and V^T straight into
// LDS (F8Dma); the others stage them through registers (F8Tile).
constexpr float kP8Scale = 112.0f;          // 448 / 2^2
constexpr float kLazyFp8 = 2.0f;

constexpr int kK8Stride = 9;                // K rows: 8 chunks of 16 codes + 16 B pad
constexpr int kV8Stride = 5;                // V^T rows: 4 chunks + 16 B pad

__device__ __forceinline__ i32x8_t cat8(uint4 x, uint4 y) {
  i32x8_t r;
  r[0] = (int)x.x; r[1] = (int)x.y; r[2] = (int)x.z; r[3] = (int)x.w;
  r[4] = (int)y.x; r[5] = (int)y.y; r[6] = (int)y.z; r[7] = (int)y.w;
  return r;
}

// Register staging of an fp8 K/V tile and its stores into LDS (K row-major,
// V transposed to V^T rows in the token order above, from 4-token x
// 16-channel pieces). VOP: V codes arrive already in that V^T order (the
// P.V operand layout written by the V-operand quantiser), so they are
// copied row by row like K, with no byte permutes.
template <int THREADS, bool VOP = false>
struct F8Tile {
  static constexpr int TILE = 64, D = 128;
  static constexpr int K_PER_T = TILE * D / 16 / THREADS;   // 16-code chunks per thread
  static constexpr int V_PIECES = (TILE / 4) * (D / 16);
  static constexpr int V_PER_T = (V_PIECES + THREADS - 1) / THREADS;
  static constexpr int K_LDS = TILE * kK8Stride;            // uint4 per K buffer
  static constexpr int V_LDS = D * kV8Stride;               // uint4 per V^T buffer
  uint4 kreg[K_PER_T];
  uint4 vreg[V_PER_T][4];

  __device__ __forceinline__ void load_k(rsrc_t rk, uint32_t tile_off, int tid) {
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) kreg[i] = bload(rk, tid * 16, tile_off + i * THREADS * 16);
  }
  __device__ __forceinline__ void store_k(uint4* k_lds, int tid) const {
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int c = tid + i * THREADS;
      k_lds[(c >> 3) * kK8Stride + (c & 7)] = kreg[i];
    }
  }
  static constexpr int VOP_PER_T = D * TILE / 16 / THREADS;    // 16-byte V^T chunks per thread
  static_assert(!VOP || VOP_PER_T <= 4 * V_PER_T, "V^T staging fits the V registers");
  // piece u: tokens 4*(u % 16) .. +3 x channels 16*(u / 16) .. +15
  __device__ __forceinline__ void load_v(rsrc_t rv, uint32_t tile_off, int tid) {
    if constexpr (VOP) {     // chunk c: V^T row c / 4 (a channel), bytes 16 (c % 4) ..
#pragma unroll
      for (int i = 0; i < VOP_PER_T; ++i) vreg[i / 4][i % 4] = bload(rv, tid * 16, tile_off + i * THREADS * 16);
      return;
    }
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int u = tid + i * THREADS;
      if (V_PIECES % THREADS == 0 || u < V_PIECES) {
        const uint32_t voff = (uint32_t)(4 * (u & 15) * D + 16 * (u >> 4));
#pragma unroll
        for (int j = 0; j < 4; ++j) vreg[i][j] = bload(rv, voff, tile_off + j * D);
      }
    }
  }
  // tokens t0..t0+3 sit at V^T byte positions p0..p0+3 with
  // p0 = 32*h + 16*(t0/32) + 4*((t0/8)%4), h = (t0/4)%2
  __device__ __forceinline__ void store_v(uint4* v_lds, int tid) const {
    if constexpr (VOP) {
#pragma unroll
      for (int i = 0; i < VOP_PER_T; ++i) {
        const int c = tid + i * THREADS;
        v_lds[(c >> 2) * kV8Stride + (c & 3)] = vreg[i / 4][i % 4];
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int u = tid + i * THREADS;
      if (V_PIECES % THREADS == 0 || u < V_PIECES) {
        const int cg = u >> 4, tok0 = 4 * (u & 15);
        const int hh = (tok0 >> 2) & 1, A = tok0 >> 5, B = (tok0 >> 3) & 3;
        const int p0 = 32 * hh + 16 * A + 4 * B;
        uint32_t* dst = reinterpret_cast<uint32_t*>(v_lds + (16 * cg) * kV8Stride) + (p0 >> 2);
#pragma unroll
        for (int dw = 0; dw < 4; ++dw) {
          const uint32_t x01l = __builtin_amdgcn_perm(vreg[i][1][dw], vreg[i][0][dw], 0x05010400u);
          const uint32_t x01h = __builtin_amdgcn_perm(vreg[i][1][dw], vreg[i][0][dw], 0x07030602u);
          const uint32_t x23l = __builtin_amdgcn_perm(vreg[i][3][dw], vreg[i][2][dw], 0x05010400u);
          const uint32_t x23h = __builtin_amdgcn_perm(vreg[i][3][dw], vreg[i][2][dw], 0x07030602u);
          dst[(4 * dw + 0) * kV8Stride * 4] = __builtin_amdgcn_perm(x23l, x01l, 0x05040100u);
          dst[(4 * dw + 1) * kV8Stride * 4] = __builtin_amdgcn_perm(x23l, x01l, 0x07060302u);
          dst[(4 * dw + 2) * kV8Stride * 4] = __builtin_amdgcn_perm(x23h, x01h, 0x05040100u);
          dst[(4 * dw + 3) * kV8Stride * 4] = __builtin_amdgcn_perm(x23h, x01h, 0x07060302u);
        }
      }
    }
  }
};

// Direct copies (buffer_load ... lds, 16 bytes a lane) of one fp8 tile into
// the padded LDS rows, for one-tile workgroups (two waves) with V in the
// P.V operand layout, where K and V^T are both plain row copies. Copy j of
// wave w fills the 1 KB of LDS chunks 64 * (w + 2 j) .. +63; chunk p is row
// p / RS, chunk p % RS of the tile (the pad chunk takes a copy of the row's
// last chunk and is never read). K: 64 rows of 8 chunks (9 copies), V^T: 128
// rows of 4 chunks (10 copies). Source offsets are per lane, kept in
// registers for the whole walk.
typedef __attribute__((address_space(3))) void lds_void_t;
__device__ __forceinline__ void dma16(rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, (int)voff, (int)soff, 0, 0);
}
// s_waitcnt with vmcnt 0 (expcnt and lgkmcnt at their maxima)
__device__ __forceinline__ void wait_vmcnt0() {
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
}
struct F8Dma {
  static constexpr int KN = 64 * kK8Stride / 64, VN = 128 * kV8Stride / 64;   // 9, 10 copies
  static_assert(KN == 9 && VN == 10, "copy counts of the padded rows");
  uint32_t kvo[5], vvo[5];
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      const int p = 64 * (wave + 2 * j) + lane;
      kvo[j] = (uint32_t)((p / kK8Stride) * 128 + min(p % kK8Stride, kK8Stride - 2) * 16);
      vvo[j] = (uint32_t)((p / kV8Stride) * 64 + min(p % kV8Stride, kV8Stride - 2) * 16);
    }
  }
  // the tile at byte offset soff (wave-uniform) of rk / rv
  __device__ __forceinline__ void issue_k(rsrc_t rk, uint4* lds, uint32_t soff, int wave) const {
#pragma unroll
    for (int j = 0; j < 5; ++j)
      if (wave + 2 * j < KN) dma16(rk, reinterpret_cast<char*>(lds) + 1024 * (wave + 2 * j), kvo[j], soff);
  }
  __device__ __forceinline__ void issue_v(rsrc_t rv, uint4* lds, uint32_t soff, int wave) const {
#pragma unroll
    for (int j = 0; j < 5; ++j)
      dma16(rv, reinterpret_cast<char*>(lds) + 1024 * (wave + 2 * j), vvo[j], soff);
  }
};

// S^T (64 kv tokens x 32 query rows, raw code products) from one K buffer
// (kb = buffer + lane base)
__device__ __forceinline__ void f8_scores(const uint4* kb, const i32x8_t (&qf)[2], f32x16_t (&sacc)[2]) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const i32x8_t kf = cat8(kb[mb * 32 * kK8Stride + 4 * ks], kb[mb * 32 * kK8Stride + 4 * ks + 1]);
      sacc[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qf[ks], ks == 0 ? f32x16_t{} : sacc[mb],
                                                                 0, 0, 0, 127, 0, 127);
    }
}

// P8^T = e4m3(exp2(S * cs + e0)) for the tile's 32 scores of this lane (e0 =
// log2 ps - m_run). VSUM: also returns the sum of the unrounded p * ps (the
// one-tile walk; the four-tile walk sums the rounded values on the matrix
// core, f8_rowsum).
template <bool VSUM>
__device__ __forceinline__ float f8_exp_pack(const f32x16_t (&s)[2], float cs, float e0, i32x8_t& pk) {
  float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int mb = i >> 2, r0 = 4 * (i & 3);
    const float x0 = fmaf(s[mb][r0 + 0], cs, e0);
    const float p0 = fast_exp2(x0);
    const float p1 = fast_exp2(fmaf(s[mb][r0 + 1], cs, e0));
    const float p2 = fast_exp2(fmaf(s[mb][r0 + 2], cs, e0));
    const float p3 = fast_exp2(fmaf(s[mb][r0 + 3], cs, e0));
    if constexpr (VSUM) {
      acc0 = i == 0 ? p0 + p1 : acc0 + (p0 + p1);
      acc1 = i == 0 ? p2 + p3 : acc1 + (p2 + p3);
    }
    // the second conversion fills the upper half that the first leaves as it
    // was, so the first may start from any dead word (here x0's) rather than
    // a zero that would take a move
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, __float_as_int(x0), false);
    pk[i] = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, w, true);
  }
  return acc0 + acc1;
}

// Row sums of the packed P8 on the matrix core. Read as the B operand of a
// 16x16x128 product, lane l of pk is column l % 16 and k-group l / 16, and
// holds query (l % 16) + 16 * ((l / 16) % 2), key half l / 32. The A operand
// (sel) is 1.0 (e4m3 0x38) where the k-group's parity equals bit 2 of the
// row, so output row m, column n sums both key halves of query
// n + 16 * ((m / 4) % 2); lane l receives rows 4 * (l / 16) .. +3 of column
// l % 16, which are the full 64-key sum of its own query l % 32 (in both
// half-waves). In the one-tile walk the extra product and its operands cost
// more registers than the wave has, so that walk keeps the VALU sum.
__device__ __forceinline__ i32x8_t f8_rowsum_selector(int lane) {
  const int v = (((lane >> 4) & 1) == (((lane & 15) >> 2) & 1)) ? 0x38383838 : 0;
  return i32x8_t{v, v, v, v, v, v, v, v};
}
__device__ __forceinline__ float f8_rowsum(const i32x8_t& sel, const i32x8_t& pk) {
  const f32x4_t r = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sel, pk, f32x4_t{}, 0, 0, 0, 127, 0, 127);
  return r[0];
}

// O^T += Vc^T . P8^T (vb = V^T buffer + lane base)
__device__ __forceinline__ void f8_pv(const uint4* vb, const i32x8_t& pk, f32x16_t (&oacc)[4]) {
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    const i32x8_t vf = cat8(vb[cb * 32 * kV8Stride], vb[cb * 32 * kV8Stride + 1]);
    oacc[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pk, oacc[cb], 0, 0, 0, 127, 0, 127);
  }
}

// NAT: O is written to the natural order [B, T*H*W, heads, d] (the inverse
// tile permute folded into the last store; pad rows have no natural position
// and are not written); Q, K, V codes and the lse stay tiled.
template <int QPW, bool VOP = false, bool NAT = false>
__global__ __launch_bounds__(128 * QPW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fp8_kernel(DevLayout L, AttnArgs a, int n_work) {
  constexpr int TILE = 64, D = 128, WPQ = 2, MB = 2, CB = 4, SUB = 1, KVH = 64;
  constexpr int THREADS = 64 * QPW * WPQ;
  using IO = F8Tile<THREADS, VOP>;

  // one-tile walks with V in the operand layout copy K and V straight into LDS
  constexpr bool DMA = VOP && QPW == 1;
  // separate arrays per buffer, so that reads of one buffer need not wait for
  // copies still in flight into the other
  __shared__ uint4 k_lds0[IO::K_LDS], k_lds1[IO::K_LDS];   // 64 rows x (128 + 16) B
  __shared__ uint4 v_lds0[IO::V_LDS], v_lds1[IO::V_LDS];   // V^T: 128 rows x (64 + 16) B
  auto k_buf = [&](int p) -> uint4* { return p ? k_lds1 : k_lds0; };
  auto v_buf = [&](int p) -> uint4* { return p ? v_lds1 : v_lds0; };
  extern __shared__ int sched[];
  static_assert(THREADS * 4 <= IO::K_LDS * 16, "scan scratch fits one K buffer");
  static_assert(4096 <= IO::V_LDS * 16, "marks of 4096 tiles fit one V buffer");

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int rg = wave % WPQ;

  const WaveWork ww = wave_work<QPW, WPQ>(L, a, n_work, wave);
  int len;
  bool shared = true;
  if constexpr (QPW > 1)
    len = build_schedule<QPW, WPQ>(L, ww, reinterpret_cast<uint32_t*>(v_buf(1)),
                                   reinterpret_cast<int*>(k_buf(1)), sched, tid, lane, shared);
  else len = ww.cnt;

  const long long head_bytes = L.n_padded * D;
  const rsrc_t rq = make_rsrc(static_cast<const uint8_t*>(a.q) + ww.head_row0 * D, head_bytes);
  const rsrc_t rk = make_rsrc(static_cast<const uint8_t*>(a.k) + ww.head_row0 * D, head_bytes);
  const rsrc_t rv = make_rsrc(static_cast<const uint8_t*>(a.v) + ww.head_row0 * D, head_bytes);
  const float* ksc = a.k_scale + (long long)ww.bh * L.n_tiles;
  const float* vsc = a.v_scale + (long long)ww.bh * L.n_tiles;

  // largest v scale of this (b, head): P is scaled by v_scale(tile) / wmax
  float wmax = 0.0f;
  for (int t = lane; t < L.n_tiles; t += 64) wmax = fmaxf(wmax, vsc[t]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) wmax = fmaxf(wmax, __shfl_xor(wmax, off));
  const float inv_wmax = wmax > 0.0f ? 1.0f / wmax : 0.0f;
  const int qt_c = min(ww.qt, L.n_tiles - 1);
  // a negative softmax scale is folded into Q (sign bit of every code); the
  // exponent scale is kept positive so that -inf stays -inf
  const uint32_t qsign = a.scale_log2 < 0.0f ? 0x80808080u : 0u;
  const float qk_base = a.q_scale[(long long)ww.bh * L.n_tiles + qt_c] * fabsf(a.scale_log2);

  // Q codes as B operands: query row 32*rg + l32, bytes 64*ks + 32*half .. +31
  i32x8_t qf[2];
  {
    const uint32_t row_off = (uint32_t)((qt_c * TILE + 32 * rg + l32) * D);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 x = bload(rq, row_off + 64 * ks + 32 * half, 0);
      uint4 y = bload(rq, row_off + 64 * ks + 32 * half + 16, 0);
      x = make_uint4(x.x ^ qsign, x.y ^ qsign, x.z ^ qsign, x.w ^ qsign);
      y = make_uint4(y.x ^ qsign, y.y ^ qsign, y.z ^ qsign, y.w ^ qsign);
      qf[ks] = cat8(x, y);
    }
  }

  f32x16_t oacc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) oacc[cb] = f32x16_t{};
  float m_run = -FLT_MAX, l_run = 0.0f;

  const int steps = len;
  IO io;
  SchedWindow<QPW, SUB, KVH> win;
  // per-tile exponent scale, log2 ps and 1/ps of the window's tiles (lane i: entry base + i)
  float cs_v = 0.0f, lps_v = 0.0f, ips_v = 1.0f;
  auto fill = [&](int base) {
    win.fill(L, ww, sched, len, base, lane);
    const int t = win.tile_v;
    const float vs = vsc[t];
    float ps = vs > 0.0f ? fmaxf(kP8Scale * vs * inv_wmax, 0x1p-60f) : kP8Scale;
    cs_v = fmaxf(qk_base * ksc[t], FLT_MIN);         // > 0, so a masked -inf stays -inf
    lps_v = __log2f(ps);
    ips_v = 1.0f / ps;
  };
  fill(0);
  auto cover = [&](int s) {
    if (min(s + 2, max(steps - 1, 0)) - win.base >= 64) fill(s);
  };
  auto rd = [&](float v, int s) { return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), s - win.base)); };
  auto tile_off = [&](int step) -> uint32_t {
    step = min(step, steps - 1);
    return (uint32_t)(win.tile(step) * TILE * D);
  };
  const int k_lane = l32 * kK8Stride + 2 * half;
  const int v_lane = l32 * kV8Stride + 2 * half;
  // row sums on the matrix core for the four-tile walk (full sums in both half-waves)
  constexpr bool MSUM = QPW > 1;
  const i32x8_t rsel = f8_rowsum_selector(lane);
  // pad mask, running-max update (rare rescale of O) and exp2/pack of block
  // s; returns the packed P8^T operand
  auto softmax = [&](int s, f32x16_t (&sc)[MB], float hi) __attribute__((always_inline)) {
    const float cs = rd(cs_v, s);
    const float mx = hi * cs;
    float alpha = 1.0f;
    if (mx > m_run + kLazyFp8) {
      alpha = fast_exp2(m_run - mx);
      m_run = mx;
      l_run *= alpha;
    }
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {   // lanes whose max did not move multiply by 1
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) oacc[cb] *= alpha;
    }
    i32x8_t pk;
    const float psum = f8_exp_pack<!MSUM>(sc, cs, rd(lps_v, s) - m_run, pk);
    l_run = fmaf(MSUM ? f8_rowsum(rsel, pk) : psum, rd(ips_v, s), l_run);
    return pk;
  };
  // pad mask of block s (s < steps) applied to its scores
  auto mask_block = [&](int s, f32x16_t (&sc)[MB]) __attribute__((always_inline)) {
    if ((win.flags(s) & 1) != 0) mask_scores<MB>(sc, kv_pad_ballot<MB>(L, win.tile(s), 0, lane));
  };

  if (shared) {
    // Pipelined walk: step s computes the scores of tile s+1 and the PV
    // products of tile s under the softmax of tile s (buffers as in the
    // bf16 kernel: V(s) in V buffer P, K(s+1) in K buffer P^1; K(s+2) and
    // V(s+1) are staged into K buffer P and V buffer P^1).
    f32x16_t s_a[MB], s_b[MB];
    float hi = 0.0f;
    F8Dma dma;
    const int w2 = wave & 1;                 // a one-tile workgroup has two waves
    if constexpr (DMA) dma.init(w2, lane);
    if (steps > 0) {
      if constexpr (DMA) {
        dma.issue_k(rk, k_buf(0), tile_off(0), w2);
        dma.issue_v(rv, v_buf(0), tile_off(0), w2);
        dma.issue_k(rk, k_buf(1), tile_off(1), w2);
        wait_vmcnt0();
      } else {
        io.load_k(rk, tile_off(0), tid);
        io.load_v(rv, tile_off(0), tid);
        io.store_k(k_buf(0), tid);
        io.store_v(v_buf(0), tid);
        io.load_k(rk, tile_off(1), tid);
        io.store_k(k_buf(1), tid);
      }
      __syncthreads();
      f8_scores(k_buf(0) + k_lane, qf, s_a);
      mask_block(0, s_a);
      hi = bf_row_max<MB>(s_a);
      __syncthreads();                   // K buffer 0 is refilled during step 0
    }
    auto step = [&](auto parity, int s, f32x16_t (&scur)[MB],
                    f32x16_t (&snext)[MB]) __attribute__((always_inline)) {
      constexpr int P = decltype(parity)::value;
      cover(s);
      if constexpr (DMA) {
        dma.issue_k(rk, k_buf(P), tile_off(s + 2), w2);
        dma.issue_v(rv, v_buf(P ^ 1), tile_off(s + 1), w2);
      } else {
        io.load_k(rk, tile_off(s + 2), tid);
        io.load_v(rv, tile_off(s + 1), tid);
      }
      f8_scores(k_buf(P ^ 1) + k_lane, qf, snext);
      const i32x8_t pk = softmax(s, scur, hi);
      f8_pv(v_buf(P) + v_lane, pk, oacc);
      if (s + 1 < steps) mask_block(s + 1, snext);   // masked before its maximum is taken
      hi = bf_row_max<MB>(snext);
      interleave_hint<8, 2, 8>();
      __builtin_amdgcn_sched_barrier(0);  // the staging stores (copies) wait for their loads here
      if constexpr (DMA) {
        wait_vmcnt0();                    // this wave's copies have landed
      } else {
        io.store_k(k_buf(P), tid);
        io.store_v(v_buf(P ^ 1), tid);
      }
      __syncthreads();
    };
    for (int s = 0; s < steps; s += 2) {
      step(std::integral_constant<int, 0>{}, s, s_a, s_b);
      if (s + 1 >= steps) break;
      step(std::integral_constant<int, 1>{}, s + 1, s_b, s_a);
    }
  } else {
    if (steps > 0) {
      io.load_k(rk, tile_off(0), tid);
      io.load_v(rv, tile_off(0), tid);
      io.store_k(k_buf(0), tid);
      io.store_v(v_buf(0), tid);
      __syncthreads();
    }
    for (int s = 0; s < steps; ++s) {
      const int P = s & 1;
      const bool has_next = s + 1 < steps;
      cover(s);
      if (has_next) {
        io.load_k(rk, tile_off(s + 1), tid);
        io.load_v(rv, tile_off(s + 1), tid);
      }
      if ((win.flags(s) >> (8 + ww.slot)) & 1) {
        f32x16_t sc[MB];
        f8_scores(k_buf(P) + k_lane, qf, sc);
        mask_block(s, sc);
        const float hi = bf_row_max<MB>(sc);
        const i32x8_t pk = softmax(s, sc, hi);
        f8_pv(v_buf(P) + v_lane, pk, oacc);
      }
      if (has_next) {
        io.store_k(k_buf(P ^ 1), tid);
        io.store_v(v_buf(P ^ 1), tid);
      }
      __syncthreads();
    }
  }

  if (!ww.active) return;
  const TileValid tq = tile_valid(L, ww.qt);
  const int qrow = 32 * rg + l32;
  const float lt = MSUM ? l_run : halves_sum(l_run);
  const bool real = row_is_real(L, tq, qrow);
  const float inv = (real && lt > 0.0f) ? wmax / (kP8Scale * lt) : 0.0f;
  const long long orow = ww.head_row0 + (long long)ww.qt * TILE + qrow;
  long long obase = orow;
  bool store = true;
  if constexpr (NAT) {
    const int n = natural_index(L, ww.qt, qrow);
    const int b = ww.bh / L.heads, h = ww.bh - b * L.heads;
    store = n >= 0;
    obase = ((long long)b * L.n_tokens + max(n, 0)) * L.heads + h;
  }
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (!store) break;
      const int c0 = 32 * cb + 8 * g + 4 * half;
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + obase * D + c0) =
          make_uint2(pack2(oacc[cb][4 * g] * inv, oacc[cb][4 * g + 1] * inv),
                     pack2(oacc[cb][4 * g + 2] * inv, oacc[cb][4 * g + 3] * inv));
    }
  if (a.lse && half == 0) {
    a.lse[orow] = (real && lt > 0.0f) ? (m_run + __log2f(lt)) * 0.69314718055994531f : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
template <int TILE, int KVH, int D, int QPW, bool F32IN, int NBUF = 2, bool VOP = false>
hipError_t launch_bf16(const DevLayout& L, const AttnArgs& a, hipStream_t s) {
  const int n_work = L.B * L.heads * ((L.n_tiles + QPW - 1) / QPW);
  const size_t dyn = QPW > 1 ? (size_t)L.n_tiles * sizeof(int) : 0;
  if (a.natural_io)
    hipLaunchKernelGGL((attn_bf16_kernel<TILE, KVH, D, QPW, F32IN, NBUF, true, VOP>), dim3(n_work),
                       dim3(64 * QPW * (TILE / 32)), dyn, s, L, a, n_work);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<TILE, KVH, D, QPW, F32IN, NBUF, false, VOP>), dim3(n_work),
                       dim3(64 * QPW * (TILE / 32)), dyn, s, L, a, n_work);
  return hipGetLastError();
}

template <int QPW, bool VOP = false>
hipError_t launch_fp8(const DevLayout& L, const AttnArgs& a, hipStream_t s) {
  const int n_work = L.B * L.heads * ((L.n_tiles + QPW - 1) / QPW);
  const size_t dyn = QPW > 1 ? (size_t)L.n_tiles * sizeof(int) : 0;
  if (a.natural_io)
    hipLaunchKernelGGL((attn_fp8_kernel<QPW, VOP, true>), dim3(n_work), dim3(128 * QPW), dyn, s, L, a, n_work);
  else
    hipLaunchKernelGGL((attn_fp8_kernel<QPW, VOP, false>), dim3(n_work), dim3(128 * QPW), dyn, s, L, a, n_work);
  return hipGetLastError();
}

template <int TILE, int D, bool F32IN>
hipError_t launch_bf16_shape(const DevLayout& L, const AttnArgs& a, bool grouped, hipStream_t s) {
  if constexpr (TILE == 64) {
    return grouped ? launch_bf16<64, 64, D, 4, F32IN, 4>(L, a, s)
                   : launch_bf16<64, 32, D, 1, F32IN>(L, a, s);
  } else {
    return grouped ? launch_bf16<32, 32, D, 4, F32IN>(L, a, s) : launch_bf16<32, 32, D, 1, F32IN>(L, a, s);
  }
}

}  // namespace

hipError_t launch_attn(const DevLayout& L, int dtype, const AttnArgs& a, hipStream_t s) {
  // Shared (head-invariant) or dense lists: neighbouring query tiles share key
  // tiles, so four query tiles walk their union together. Routed lists, and
  // shared tables the caller marks as walked per tile (list_mode 2): one
  // query tile per workgroup.
  const bool grouped = (a.kv_idx == nullptr || a.list_mode == 0) && L.n_tiles <= 4096;
  if (dtype == 4) {   // bf16 with V in the P.V operand layout
    if (L.C != 64 || (L.d != 128 && L.d != 64)) return hipErrorInvalidValue;
    if (L.d == 128)
      return grouped ? launch_bf16<64, 64, 128, 4, false, 4, true>(L, a, s)
                     : launch_bf16<64, 32, 128, 1, false, 2, true>(L, a, s);
    return grouped ? launch_bf16<64, 64, 64, 4, false, 4, true>(L, a, s)
                   : launch_bf16<64, 32, 64, 1, false, 2, true>(L, a, s);
  }
  if (dtype == 3) {   // e4m3 with V codes in the P.V operand layout
    if (L.C != 64 || L.d != 128) return hipErrorInvalidValue;
    return grouped ? launch_fp8<4, true>(L, a, s) : launch_fp8<1, true>(L, a, s);
  }
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
