// Backward pass of the block-sparse attention on gfx950 MFMA: dQ, dK and dV
// over the same key-tile lists as the forward. The pages train through this
// attention (VSA, Research Type and Experiment Setup rows: a trainable
// sparse attention used in DiT pretraining and fine-tuning; FPSAttention,
// Approach: training-aware FP8 and tile sparsity). The gradients are the
// chain rule of the forward's definition; with the forward's natural-log
// lse and D_i = dO_i . O_i:
//   P_ij  = exp(sigma q_i.k_j - lse_i)            (j in A(i))
//   dV_j  = sum_i P_ij dO_i
//   dS_ij = P_ij (dO_i.v_j - D_i)
//   dQ_i  = sigma sum_j dS_ij k_j,   dK_j = sigma sum_i dS_ij q_i
//
// Three kernels, in stream order:
//   rowstat: lse_i * log2(e) (+inf where the row has no weight) and D_i;
//   dq:  one workgroup per query tile, walking the tile's forward list; a
//        wave owns 32 query rows and computes the transposed products
//          S^T = K . Q^T,  dP^T = V . dO^T,  dQ^T += K^T . dS^T
//        so every lane holds one query row: its lse and D stay in registers;
//   dkv: one workgroup per key tile, walking the transposed list (the query
//        tiles whose lists hold it); a wave owns 16 key rows and computes
//          S = Q . K^T,  dP = dO . V^T,  dV^T += dO^T . P,  dK^T += Q^T . dS
//        so every lane holds one key column and its K, V operands stay in
//        registers for the whole walk.
// The walked tensors (K and V for dq, Q and dO for dkv) pass through LDS in
// 32-token blocks of padded row-major rows, one barrier per block: K and V
// through registers one block ahead, Q and dO (bf16) copied straight into a
// four-slot ring two blocks ahead. The
// operands that contract over tokens (K^T, dO^T, Q^T) are read from those
// same rows with ds_read_b64_tr_b16, whose transposition hands each lane
// four consecutive token rows of one channel. The probabilities and dS
// leave the score accumulators as B operands without moving between lanes:
// the token contraction runs in the accumulator's row order, and the
// transposed reads gather the tokens in that same order.
#include <float.h>

#include <type_traits>

#include <mutex>

#include "vsa_internal.h"

namespace vsa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr float kLog2e = 1.4426950408889634f;

// two floats -> two bf16 (round to nearest even) in one dword, lo first
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

// Buffer-resource loads of one (b, head) slice: 32-bit offsets, reads past
// the slice return zero.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, long long bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)(bytes < 0x7FFFFFFFll ? bytes : 0x7FFFFFFFll),
                                           0x00020000);
}
__device__ __forceinline__ uint4 bload(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
// 8 consecutive elements at byte offset voff + soff as 8 bf16 (f32 input: rounded)
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

__device__ __forceinline__ f32x16_t mfma(uint4 a, uint4 b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Row statistics. LPR = D/8 lanes per row, 8 elements each.
template <int D, bool F32IN>
__global__ __launch_bounds__(256) void rowstat_kernel(const void* out, const void* dout,
                                                      const float* lse, float2* st, long long rows) {
  constexpr int LPR = D / 8;
  constexpr int RPB = 256 / LPR;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / LPR;
  const int part = threadIdx.x % LPR;
  float acc = 0.0f;
  if (row < rows) {
    const long long e0 = row * D + part * 8;
    if constexpr (F32IN) {
      const float4* o = reinterpret_cast<const float4*>(static_cast<const float*>(out) + e0);
      const float4* g = reinterpret_cast<const float4*>(static_cast<const float*>(dout) + e0);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float4 x = o[i], y = g[i];
        acc += x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
      }
    } else {
      const uint4 x = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(out) + e0);
      const uint4 y = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(dout) + e0);
      const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ys[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) acc += bf_lo(xs[i]) * bf_lo(ys[i]) + bf_hi(xs[i]) * bf_hi(ys[i]);
    }
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && part == 0) {
    const float l = lse[row];
    const bool live = l > -INFINITY;      // -inf: pad row or empty key set
    st[row] = make_float2(live ? l * kLog2e : INFINITY, live ? acc : 0.0f);
  }
}

// ---------------------------------------------------------------------------
// Transposed lists: one workgroup per (list head, key tile j) tests every
// query tile's ascending list for j by binary search and compacts the hits
// in ascending order (ballot prefix counts), so the result is deterministic.
__global__ __launch_bounds__(256) void transpose_lists_kernel(int n_tiles, const int32_t* kv_idx,
                                                              const int32_t* kv_cnt, int max_kv,
                                                              int32_t* q_idx, int32_t* q_cnt) {
  __shared__ int wcnt[4];
  const int j = blockIdx.x;
  const long long lh = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int32_t* idx = kv_idx + lh * n_tiles * (long long)max_kv;
  const int32_t* cnt = kv_cnt + lh * n_tiles;
  int32_t* dst = q_idx + (lh * n_tiles + j) * (long long)n_tiles;
  int total = 0;
  for (int i0 = 0; i0 < n_tiles; i0 += 256) {
    const int i = i0 + tid;
    bool hit = false;
    if (i < n_tiles) {
      const int32_t* row = idx + (long long)i * max_kv;
      const int c = min(max(cnt[i], 0), max_kv);
      int lo = 0, hi = c;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (row[mid] < j) lo = mid + 1;
        else hi = mid;
      }
      hit = lo < c && row[lo] == j;
    }
    const unsigned long long m = __ballot(hit);
    if (lane == 0) wcnt[wave] = __popcll(m);
    __syncthreads();
    int off = total;
    for (int w = 0; w < wave; ++w) off += wcnt[w];
    if (hit) dst[off + __popcll(m & ((1ull << lane) - 1ull))] = i;
    total += wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
    __syncthreads();
  }
  if (tid == 0) q_cnt[lh * n_tiles + j] = total;
}

// Row padding of the LDS blocks, in 16-byte chunks. With 32 bytes the four
// consecutive rows that one 16-lane group of a transposed read
// (ds_read_b64_tr_b16, 32 bytes per row) touches start 8 banks apart and do
// not overlap; with 16 bytes they overlapped by half. Measured on the 768p
// Skiparse backward: 118.4 -> 108.5-112.5 ms (dK/dV gains most; 48 bytes for
// dQ is no better, 64 bytes costs 9 ms; dK/dV cannot take more than 32 and
// keep two workgroups per CU).
constexpr int kPadDq = 2, kPadDkv = 2;

// ---------------------------------------------------------------------------
// Register staging of one 32-token block (32 rows x D channels, row-major in
// HBM) and its store into padded LDS rows (PAD chunks of 16 bytes per row).
template <int D, int THREADS, bool F32IN, int PAD>
struct RowBlock {
  static constexpr int ES = F32IN ? 4 : 2;
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int RS = CPR + PAD;              // padded row stride, uint4
  static constexpr int RSE = RS * 8;                // padded row stride, bf16 elements
  static constexpr int CHUNKS = 32 * CPR;
  static constexpr int PER_T = (CHUNKS + THREADS - 1) / THREADS;
  static constexpr int LDS = 32 * RS;               // uint4 per buffer
  static_assert(CHUNKS % THREADS == 0 || THREADS % CHUNKS == 0, "even split of the chunks");
  uint4 reg[PER_T];

  // block_off: byte offset of the block's first row inside the (b, head) slice
  __device__ __forceinline__ void load(rsrc_t r, uint32_t block_off, int tid) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i)
      if (CHUNKS >= THREADS || tid < CHUNKS)
        reg[i] = bload8<F32IN>(r, (tid + i * THREADS) * 8 * ES, block_off);
  }
  __device__ __forceinline__ void store(uint4* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int c = tid + i * THREADS;
      if (CHUNKS >= THREADS || c < CHUNKS) lds[(c / CPR) * RS + c % CPR] = reg[i];
    }
  }
};

// Per-lane element offset for the transposed reads below: in each 16-lane
// group, source lane i reads row 4*half + i/4 at channels 16*(group%2) +
// 4*(i%4) .. +3, so that the transposition hands lane i rows 4*half + 0..3
// of channel 16*(group%2) + i.
template <int RSE>
__device__ __forceinline__ int tr_lane_offset(int lane) {
  const int g = lane >> 4, i = lane & 15;
  return (4 * (g >> 1) + (i >> 2)) * RSE + 16 * (g & 1) + 4 * (i & 3);
}

__device__ __forceinline__ uint2 lds_tr(const uint16_t* p) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p));
}

// A operand X^T (32 channels c0.., 16 tokens of chunk kc) from row-major X
// rows in LDS, tokens in the score accumulator's row order: operand slot s
// of half-wave h is token 16*kc + 8*(s/4) + 4*h + s%4.
// base = LDS rows + tr_lane_offset(lane).
template <int RSE>
__device__ __forceinline__ uint4 frag_t(const uint16_t* base, int c0, int kc) {
  const uint2 lo = lds_tr(base + (16 * kc) * RSE + c0);
  const uint2 hi = lds_tr(base + (16 * kc + 8) * RSE + c0);
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// Bit r set iff token 8*(r/4) + 4*half + r%4 of the block (tokens tok0 ..
// tok0+31 of tile `tile`) is real.
__device__ __forceinline__ uint32_t block_real_bits(const DevLayout& L, int tile, int tok0, int lane,
                                                    int half) {
  const TileValid tv = tile_valid(L, tile);
  if (tv.full) return 0xFFFFu;
  const unsigned long long vm = __ballot(lane < 32 && row_is_real(L, tv, tok0 + lane));
  uint32_t m = 0;
#pragma unroll
  for (int g = 0; g < 4; ++g) m |= (uint32_t)((vm >> (8 * g + 4 * half)) & 0xFull) << (4 * g);
  return m;
}

// Write 32 rows x D of a transposed accumulator (lane holds row `row` and
// channels 32*mt + 8*g + 4*half + 0..3) scaled by f, as bf16 or f32; rows
// with real == false are written as zeros (whatever the accumulator holds).
template <int D, bool F32IN>
__device__ __forceinline__ void store_rows_t(void* dst, long long row, int half,
                                             const f32x16_t (&acc)[D / 32], float f, bool real) {
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c0 = 32 * mt + 8 * g + 4 * half;
      const float x0 = real ? acc[mt][4 * g] * f : 0.0f, x1 = real ? acc[mt][4 * g + 1] * f : 0.0f;
      const float x2 = real ? acc[mt][4 * g + 2] * f : 0.0f, x3 = real ? acc[mt][4 * g + 3] * f : 0.0f;
      if constexpr (F32IN) {
        *reinterpret_cast<float4*>(static_cast<float*>(dst) + row * D + c0) = make_float4(x0, x1, x2, x3);
      } else {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(dst) + row * D + c0) =
            make_uint2(pack2(x0, x1), pack2(x2, x3));
      }
    }
}

// ---------------------------------------------------------------------------
// Union of the QPW query-tile slots' lists (slot i's list: `list`, `cnt` of
// the waves of slot i; null list = every tile) written to sched[] in
// ascending order, each entry tile | (mask of slots listing it) << 24;
// returns its length and sets `shared` when every entry is listed by every
// active slot. `marks` (one byte per tile) and `scan` (one int per thread)
// are scratch the caller may alias onto LDS it only uses afterwards.
template <int QPW, int WPQ>
__device__ int union_lists(int n_tiles, const int32_t* list, int cnt, int slot, bool active_slot,
                           int active_mask, uint32_t* marks, int* scan, int* sched, int tid,
                           int lane, bool& shared) {
  constexpr int THREADS = 64 * QPW * WPQ;
  const int words = (n_tiles + 3) >> 2;
  for (int t = tid; t < words; t += THREADS) marks[t] = 0;
  __syncthreads();
  if (active_slot && (tid >> 6) % WPQ == 0) {
    for (int i = lane; i < cnt; i += 64) {
      const int t = list ? min(max(list[i], 0), n_tiles - 1) : i;
      atomicOr(&marks[t >> 2], 1u << (8 * (t & 3) + slot));
    }
  }
  __syncthreads();
  auto mark = [&](int t) -> int { return (marks[t >> 2] >> (8 * (t & 3))) & 0xFF; };
  const int per = (n_tiles + THREADS - 1) / THREADS;
  const int lo = min(tid * per, n_tiles), hi = min(lo + per, n_tiles);
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
  bool same = true;
  for (int t = lo; t < hi; ++t) {
    const int m = mark(t);
    if (m) sched[pos++] = t | (m << 24);
    same = same && (m == 0 || m == active_mask);
  }
  shared = __syncthreads_and(same) != 0;
  return len;
}

// dQ: QPW consecutive query tiles per workgroup (C/32 waves each). With
// QPW = 4 (shared and dense lists) the tiles walk the ascending union of
// their lists once, each K/V block staged in LDS once for all of them; a
// wave whose tile's list lacks a block skips its math. QPW = 1 walks one
// tile's own list (per-head routed lists, where neighbouring tiles share
// few key tiles). K and V go through registers into double-buffered padded
// LDS rows, one barrier per 32-key block.
template <int C, int D, bool F32IN, int QPW>
__global__ __launch_bounds__(2 * C * QPW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dq_kernel(DevLayout L, BwdArgs a, int n_work) {
  constexpr int WPQ = C / 32, THREADS = 64 * WPQ * QPW, SUB = C / 32;
  constexpr int ES = F32IN ? 4 : 2;
  using RB = RowBlock<D, THREADS, F32IN, kPadDq>;
  __shared__ uint4 k_lds[2][RB::LDS];
  __shared__ uint4 v_lds[2][RB::LDS];
  __shared__ int sched[QPW > 1 ? 4096 : 1];
  static_assert(QPW == 1 || THREADS * 4 <= RB::LDS * 16, "scan scratch fits one K buffer");
  static_assert(QPW == 1 || 4096 <= RB::LDS * 16, "marks of 4096 tiles fit one V buffer");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  const int slot = wave / WPQ, rg = wave % WPQ;
  const int item = a.kv_idx && a.list_mode == 1 ? xcd_chunked(blockIdx.x, n_work, 64)
                                                 : xcd_remap(blockIdx.x, n_work);
  const int wg_per_bh = (L.n_tiles + QPW - 1) / QPW;
  const int bh = item / wg_per_bh;
  const int qt0 = (item - bh * wg_per_bh) * QPW;
  const int qt = qt0 + slot;
  const bool active = qt < L.n_tiles;
  const long long row0 = (long long)bh * L.n_padded;
  const long long slice = (long long)L.n_padded * D * ES;
  const rsrc_t rq = make_rsrc(static_cast<const char*>(a.q) + row0 * D * ES, slice);
  const rsrc_t rk = make_rsrc(static_cast<const char*>(a.k) + row0 * D * ES, slice);
  const rsrc_t rv = make_rsrc(static_cast<const char*>(a.v) + row0 * D * ES, slice);
  const rsrc_t rg_ = make_rsrc(static_cast<const char*>(a.dout) + row0 * D * ES, slice);

  const int32_t* list = nullptr;
  int cnt = L.n_tiles;
  if (a.kv_idx && active) {
    const long long r = (a.list_mode ? (long long)bh * L.n_tiles : 0ll) + qt;
    list = a.kv_idx + r * a.max_kv;
    cnt = min(max(a.kv_cnt[r], 0), a.max_kv);
  }
  int len = active ? cnt : 0;
  bool shared = true;
  if constexpr (QPW > 1) {
    const int active_mask = (1 << min(max(L.n_tiles - qt0, 0), QPW)) - 1;
    len = union_lists<QPW, WPQ>(L.n_tiles, a.kv_idx ? list : nullptr, cnt, slot, active,
                                active_mask, reinterpret_cast<uint32_t*>(v_lds[1]),
                                reinterpret_cast<int*>(k_lds[1]), sched, tid, lane, shared);
  }

  // B operands Q^T and dO^T: row qrow, channels 16*ks + 8*half .. +7
  const int qrow = 32 * rg + l32;
  const uint32_t qoff = (uint32_t)((min(qt, L.n_tiles - 1) * C + qrow) * D * ES);
  uint4 qf[D / 16], gf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    qf[ks] = bload8<F32IN>(rq, qoff + (16 * ks + 8 * half) * ES, 0);
    gf[ks] = bload8<F32IN>(rg_, qoff + (16 * ks + 8 * half) * ES, 0);
  }
  const float2 st = a.rowstat[row0 + min(qt, L.n_tiles - 1) * C + qrow];
  const float nl = -st.x, dd = st.y;
  // dP^T accumulators start at -D, so they end as dP - D
  f32x16_t neg_dd;
#pragma unroll
  for (int r = 0; r < 16; ++r) neg_dd[r] = -dd;
  const float sl2 = a.scale_log2;

  f32x16_t acc[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) acc[mt] = f32x16_t{};

  const int nblk = len * SUB;
  auto entry = [&](int b) -> int {
    const int e = b / SUB;
    if constexpr (QPW > 1) return sched[e];
    else return (list ? min(max(list[e], 0), L.n_tiles - 1) : e) | (1 << 24);
  };
  auto block_off = [&](int b) -> uint32_t {
    return (uint32_t)(((entry(b) & 0xFFFFFF) * C + 32 * (b % SUB)) * D * ES);
  };

  RB kio, vio;
  if (nblk > 0) {
    const uint32_t off = block_off(0);
    kio.load(rk, off, tid);
    vio.load(rv, off, tid);
    kio.store(k_lds[0], tid);
    vio.store(v_lds[0], tid);
  }
  __syncthreads();
  const int tro = tr_lane_offset<RB::RSE>(lane);
  for (int b = 0; b < nblk; ++b) {
    const int buf = b & 1;
    if (b + 1 < nblk) {
      const uint32_t off = block_off(b + 1);
      kio.load(rk, off, tid);
      vio.load(rv, off, tid);
    }
    const int ent = entry(b);
    if (QPW == 1 || (active && ((ent >> (24 + slot)) & 1))) {
      const uint32_t kbits = block_real_bits(L, ent & 0xFFFFFF, 32 * (b % SUB), lane, half);
      const uint4* kb = k_lds[buf] + l32 * RB::RS + half;
      const uint4* vb = v_lds[buf] + l32 * RB::RS + half;
      f32x16_t s = {}, dp = neg_dd;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        s = mfma(kb[2 * ks], qf[ks], s);
        dp = mfma(vb[2 * ks], gf[ks], dp);
      }
      // dS^T operands; pad keys (only in tiles with pads) get p = 0
      uint4 dsp[2];
      auto ds_pack = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          float x[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int r = 8 * c + i;
            float p = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, nl));
            if constexpr (decltype(masked)::value) p = ((kbits >> r) & 1u) ? p : 0.0f;
            x[i] = p * dp[r];
          }
          dsp[c] = make_uint4(pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7]));
        }
      };
      if (kbits == 0xFFFFu) ds_pack(std::false_type{});    // full tiles: uniform across the wave
      else ds_pack(std::true_type{});
      const uint16_t* kt = reinterpret_cast<const uint16_t*>(k_lds[buf]) + tro;
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
        for (int c = 0; c < 2; ++c) acc[mt] = mfma(frag_t<RB::RSE>(kt, 32 * mt, c), dsp[c], acc[mt]);
    }
    if (b + 1 < nblk) {
      kio.store(k_lds[buf ^ 1], tid);
      vio.store(v_lds[buf ^ 1], tid);
    }
    __syncthreads();
  }
  if (active) {
    const bool real = row_is_real(L, tile_valid(L, qt), qrow);
    store_rows_t<D, F32IN>(a.dq, row0 + qt * C + qrow, half, acc, a.scale, real);
  }
}

// ---------------------------------------------------------------------------
// Direct copies from HBM into LDS (buffer_load ... lds): each 64-lane copy
// writes 1 KB of LDS, lane i at byte 16*i from the wave-uniform base.
typedef __attribute__((address_space(3))) void lds_void_t;
__device__ __forceinline__ void dma16(rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, (int)voff, (int)soff, 0, 0);
}
// s_waitcnt with vmcnt <= N (expcnt and lgkmcnt at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Copies of one 32-row block into padded LDS rows (RowBlock's layout) by the
// WAVES waves of a workgroup: copy j of a wave covers LDS chunks
// 64*(wave + WAVES*j) + lane, i.e. row p / RS, chunk p % RS (pad chunks
// take a copy of the row's last chunk; they are never read).
template <int D, int WAVES, int PAD>
struct BlockCopy {
  static constexpr int CPR = D / 8, RS = CPR + PAD, CHUNKS = 32 * RS;
  static constexpr int NI = (CHUNKS + 63) / 64;           // copies per block
  static constexpr int NIW0 = (NI + WAVES - 1) / WAVES;   // copies of wave 0 (the most)
  static constexpr int NIW1 = NI / WAVES;                 // of the last wave
  uint32_t voff[NIW0];
  bool valid[NIW0];
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int j = 0; j < NIW0; ++j) {
      const int p = 64 * (wave + WAVES * j) + lane;
      valid[j] = (wave + WAVES * j) < NI && p < CHUNKS;
      voff[j] = (uint32_t)((p / RS) * D * 2 + min(p % RS, CPR - 1) * 16);
    }
  }
  // the 32 rows starting at byte offset soff (wave-uniform) of r, into lds
  __device__ __forceinline__ void issue(rsrc_t r, uint4* lds, uint32_t soff, int wave) const {
#pragma unroll
    for (int j = 0; j < NIW0; ++j)
      if ((j < NIW1 || wave == 0) && valid[j])
        dma16(r, reinterpret_cast<char*>(lds) + 1024 * (wave + WAVES * j), voff[j], soff);
  }
};

// dK and dV: one workgroup per (b, head, key tile), 16 key rows per wave
// for the scores (v_mfma_f32_16x16x32_bf16, C/16 waves per tile). A wave
// holds its K and V operands and the accumulators of its share of dK/dV in
// about 210 registers, so two waves share each SIMD and cover each other's
// latencies (owning 32 keys with 32x32 products needs more than 256
// registers, one wave per SIMD). Per 32-query block a wave computes
//   S = Q . K^T, dP = dO . V^T          (its 16 keys; 2 query tiles x 4
//                                        channel chunks each)
//   dV^T += dO^T . P, dK^T += Q^T . dS  (its D/WAVES channels x all C keys,
//                                        the 32 queries as one contraction
//                                        chunk)
// 16x16x32 operand layouts: A lane l holds row l%16, k = 8*(l/16) .. +7; B
// lane l holds column l%16, the same k; C lane l holds rows 4*(l/16) + i,
// column l%16. The 32 queries of P and dS (C rows 4g + i of the two query
// tiles, g = l/16) are the contraction slots: slot s of lane group g is query
// 4g + s (s < 4) or 16 + 4g + s - 4, and the transposed LDS reads of dO and
// Q gather the same queries. For the dV/dK products the waves split the
// channels instead of the keys: each wave publishes its packed P and dS (the
// B operands of its 16 keys, 1 KB each) in LDS, and wave w accumulates
// channels D/WAVES*w .. for all C keys from every wave's operands, so each
// wave reads only its own channels of dO^T and Q^T (the half-rate transposed
// reads) instead of all of them. Q and dO blocks are copied into a
// three-slot LDS ring one block ahead (bf16) or staged through registers
// (fp32 inputs); the P/dS exchange has three slots as well.
template <int RSE>
__device__ __forceinline__ int tr16_lane_offset(int lane) {
  const int g = lane >> 4, i = lane & 15;
  return (4 * g + (i >> 2)) * RSE + 4 * (i & 3);
}
__device__ __forceinline__ f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <int C, int D, bool F32IN>
__global__ __launch_bounds__(4 * C) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dkv16_kernel(DevLayout L, BwdArgs a, int n_work) {
  constexpr int WAVES = C / 16, THREADS = 64 * WAVES, SUB = C / 32, NBUF = 3;
  constexpr int NCT = D / WAVES / 16, NKT = WAVES;    // channel and key tiles of a wave's dK/dV
  constexpr int ES = F32IN ? 4 : 2;
  constexpr bool DMA = !F32IN;
  using RB = RowBlock<D, THREADS, F32IN, kPadDkv>;
  using BC = BlockCopy<D, WAVES, kPadDkv>;
  constexpr int RSE = RB::RSE;
  __shared__ uint4 q_s0[RB::LDS], q_s1[RB::LDS], q_s2[RB::LDS];
  __shared__ uint4 g_s0[RB::LDS], g_s1[RB::LDS], g_s2[RB::LDS];
  __shared__ float4 st_s0[16], st_s1[16], st_s2[16];   // 32 rows of {lse2, D}
  __shared__ uint4 xp0[THREADS], xp1[THREADS], xp2[THREADS];   // P / dS exchange, slot = block % 3
  __shared__ uint4 xd0[THREADS], xd1[THREADS], xd2[THREADS];
  auto qbuf = [&](int i) -> uint4* { return i == 0 ? q_s0 : i == 1 ? q_s1 : q_s2; };
  auto gbuf = [&](int i) -> uint4* { return i == 0 ? g_s0 : i == 1 ? g_s1 : g_s2; };
  auto sbuf = [&](int i) -> float4* { return i == 0 ? st_s0 : i == 1 ? st_s1 : st_s2; };
  auto xpbuf = [&](int i) -> uint4* { return i == 0 ? xp0 : i == 1 ? xp1 : xp2; };
  auto xdbuf = [&](int i) -> uint4* { return i == 0 ? xd0 : i == 1 ? xd1 : xd2; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int item = a.q_idx && a.list_mode == 1 ? xcd_chunked(blockIdx.x, n_work, 64)
                                                : xcd_remap(blockIdx.x, n_work);
  const int bh = item / L.n_tiles, kt = item - bh * L.n_tiles;
  const long long row0 = (long long)bh * L.n_padded;
  const long long slice = (long long)L.n_padded * D * ES;
  const rsrc_t rq = make_rsrc(static_cast<const char*>(a.q) + row0 * D * ES, slice);
  const rsrc_t rk = make_rsrc(static_cast<const char*>(a.k) + row0 * D * ES, slice);
  const rsrc_t rv = make_rsrc(static_cast<const char*>(a.v) + row0 * D * ES, slice);
  const rsrc_t rg = make_rsrc(static_cast<const char*>(a.dout) + row0 * D * ES, slice);
  const rsrc_t rs = make_rsrc(a.rowstat + row0, (long long)L.n_padded * 8);
  const float2* rst = a.rowstat + row0;

  const int32_t* list = nullptr;
  int cnt = L.n_tiles;
  if (a.q_idx) {
    const long long r = (a.list_mode ? (long long)bh * L.n_tiles : 0ll) + kt;
    list = a.q_idx + r * L.n_tiles;
    cnt = min(max(a.q_cnt[r], 0), L.n_tiles);
  }

  // B operands K^T and V^T: key krow, channels 32*kc + 8*g .. +7
  const int krow = 16 * wave + l16;
  const uint32_t koff = (uint32_t)((kt * C + krow) * D * ES);
  uint4 kf[D / 32], vf[D / 32];
#pragma unroll
  for (int kc = 0; kc < D / 32; ++kc) {
    kf[kc] = bload8<F32IN>(rk, koff + (32 * kc + 8 * g) * ES, 0);
    vf[kc] = bload8<F32IN>(rv, koff + (32 * kc + 8 * g) * ES, 0);
  }
  const float sl2 = a.scale_log2;
  // dK^T / dV^T of channel tile ct (channels D/WAVES*wave + 16 ct ..) and key tile j (keys 16 j ..)
  f32x4_t dk[NCT][NKT], dv[NCT][NKT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int j = 0; j < NKT; ++j) dk[ct][j] = dv[ct][j] = f32x4_t{};

  const int nblk = cnt * SUB;
  // list entries come from a 64-entry register window (lane i holds entry
  // base + i), refilled once per 64 entries: no per-block memory load whose
  // wait would also wait for the copies in flight
  int lwin = 0, lbase = -64;
  auto first_row = [&](int b) -> int {
    b = min(b, nblk - 1);
    const int e = b / SUB;
    if (e - lbase >= 64) {
      lbase = e & ~63;
      lwin = list ? list[min(lbase + lane, cnt - 1)] : lbase + lane;
    }
    const int t = min(max(__builtin_amdgcn_readlane(lwin, e - lbase), 0), L.n_tiles - 1);
    return __builtin_amdgcn_readfirstlane(t * C + 32 * (b % SUB));
  };
  BC cp;
  if constexpr (DMA) cp.init(wave, lane);
  RB qio, gio;
  float2 streg = make_float2(0.0f, 0.0f);
  auto copy_blk = [&](int r, uint4* qd, uint4* gd, float4* sd) __attribute__((always_inline)) {
    if constexpr (DMA) {
      const uint32_t soff = (uint32_t)(r * D * ES);
      cp.issue(rq, qd, soff, wave);
      cp.issue(rg, gd, soff, wave);
      if (wave == 0 && lane < 16) dma16(rs, sd, lane * 16, (uint32_t)(r * 8));
    } else {
      qio.load(rq, (uint32_t)(r * D * ES), tid);
      gio.load(rg, (uint32_t)(r * D * ES), tid);
      if (tid < 32) streg = rst[r + tid];
    }
  };
  auto store_regs = [&](uint4* qd, uint4* gd, float4* sd) __attribute__((always_inline)) {
    if constexpr (!DMA) {
      qio.store(qd, tid);
      gio.store(gd, tid);
      if (tid < 32) reinterpret_cast<float2*>(sd)[tid] = streg;
    }
  };
  // every copy this wave has issued has landed in LDS
  auto wait_copies = [&]() __attribute__((always_inline)) {
    if constexpr (DMA) wait_vmcnt<0>();
  };
  const int tro = tr16_lane_offset<RSE>(lane);

  // dV^T += dO^T . P and dK^T += Q^T . dS for this wave's channel tiles and
  // every wave's keys (xp / xd: the published B operands of one block)
  const int ch0 = (D / WAVES) * wave;
  auto accumulate = [&](const uint4* qs, const uint4* gs, const uint4* xp, const uint4* xd)
      __attribute__((always_inline)) {
    const uint16_t* gt = reinterpret_cast<const uint16_t*>(gs) + tro + ch0;
    const uint16_t* qt_ = reinterpret_cast<const uint16_t*>(qs) + tro + ch0;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const uint2 glo = lds_tr(gt + 16 * ct), ghi = lds_tr(gt + 16 * RSE + 16 * ct);
      const uint2 qlo = lds_tr(qt_ + 16 * ct), qhi = lds_tr(qt_ + 16 * RSE + 16 * ct);
      const uint4 ga = make_uint4(glo.x, glo.y, ghi.x, ghi.y), qa = make_uint4(qlo.x, qlo.y, qhi.x, qhi.y);
#pragma unroll
      for (int j = 0; j < NKT; ++j) {
        dv[ct][j] = mfma16(ga, xp[64 * j + lane], dv[ct][j]);
        dk[ct][j] = mfma16(qa, xd[64 * j + lane], dk[ct][j]);
      }
    }
  };
  // block s's scores and packed P, dS (published in exchange slot s % 3);
  // block s-1's dV / dK products from its Q / dO slot and exchange slot (not
  // refilled before the next barrier)
  auto step = [&](const uint4* qs, const uint4* gs, const float4* st, const uint4* qp,
                  const uint4* gp, const uint4* xpr, const uint4* xdr, uint4* xpw, uint4* xdw)
      __attribute__((always_inline)) {
    // S and dP: two 16-query tiles
    f32x4_t sc[2], dp[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const uint4* qb = qs + (16 * mt + l16) * RB::RS + g;
      const uint4* gb = gs + (16 * mt + l16) * RB::RS + g;
      sc[mt] = f32x4_t{};
      dp[mt] = f32x4_t{};
#pragma unroll
      for (int kc = 0; kc < D / 32; ++kc) {
        sc[mt] = mfma16(qb[4 * kc], kf[kc], sc[mt]);
        dp[mt] = mfma16(gb[4 * kc], vf[kc], dp[mt]);
      }
    }
    // P and dS for queries 16*mt + 4g + i, packed as the 32-query B operands
    float p[8], x[8];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const float4 s01 = st[8 * mt + 2 * g];         // rows 16mt+4g+0, +1
      const float4 s23 = st[8 * mt + 2 * g + 1];     // rows 16mt+4g+2, +3
      const float l2[4] = {s01.x, s01.z, s23.x, s23.z};
      const float dd[4] = {s01.y, s01.w, s23.y, s23.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[4 * mt + i] = __builtin_amdgcn_exp2f(fmaf(sc[mt][i], sl2, -l2[i]));
        x[4 * mt + i] = p[4 * mt + i] * (dp[mt][i] - dd[i]);
      }
    }
    const uint4 pp = make_uint4(pack2(p[0], p[1]), pack2(p[2], p[3]), pack2(p[4], p[5]), pack2(p[6], p[7]));
    const uint4 dsp = make_uint4(pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7]));
    accumulate(qp, gp, xpr, xdr);
    xpw[tid] = pp;
    xdw[tid] = dsp;
  };

  using C1 = std::integral_constant<int, 1>;
  using C0 = std::integral_constant<int, 0>;
  // "block -1": zero Q / dO slot 2 and exchange slot 2, so step 0 adds nothing.
  // The walk is unrolled by three so that every slot is a compile-time array:
  // reads of one slot then need not wait for the copy in flight into another.
  int nrow = 0;                           // first row of the next block to copy
  if (nblk > 0) {
    for (int i = tid; i < RB::LDS; i += THREADS) {
      q_s2[i] = make_uint4(0u, 0u, 0u, 0u);
      g_s2[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    xp2[tid] = make_uint4(0u, 0u, 0u, 0u);
    xd2[tid] = make_uint4(0u, 0u, 0u, 0u);
    copy_blk(first_row(0), q_s0, g_s0, st_s0);
    store_regs(q_s0, g_s0, st_s0);
    nrow = first_row(1);
    wait_copies();
    __syncthreads();
  }
  wait_vmcnt<0>();                        // K / V operands in registers (also when the list is empty)
  auto body = [&](auto phase, int s) __attribute__((always_inline)) {
    constexpr int cur = decltype(phase)::value, in = (cur + 1) % NBUF, prv = (cur + NBUF - 1) % NBUF;
    const int r2 = first_row(s + 2);      // before the copies: a window refill waits for nothing else
    copy_blk(nrow, qbuf(in), gbuf(in), sbuf(in));
    nrow = r2;
    step(qbuf(cur), gbuf(cur), sbuf(cur), qbuf(prv), gbuf(prv), xpbuf(prv), xdbuf(prv), xpbuf(cur),
         xdbuf(cur));
    store_regs(qbuf(in), gbuf(in), sbuf(in));
    wait_copies();                    // block s+1 has landed
    __syncthreads();
  };
  using C2 = std::integral_constant<int, 2>;
  for (int s = 0; s < nblk; s += 3) {
    body(C0{}, s);
    if (s + 1 >= nblk) break;
    body(C1{}, s + 1);
    if (s + 2 >= nblk) break;
    body(C2{}, s + 2);
  }
  if (nblk > 0)
    accumulate(qbuf((nblk - 1) % NBUF), gbuf((nblk - 1) % NBUF), xpbuf((nblk - 1) % NBUF),
               xdbuf((nblk - 1) % NBUF));
  wait_copies();                      // no copy into LDS outlives the workgroup

  const TileValid tvk = tile_valid(L, kt);
#pragma unroll
  for (int t = 0; t < NCT * NKT; ++t) {
    const int ct = t / NKT, j = t % NKT;
    const bool real = row_is_real(L, tvk, 16 * j + l16);
    const long long orow = row0 + kt * C + 16 * j + l16;
    const int c0 = ch0 + 16 * ct + 4 * g;
    const float f = a.scale;
    const float k0 = real ? dk[ct][j][0] * f : 0.0f, k1 = real ? dk[ct][j][1] * f : 0.0f;
    const float k2 = real ? dk[ct][j][2] * f : 0.0f, k3 = real ? dk[ct][j][3] * f : 0.0f;
    const float v0 = real ? dv[ct][j][0] : 0.0f, v1 = real ? dv[ct][j][1] : 0.0f;
    const float v2 = real ? dv[ct][j][2] : 0.0f, v3 = real ? dv[ct][j][3] : 0.0f;
    if constexpr (F32IN) {
      *reinterpret_cast<float4*>(static_cast<float*>(a.dk) + orow * D + c0) = make_float4(k0, k1, k2, k3);
      *reinterpret_cast<float4*>(static_cast<float*>(a.dv) + orow * D + c0) = make_float4(v0, v1, v2, v3);
    } else {
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.dk) + orow * D + c0) =
          make_uint2(pack2(k0, k1), pack2(k2, k3));
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.dv) + orow * D + c0) =
          make_uint2(pack2(v0, v1), pack2(v2, v3));
    }
  }
}

template <int C, int D, bool F32IN>
hipError_t launch_bwd_shape(const DevLayout& L, const BwdArgs& a, hipStream_t s) {
  const long long rows = (long long)L.B * L.heads * L.n_padded;
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL((rowstat_kernel<D, F32IN>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256),
                     0, s, a.out, a.dout, a.lse, a.rowstat, rows);
  const int n_work = L.B * L.heads * L.n_tiles;
  if (a.list_mode == 1 || L.n_tiles > 4096) {
    hipLaunchKernelGGL((dq_kernel<C, D, F32IN, 1>), dim3(n_work), dim3(2 * C), 0, s, L, a, n_work);
  } else {
    const int n_grp = L.B * L.heads * ((L.n_tiles + 3) / 4);
    hipLaunchKernelGGL((dq_kernel<C, D, F32IN, 4>), dim3(n_grp), dim3(8 * C), 0, s, L, a, n_grp);
  }
  hipLaunchKernelGGL((dkv16_kernel<C, D, F32IN>), dim3(n_work), dim3(4 * C), 0, s, L, a, n_work);
  return hipGetLastError();
}

template <bool F32IN>
hipError_t launch_bwd_dtype(const DevLayout& L, const BwdArgs& a, hipStream_t s) {
  if (L.C == 64) return L.d == 128 ? launch_bwd_shape<64, 128, F32IN>(L, a, s)
                                   : launch_bwd_shape<64, 64, F32IN>(L, a, s);
  return L.d == 128 ? launch_bwd_shape<32, 128, F32IN>(L, a, s) : launch_bwd_shape<32, 64, F32IN>(L, a, s);
}

}  // namespace

hipError_t launch_transpose_lists(const DevLayout& L, const int32_t* kv_idx, const int32_t* kv_cnt,
                                  int max_kv, int list_mode, int32_t* q_idx, int32_t* q_cnt,
                                  hipStream_t s) {
  const int lh = list_mode ? L.B * L.heads : 1;
  hipLaunchKernelGGL(transpose_lists_kernel, dim3(L.n_tiles, lh), dim3(256), 0, s, L.n_tiles, kv_idx,
                     kv_cnt, max_kv, q_idx, q_cnt);
  return hipGetLastError();
}

size_t attn_bwd_workspace_bytes(const DevLayout& L) {
  return (size_t)L.B * L.heads * L.n_padded * sizeof(float2);
}

// Row statistics of the allocation-free backward: a file-scope device array,
// one copy per GPU (at its own address), held until the process ends. Every
// call rewrites the rows it uses before reading them, so nothing needs
// clearing; calls that overlap on one GPU share it and race.
static __device__ __align__(256) unsigned char scratch[kBwdScratchBytes];

hipError_t attn_bwd_scratch(void** ptr) {
  static std::mutex mu;
  static void* per_device[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!per_device[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

hipError_t launch_attn_bwd(const DevLayout& L, int dtype, const BwdArgs& a, hipStream_t s) {
  return dtype == 0 ? launch_bwd_dtype<true>(L, a, s) : launch_bwd_dtype<false>(L, a, s);
}

}  // namespace vsa
