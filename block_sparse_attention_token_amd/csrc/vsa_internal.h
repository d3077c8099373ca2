// Internal declarations shared by the libvsa HIP sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vsa {

// Layout with every derived size precomputed on the host; passed to kernels by value.
struct DevLayout {
  int B, heads, d;
  int T, H, W;
  int kind;                 // 0 = 3D tiles, 1 = Skiparse-2D groups
  int tt, th, tw;           // tile extents
  int sh, sw;               // Skiparse strides
  int C;                    // tokens per tile
  int n_tiles;
  int ntt, nth, ntw;        // 3D tile grid
  int tiles_per_group;      // Skiparse: tiles per residue group
  int group_len;            // Skiparse: real tokens per group
  long long n_tokens;       // T * H * W
  long long n_padded;       // n_tiles * C
};

// Natural token index of row r of tile `tile`, or -1 for a pad row.
__device__ __forceinline__ int natural_index(const DevLayout& L, int tile, int r) {
  if (L.kind == 0) {
    const int per_a = L.nth * L.ntw;
    const int a = tile / per_a;
    const int rem = tile - a * per_a;
    const int b = rem / L.ntw;
    const int c = rem - b * L.ntw;
    const int per_i = L.th * L.tw;
    const int i = r / per_i;
    const int rr = r - i * per_i;
    const int j = rr / L.tw;
    const int k = rr - j * L.tw;
    const int t = a * L.tt + i, h = b * L.th + j, w = c * L.tw + k;
    return (t < L.T && h < L.H && w < L.W) ? (t * L.H + h) * L.W + w : -1;
  }
  const int g = tile / L.tiles_per_group;
  const int chunk = tile - g * L.tiles_per_group;
  const int pos = chunk * L.C + r;
  if (pos >= L.group_len) return -1;
  const int Hg = L.H / L.sh, Wg = L.W / L.sw;
  const int t = pos / (Hg * Wg);
  const int rem = pos - t * (Hg * Wg);
  const int hh = rem / Wg;
  const int ww = rem - hh * Wg;
  const int rh = g / L.sw, rw = g - rh * L.sw;
  return (t * L.H + hh * L.sh + rh) * L.W + ww * L.sw + rw;
}

// Real-token description of one tile, cheap to test per row:
// 3D tiles: real rows are those with (i < vt, j < vh, k < vw);
// Skiparse: real rows are r < vlen.
struct TileValid {
  int full;       // 1 if every row is real
  int vt, vh, vw;
  int vlen;
};

__device__ __forceinline__ TileValid tile_valid(const DevLayout& L, int tile) {
  TileValid v;
  if (L.kind == 0) {
    const int per_a = L.nth * L.ntw;
    const int a = tile / per_a;
    const int rem = tile - a * per_a;
    const int b = rem / L.ntw;
    const int c = rem - b * L.ntw;
    v.vt = min(L.tt, L.T - a * L.tt);
    v.vh = min(L.th, L.H - b * L.th);
    v.vw = min(L.tw, L.W - c * L.tw);
    v.vlen = L.C;
    v.full = (v.vt == L.tt && v.vh == L.th && v.vw == L.tw);
  } else {
    const int chunk = tile % L.tiles_per_group;
    v.vt = v.vh = v.vw = 0;
    v.vlen = min(L.C, L.group_len - chunk * L.C);
    v.full = (v.vlen == L.C);
  }
  return v;
}

__device__ __forceinline__ bool row_is_real(const DevLayout& L, const TileValid& v, int r) {
  if (v.full) return true;
  if (L.kind == 0) {
    const int per_i = L.th * L.tw;
    const int i = r / per_i;
    const int rr = r - i * per_i;
    const int j = rr / L.tw;
    const int k = rr - j * L.tw;
    return i < v.vt && j < v.vh && k < v.vw;
  }
  return r < v.vlen;
}

__host__ __device__ inline int real_rows(const DevLayout& L, const TileValid& v) {
  return L.kind == 0 ? v.vt * v.vh * v.vw : v.vlen;
}

// Workgroup index -> work item, so that each of the 8 XCDs (which receive
// workgroups round-robin) processes one contiguous range of work items and
// items that share K/V stay in one XCD's L2.
__device__ __forceinline__ int xcd_remap(int i, int n) {
  const int q = n >> 3, r = n & 7;
  const int x = i & 7, j = i >> 3;
  return x * q + min(x, r) + j;
}

// Workgroup index -> work item in chunks of G consecutive items dealt to the
// XCDs in turn, so that every XCD gets a slice of every head: for per-head
// routed lists, whose lengths differ from head to head, this keeps the XCDs
// equally loaded; neighbouring query tiles still share an L2 within a chunk.
// The tail that does not fill a round of 8 chunks is split contiguously.
__device__ __forceinline__ int xcd_chunked(int i, int n, int G) {
  const int R = 8 * G, full = n / R;
  const int x = i & 7, k = i >> 3;
  if (k < full * G) return ((k / G) * 8 + x) * G + (k % G);
  return full * R + xcd_remap(i - full * R, n - full * R);
}

// ----- launchers (return hipError_t of the launch) -----
hipError_t launch_permute(const DevLayout& L, int esize, const void* src, void* dst, int inverse,
                          hipStream_t s);
// natural bf16 -> tiled V in the bf16 P.V operand layout (64-token tiles, d % 8 == 0, d <= 256)
hipError_t launch_permute_vop(const DevLayout& L, const void* src, void* dst, hipStream_t s);
hipError_t launch_mask_window(const DevLayout& L, int rt, int rh, int rw, int max_kv,
                              int32_t* kv_idx, int32_t* kv_cnt, hipStream_t s);
hipError_t launch_route(const DevLayout& L, const void* q, const void* k, float coarse_scale,
                        int top_k, float top_p, int k_floor, int max_kv, int32_t* kv_idx,
                        int32_t* kv_cnt, float* scores, void* ws, hipStream_t s);
hipError_t launch_route_pooled(const DevLayout& L, const float* q_pooled, const float* k_pooled,
                               float coarse_scale, int top_k, float top_p, int k_floor, int max_kv,
                               int32_t* kv_idx, int32_t* kv_cnt, float* scores, hipStream_t s);
hipError_t launch_permute_pool(const DevLayout& L, const void* src, void* dst, float* pooled,
                               hipStream_t s);
// workspace of vsa_build_mask_topk: the pooled means of Q and K
size_t route_workspace_bytes(const DevLayout& L);
hipError_t launch_quant_fp8(const DevLayout& L, const void* x, uint8_t* codes, float* scales,
                            bool v_operand, hipStream_t s);
// natural order -> tiled e4m3 codes (+ scales, + tile means when pooled != null)
hipError_t launch_quant_fp8_nat(const DevLayout& L, const void* x, uint8_t* codes, float* scales,
                                float* pooled, bool v_operand, hipStream_t s);
hipError_t launch_mask_window_grouped(const DevLayout& L, int gt, int gh, int gw, int et, int eh,
                                      int ew, int max_kv, int32_t* kv_idx, int32_t* kv_cnt,
                                      hipStream_t s);
hipError_t launch_quant_fp8_grouped(const DevLayout& L, int gt, int gh, int gw, const void* x,
                                    uint8_t* codes, float* scales, bool v_operand, hipStream_t s);

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  const int32_t* kv_idx;   // null: dense
  const int32_t* kv_cnt;
  int max_kv;
  int list_mode;           // 0 shared table, 1 per (batch, head), 2 shared table walked per tile
  float scale_log2;        // softmax scale * log2(e)
  void* out;
  float* lse;
  int natural_io;          // out written to [B, T*H*W, heads, d]; bf16/f32 also read q from it
  const int32_t* work_order;   // list_mode 1 only (one query tile per workgroup): item dealt
                               // at position p is work_order[p]; null: index order
};
hipError_t launch_attn(const DevLayout& L, int dtype, const AttnArgs& a, hipStream_t s);

// Heavy-first order of the (b, head, query tile) items of per-head lists:
// heads by total pairs, then query tiles by list length, both descending.
size_t work_order_lds_bytes(const DevLayout& L);
hipError_t launch_work_order(const DevLayout& L, const int32_t* kv_cnt, int32_t* order, hipStream_t s);

// For every key tile j (per list head): the ascending query tiles whose
// list holds j. q_idx [LH, n_tiles, n_tiles], q_cnt [LH, n_tiles].
hipError_t launch_transpose_lists(const DevLayout& L, const int32_t* kv_idx, const int32_t* kv_cnt,
                                  int max_kv, int list_mode, int32_t* q_idx, int32_t* q_cnt,
                                  hipStream_t s);

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const void* dout;
  const float* lse;
  const int32_t* kv_idx;   // forward lists (null: dense)
  const int32_t* kv_cnt;
  int max_kv;
  const int32_t* q_idx;    // transposed lists (null: dense)
  const int32_t* q_cnt;
  int list_mode;           // 0 shared tables, 1 per (batch, head)
  float scale;             // softmax scale
  float scale_log2;        // softmax scale * log2(e)
  void* dq;
  void* dk;
  void* dv;
  float2* rowstat;         // workspace: per row {lse * log2(e) (+inf: no weight), dO . O}
};
size_t attn_bwd_workspace_bytes(const DevLayout& L);
// Built-in scratch of the allocation-free backward (row statistics): its
// size, and its device address on the current device (looked up once per
// device with hipGetSymbolAddress, then cached).
constexpr size_t kBwdScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;
hipError_t attn_bwd_scratch(void** ptr);
hipError_t launch_attn_bwd(const DevLayout& L, int dtype, const BwdArgs& a, hipStream_t s);

}  // namespace vsa
