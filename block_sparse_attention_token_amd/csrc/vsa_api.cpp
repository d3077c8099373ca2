// C ABI of libvsa: argument checks, layout derivation and kernel dispatch.
// Every check runs before any launch, so an error return means nothing was
// written. Nothing here allocates device memory or synchronises.
#include <math.h>
#include <stdarg.h>

#include <algorithm>
#include <stdio.h>
#include <string.h>

#include <string>

#include "../../include/vsa.h"
#include "vsa_internal.h"

namespace {

thread_local std::string g_last_error;

vsa_status fail(vsa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
vsa_status fail(vsa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

vsa_status ok() {
  g_last_error.clear();
  return VSA_OK;
}

vsa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(VSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Derive every size of a layout; returns VSA_OK or an error (message set).
vsa_status derive(const vsa_layout* lay, vsa::DevLayout* L, vsa_layout_info* info) {
  if (!lay) return fail(VSA_ERR_INVALID, "layout is NULL");
  if (lay->batch < 1 || lay->heads < 1 || lay->head_dim < 1)
    return fail(VSA_ERR_INVALID, "batch, heads and head_dim must be >= 1");
  if (lay->T < 1 || lay->H < 1 || lay->W < 1) return fail(VSA_ERR_INVALID, "T, H, W must be >= 1");
  if (lay->tile_t < 1 || lay->tile_h < 1 || lay->tile_w < 1)
    return fail(VSA_ERR_INVALID, "tile extents must be >= 1");
  const long long C = (long long)lay->tile_t * lay->tile_h * lay->tile_w;
  const long long n_tokens = (long long)lay->T * lay->H * lay->W;
  if (C > 4096) return fail(VSA_ERR_INVALID, "tile of %lld tokens exceeds 4096", C);
  vsa::DevLayout d{};
  d.B = lay->batch;
  d.heads = lay->heads;
  d.d = lay->head_dim;
  d.T = lay->T;
  d.H = lay->H;
  d.W = lay->W;
  d.kind = lay->kind;
  d.tt = lay->tile_t;
  d.th = lay->tile_h;
  d.tw = lay->tile_w;
  d.sh = 1;
  d.sw = 1;
  d.C = (int)C;
  d.n_tokens = n_tokens;
  long long n_tiles;
  if (lay->kind == VSA_TILE3D) {
    d.ntt = (lay->T + lay->tile_t - 1) / lay->tile_t;
    d.nth = (lay->H + lay->tile_h - 1) / lay->tile_h;
    d.ntw = (lay->W + lay->tile_w - 1) / lay->tile_w;
    n_tiles = (long long)d.ntt * d.nth * d.ntw;
    d.tiles_per_group = (int)n_tiles;
    d.group_len = (int)n_tokens;
  } else if (lay->kind == VSA_SKIPARSE2D) {
    if (lay->stride_h < 1 || lay->stride_w < 1)
      return fail(VSA_ERR_INVALID, "Skiparse strides must be >= 1");
    if (lay->H % lay->stride_h || lay->W % lay->stride_w)
      return fail(VSA_ERR_INVALID, "Skiparse needs H %% stride_h == 0 and W %% stride_w == 0");
    d.sh = lay->stride_h;
    d.sw = lay->stride_w;
    const long long glen = (long long)lay->T * (lay->H / d.sh) * (lay->W / d.sw);
    const long long tpg = (glen + C - 1) / C;
    n_tiles = tpg * d.sh * d.sw;
    d.tiles_per_group = (int)tpg;
    d.group_len = (int)glen;
  } else {
    return fail(VSA_ERR_INVALID, "unknown layout kind %d", lay->kind);
  }
  if (n_tiles > (1 << 22)) return fail(VSA_ERR_INVALID, "too many tiles (%lld)", n_tiles);
  d.n_tiles = (int)n_tiles;
  d.n_padded = n_tiles * C;
  // element offsets are computed in 64-bit; indices of rows per (b, head) fit 32-bit
  if (d.n_padded >= (1ll << 31) || n_tokens >= (1ll << 31))
    return fail(VSA_ERR_INVALID, "grid too large");
  if (L) *L = d;
  if (info) {
    info->n_tokens = n_tokens;
    info->n_padded = d.n_padded;
    info->n_tiles = d.n_tiles;
    info->tile_tokens = d.C;
    info->n_groups = lay->kind == VSA_SKIPARSE2D ? d.sh * d.sw : 1;
    info->tiles_per_group = d.tiles_per_group;
    info->group_len = d.group_len;
    info->tiles_t = lay->kind == VSA_TILE3D ? d.ntt : 0;
    info->tiles_h = lay->kind == VSA_TILE3D ? d.nth : 0;
    info->tiles_w = lay->kind == VSA_TILE3D ? d.ntw : 0;
  }
  return VSA_OK;
}

int longest_window_list(const vsa::DevLayout& L, int rt, int rh, int rw) {
  if (rt < 0 || rh < 0 || rw < 0) return L.n_tiles;
  if (L.kind == VSA_SKIPARSE2D) return L.tiles_per_group;
  auto ax = [](int n, int r) { return (int)std::min<long long>(2ll * r + 1, n); };
  return ax(L.ntt, rt) * ax(L.nth, rh) * ax(L.ntw, rw);
}

}  // namespace

extern "C" {

vsa_status vsa_layout_query(const vsa_layout* layout, vsa_layout_info* info) {
  if (!info) return fail(VSA_ERR_INVALID, "info is NULL");
  const vsa_status st = derive(layout, nullptr, info);
  return st == VSA_OK ? ok() : st;
}

vsa_status vsa_tile_permute(const vsa_layout* layout, int32_t dtype, const void* src, void* dst,
                            int32_t inverse, void* stream) {
  vsa::DevLayout L;
  vsa_status st = derive(layout, &L, nullptr);
  if (st != VSA_OK) return st;
  if (!src || !dst) return fail(VSA_ERR_INVALID, "src and dst must be non-NULL");
  if (!aligned16(src) || !aligned16(dst)) return fail(VSA_ERR_INVALID, "pointers must be 16-byte aligned");
  int esize;
  if (dtype == VSA_F32) esize = 4;
  else if (dtype == VSA_BF16) esize = 2;
  else return fail(VSA_ERR_UNSUPPORTED, "permute supports VSA_F32 and VSA_BF16 only");
  if ((L.d * esize) % 16) return fail(VSA_ERR_UNSUPPORTED, "head_dim * element size must be a multiple of 16 bytes");
  if (L.n_tiles > 65535 * 64 || L.heads > 65535 || L.B > 65535)
    return fail(VSA_ERR_UNSUPPORTED, "grid too large for one launch");
  return hip_status(vsa::launch_permute(L, esize, src, dst, inverse ? 1 : 0,
                                        static_cast<hipStream_t>(stream)), "vsa_tile_permute");
}

vsa_status vsa_tile_permute_v(const vsa_layout* layout, const void* src, void* dst, void* stream) {
  vsa::DevLayout L;
  vsa_status st = derive(layout, &L, nullptr);
  if (st != VSA_OK) return st;
  if (!src || !dst) return fail(VSA_ERR_INVALID, "src and dst must be non-NULL");
  if (!aligned16(src) || !aligned16(dst)) return fail(VSA_ERR_INVALID, "pointers must be 16-byte aligned");
  if (L.C != 64) return fail(VSA_ERR_UNSUPPORTED, "the V operand layout needs 64-token tiles");
  if (L.d % 8 || L.d > 256) return fail(VSA_ERR_UNSUPPORTED, "head_dim must be <= 256 and a multiple of 8");
  if (L.heads > 65535 || L.B > 65535)
    return fail(VSA_ERR_UNSUPPORTED, "grid too large for one launch");
  const long long sb = (long long)L.B * L.n_tokens * L.heads * L.d * 2;
  const long long db = (long long)L.B * L.heads * L.n_padded * L.d * 2;
  const char* s0 = static_cast<const char*>(src);
  const char* d0 = static_cast<const char*>(dst);
  if (s0 < d0 + db && d0 < s0 + sb) return fail(VSA_ERR_INVALID, "src and dst must not overlap");
  return hip_status(vsa::launch_permute_vop(L, src, dst, static_cast<hipStream_t>(stream)),
                    "vsa_tile_permute_v");
}

vsa_status vsa_tile_permute_pool(const vsa_layout* layout, const void* src, void* dst,
                                 float* pooled, void* stream) {
  vsa::DevLayout L;
  vsa_status st = derive(layout, &L, nullptr);
  if (st != VSA_OK) return st;
  if (!src || !pooled) return fail(VSA_ERR_INVALID, "src and pooled must be non-NULL");
  if (!aligned16(src) || !aligned16(dst) || !aligned16(pooled))
    return fail(VSA_ERR_INVALID, "src, dst and pooled must be 16-byte aligned");
  if (L.d % 8 || L.d > 256) return fail(VSA_ERR_UNSUPPORTED, "head_dim must be <= 256 and a multiple of 8");
  if (L.heads > 65535 || L.B > 65535) return fail(VSA_ERR_UNSUPPORTED, "grid too large for one launch");
  const size_t bytes = (size_t)L.B * L.heads * L.d * 2;
  const char* s0 = static_cast<const char*>(src);
  const char* d0 = static_cast<const char*>(dst);
  const char* p0 = reinterpret_cast<const char*>(pooled);
  const size_t nat_b = bytes * L.n_tokens, til_b = bytes * L.n_padded;
  const size_t pool_b = (size_t)L.B * L.heads * L.n_tiles * L.d * sizeof(float);
  auto overlap = [](const char* a, size_t na, const char* b, size_t nb) { return a < b + nb && b < a + na; };
  if ((dst && overlap(s0, nat_b, d0, til_b)) || overlap(s0, nat_b, p0, pool_b) ||
      (dst && overlap(d0, til_b, p0, pool_b)))
    return fail(VSA_ERR_INVALID, "src, dst and pooled must not overlap");
  return hip_status(vsa::launch_permute_pool(L, src, dst, pooled, static_cast<hipStream_t>(stream)),
                    "vsa_tile_permute_pool");
}

vsa_status vsa_build_mask_window(const vsa_layout* layout, int32_t rt, int32_t rh, int32_t rw,
                                 int32_t max_kv, int32_t* kv_idx, int32_t* kv_cnt, void* stream) {
  vsa::DevLayout L;
  vsa_status st = derive(layout, &L, nullptr);
  if (st != VSA_OK) return st;
  if (!kv_idx || !kv_cnt) return fail(VSA_ERR_INVALID, "kv_idx and kv_cnt must be non-NULL");
  const int need = longest_window_list(L, rt, rh, rw);
  if (max_kv < need) return fail(VSA_ERR_INVALID, "max_kv %d < longest list %d", max_kv, need);
  return hip_status(vsa::launch_mask_window(L, rt, rh, rw, max_kv, kv_idx, kv_cnt,
                                            static_cast<hipStream_t>(stream)),
                    "vsa_build_mask_window");
}

// Longest list of a grouped window: per axis the most tiles any query's
// window covers, multiplied over the axes (the window is a box).
static int longest_grouped_list(const vsa::DevLayout& L, int gt, int gh, int gw, int et, int eh,
                                int ew) {
  auto axis = [](int n, int g, int e) {
    const int ng = (n + g - 1) / g;
    int best = 0;
    for (int X = 0; X < ng; ++X) {
      const int lo = std::max(X - (e - 1) / 2, 0), hi = std::min(X - (e - 1) / 2 + e - 1, ng - 1);
      best = std::max(best, std::min((hi + 1) * g, n) - lo * g);
    }
    return best;
  };
  return axis(L.ntt, gt, et) * axis(L.nth, gh, eh) * axis(L.ntw, gw, ew);
}

vsa_status vsa_build_mask_window_grouped(const vsa_layout* layout, int32_t gt, int32_t gh,
                                         int32_t gw, int32_t et, int32_t eh, int32_t ew,
                                         int32_t max_kv, int32_t* kv_idx, int32_t* kv_cnt,
                                         void* stream) {
  vsa::DevLayout L;
  vsa_status st = derive(layout, &L, nullptr);
  if (st != VSA_OK) return st;
  if (L.kind != VSA_TILE3D) return fail(VSA_ERR_UNSUPPORTED, "grouped windows need VSA_TILE3D");
  if (!kv_idx || !kv_cnt) return fail(VSA_ERR_INVALID, "kv_idx and kv_cnt must be non-NULL");
  if (gt < 1 || gh < 1 || gw < 1 || et < 1 || eh < 1 || ew < 1)
    return fail(VSA_ERR_INVALID, "group sizes and extents must be >= 1");
  const int need = longest_grouped_list(L, gt, gh, gw, et, eh, ew);
  if (max_kv < need) return fail(VSA_ERR_INVALID, "max_kv %d < longest list %d", max_kv, need);
  return hip_status(vsa::launch_mask_window_grouped(L, gt, gh, gw, et, eh, ew, max_kv, kv_idx, kv_cnt,
                                                    static_cast<hipStream_t>(stream)),
                    "vsa_build_mask_window_grouped");
}

size_t vsa_build_mask_topk_workspace(const vsa_layout* layout) {
  vsa::DevLayout L;
  if (derive(layout, &L, nullptr) != VSA_OK) return 0;
  return vsa::route_workspace_bytes(L);
}

// Checks shared by both routing entry points (after the input pointers).
// need_ws: the call pools Q and K into the workspace (vsa_build_mask_topk);
// the call from pooled means needs none.
static vsa_status check_route(const vsa::DevLayout& L, float coarse_scale, int32_t top_k,
                              float top_p, int32_t k_floor, int32_t max_kv, const void* workspace,
                              size_t workspace_bytes, bool need_ws) {
  if (L.n_tiles > 4096) return fail(VSA_ERR_UNSUPPORTED, "routing supports at most 4096 tiles");
  if (L.d % 8 || L.d > 256) return fail(VSA_ERR_UNSUPPORTED, "routing needs head_dim <= 256, multiple of 8");
  if (!isfinite(coarse_scale)) return fail(VSA_ERR_INVALID, "coarse_scale must be finite");
  if (!(top_p <= 1.0f) || isnan(top_p)) return fail(VSA_ERR_INVALID, "top_p must be <= 1");
  if (top_p > 0.0f) {
    if (k_floor < 0) return fail(VSA_ERR_INVALID, "k_floor must be >= 0");
    if (max_kv < L.n_tiles) return fail(VSA_ERR_INVALID, "top-p needs max_kv >= n_tiles (%d)", L.n_tiles);
  } else {
    if (top_k < 1) return fail(VSA_ERR_INVALID, "top_k must be >= 1 when top_p <= 0");
    const int need = std::min(top_k, L.n_tiles);
    if (max_kv < need) return fail(VSA_ERR_INVALID, "max_kv %d < %d", max_kv, need);
  }
  if (L.B * L.heads > 65535) return fail(VSA_ERR_UNSUPPORTED, "batch * heads too large");
  if (need_ws) {
    const size_t bytes = vsa::route_workspace_bytes(L);
    if (!workspace || workspace_bytes < bytes)
      return fail(VSA_ERR_WORKSPACE, "workspace of %zu bytes needed", bytes);
    if (!aligned16(workspace)) return fail(VSA_ERR_INVALID, "workspace must be 16-byte aligned");
  }
  return VSA_OK;
}

vsa_status vsa_build_mask_topk(const vsa_layout* layout, const void* q_tiled, const void* k_tiled,
                               float coarse_scale, int32_t top_k, float top_p, int32_t k_floor,
                               int32_t max_kv, int32_t* kv_idx, int32_t* kv_cnt, float* scores,
                               void* workspace, size_t workspace_bytes, void* stream) {
  vsa::DevLayout L;
  vsa_status st = derive(layout, &L, nullptr);
  if (st != VSA_OK) return st;
  if (!q_tiled || !k_tiled || !kv_idx || !kv_cnt)
    return fail(VSA_ERR_INVALID, "q_tiled, k_tiled, kv_idx and kv_cnt must be non-NULL");
  if (!aligned16(q_tiled) || !aligned16(k_tiled)) return fail(VSA_ERR_INVALID, "pointers must be 16-byte aligned");
  st = check_route(L, coarse_scale, top_k, top_p, k_floor, max_kv, workspace, workspace_bytes, true);
  if (st != VSA_OK) return st;
  return hip_status(vsa::launch_route(L, q_tiled, k_tiled, coarse_scale, top_k, top_p, k_floor,
                                      max_kv, kv_idx, kv_cnt, scores, workspace,
                                      static_cast<hipStream_t>(stream)),
                    "vsa_build_mask_topk");
}

vsa_status vsa_build_mask_topk_pooled(const vsa_layout* layout, const float* q_pooled,
                                      const float* k_pooled, float coarse_scale, int32_t top_k,
                                      float top_p, int32_t k_floor, int32_t max_kv,
                                      int32_t* kv_idx, int32_t* kv_cnt, float* scores,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  vsa::DevLayout L;
  vsa_status st = derive(layout, &L, nullptr);
  if (st != VSA_OK) return st;
  if (!q_pooled || !k_pooled || !kv_idx || !kv_cnt)
    return fail(VSA_ERR_INVALID, "q_pooled, k_pooled, kv_idx and kv_cnt must be non-NULL");
  if (!aligned16(q_pooled) || !aligned16(k_pooled))
    return fail(VSA_ERR_INVALID, "pooled means must be 16-byte aligned");
  st = check_route(L, coarse_scale, top_k, top_p, k_floor, max_kv, workspace, workspace_bytes, false);
  if (st != VSA_OK) return st;
  (void)workspace;
  (void)workspace_bytes;
  return hip_status(vsa::launch_route_pooled(L, q_pooled, k_pooled, coarse_scale, top_k, top_p,
                                             k_floor, max_kv, kv_idx, kv_cnt, scores,
                                             static_cast<hipStream_t>(stream)),
                    "vsa_build_mask_topk_pooled");
}

static vsa_status quant_fp8(const vsa_layout* layout, const void* x_tiled, uint8_t* codes,
                            float* scales, bool v_operand, void* stream, const char* name) {
  vsa::DevLayout L;
  vsa_status st = derive(layout, &L, nullptr);
  if (st != VSA_OK) return st;
  if (!x_tiled || !codes || !scales) return fail(VSA_ERR_INVALID, "x_tiled, codes and scales must be non-NULL");
  if (!aligned16(x_tiled) || ((uintptr_t)codes & (v_operand ? 15u : 7u)))
    return fail(VSA_ERR_INVALID, "misaligned pointer");
  if (L.d % 8) return fail(VSA_ERR_UNSUPPORTED, "head_dim must be a multiple of 8");
  if (v_operand && (L.C != 64 || L.d != 128))
    return fail(VSA_ERR_UNSUPPORTED, "the P.V operand layout needs 64-token tiles and head_dim 128");
  if (L.heads > 65535 || L.B > 65535) return fail(VSA_ERR_UNSUPPORTED, "grid too large");
  return hip_status(vsa::launch_quant_fp8(L, x_tiled, codes, scales, v_operand,
                                          static_cast<hipStream_t>(stream)),
                    name);
}

vsa_status vsa_quant_fp8_tiles(const vsa_layout* layout, const void* x_tiled, uint8_t* codes,
                               float* scales, void* stream) {
  return quant_fp8(layout, x_tiled, codes, scales, false, stream, "vsa_quant_fp8_tiles");
}

vsa_status vsa_quant_fp8_tiles_v(const vsa_layout* layout, const void* x_tiled, uint8_t* codes,
                                 float* scales, void* stream) {
  return quant_fp8(layout, x_tiled, codes, scales, true, stream, "vsa_quant_fp8_tiles_v");
}

vsa_status vsa_quant_fp8_tiles_grouped(const vsa_layout* layout, int32_t gt, int32_t gh, int32_t gw,
                                       const void* x_tiled, uint8_t* codes, float* scales,
                                       int32_t v_operand, void* stream) {
  vsa::DevLayout L;
  vsa_status st = derive(layout, &L, nullptr);
  if (st != VSA_OK) return st;
  if (L.kind != VSA_TILE3D) return fail(VSA_ERR_UNSUPPORTED, "grouped scales need VSA_TILE3D");
  if (gt < 1 || gh < 1 || gw < 1) return fail(VSA_ERR_INVALID, "group sizes must be >= 1");
  if (!x_tiled || !codes || !scales) return fail(VSA_ERR_INVALID, "x_tiled, codes and scales must be non-NULL");
  if (!aligned16(x_tiled) || ((uintptr_t)codes & (v_operand ? 15u : 7u)))
    return fail(VSA_ERR_INVALID, "misaligned pointer");
  if (L.d % 8) return fail(VSA_ERR_UNSUPPORTED, "head_dim must be a multiple of 8");
  if (v_operand && (L.C != 64 || L.d != 128))
    return fail(VSA_ERR_UNSUPPORTED, "the P.V operand layout needs 64-token tiles and head_dim 128");
  if (L.heads > 65535 || L.B > 65535) return fail(VSA_ERR_UNSUPPORTED, "grid too large");
  return hip_status(vsa::launch_quant_fp8_grouped(L, gt, gh, gw, x_tiled, codes, scales, v_operand != 0,
                                                  static_cast<hipStream_t>(stream)),
                    "vsa_quant_fp8_tiles_grouped");
}

vsa_status vsa_quant_fp8_tiles_nat(const vsa_layout* layout, const void* x_nat, uint8_t* codes,
                                   float* scales, float* pooled, int32_t v_operand, void* stream) {
  vsa::DevLayout L;
  vsa_status st = derive(layout, &L, nullptr);
  if (st != VSA_OK) return st;
  if (!x_nat || !codes || !scales) return fail(VSA_ERR_INVALID, "x_nat, codes and scales must be non-NULL");
  if (!aligned16(x_nat) || ((uintptr_t)codes & (v_operand ? 15u : 7u)) || !aligned16(pooled))
    return fail(VSA_ERR_INVALID, "misaligned pointer");
  if (L.d % 8 || L.d > 256) return fail(VSA_ERR_UNSUPPORTED, "head_dim must be <= 256 and a multiple of 8");
  const int chunks = L.d / 8, groups = 256 / chunks;
  if ((L.C + groups - 1) / groups > 8)
    return fail(VSA_ERR_UNSUPPORTED, "tile_tokens * head_dim must be at most 16,384 (one tile in registers)");
  if (v_operand && (L.C != 64 || L.d != 128))
    return fail(VSA_ERR_UNSUPPORTED, "the P.V operand layout needs 64-token tiles and head_dim 128");
  if (L.heads > 65535 || L.B > 65535) return fail(VSA_ERR_UNSUPPORTED, "grid too large");
  const size_t nat_b = (size_t)L.B * L.n_tokens * L.heads * L.d * 2;
  const size_t code_b = (size_t)L.B * L.heads * L.n_padded * L.d;
  const char* x0 = static_cast<const char*>(x_nat);
  const char* c0 = reinterpret_cast<const char*>(codes);
  if (x0 < c0 + code_b && c0 < x0 + nat_b) return fail(VSA_ERR_INVALID, "x_nat and codes must not overlap");
  return hip_status(vsa::launch_quant_fp8_nat(L, x_nat, codes, scales, pooled, v_operand != 0,
                                              static_cast<hipStream_t>(stream)),
                    "vsa_quant_fp8_tiles_nat");
}

// The attention kernels address one (batch, head) slice of a tiled tensor
// through a buffer resource with 32-bit offsets.
static vsa_status check_slice(const vsa::DevLayout& L, int32_t dtype) {
  const long long es = dtype == VSA_F32 ? 4 : (dtype == VSA_BF16 || dtype == VSA_BF16_VOP ? 2 : 1);
  if ((long long)L.n_padded * L.d * es > 0x7FFFFFFFll)
    return fail(VSA_ERR_UNSUPPORTED, "one (batch, head) slice of a tiled tensor must stay below 2 GiB");
  return VSA_OK;
}

// A work order only applies to per-head lists, which are walked one query
// tile per workgroup.
static vsa_status check_order(const int32_t* work_order, const int32_t* kv_idx, int32_t list_mode) {
  if (!work_order) return VSA_OK;
  if (!kv_idx || list_mode != 1) return fail(VSA_ERR_INVALID, "work_order needs per-head lists (list_mode 1)");
  if ((uintptr_t)work_order & 3u) return fail(VSA_ERR_INVALID, "work_order must be 4-byte aligned");
  return VSA_OK;
}

vsa_status vsa_build_work_order(const vsa_layout* layout, const int32_t* kv_cnt, int32_t* order,
                                void* stream) {
  vsa::DevLayout L;
  vsa_status st = derive(layout, &L, nullptr);
  if (st != VSA_OK) return st;
  if (!kv_cnt || !order) return fail(VSA_ERR_INVALID, "kv_cnt and order must be non-NULL");
  if (((uintptr_t)kv_cnt & 3u) || ((uintptr_t)order & 3u))
    return fail(VSA_ERR_INVALID, "kv_cnt and order must be 4-byte aligned");
  const long long items = (long long)L.B * L.heads * L.n_tiles;
  if (items > 0x7FFFFFFFll) return fail(VSA_ERR_UNSUPPORTED, "too many query tiles");
  if (vsa::work_order_lds_bytes(L) > 65536)
    return fail(VSA_ERR_UNSUPPORTED, "n_tiles + batch * heads must be at most 16,384");
  const char* c0 = reinterpret_cast<const char*>(kv_cnt);
  const char* o0 = reinterpret_cast<const char*>(order);
  if (c0 < o0 + items * 4 && o0 < c0 + items * 4) return fail(VSA_ERR_INVALID, "kv_cnt and order must not overlap");
  return hip_status(vsa::launch_work_order(L, kv_cnt, order, static_cast<hipStream_t>(stream)),
                    "vsa_build_work_order");
}

vsa_status vsa_block_sparse_attn_fwd(const vsa_layout* layout, int32_t dtype, const void* q,
                                     const void* k, const void* v, const float* q_scale,
                                     const float* k_scale, const float* v_scale,
                                     const int32_t* kv_idx, const int32_t* kv_cnt, int32_t max_kv,
                                     int32_t list_mode, const int32_t* work_order,
                                     float softmax_scale, void* out, float* lse, void* stream) {
  vsa::DevLayout L;
  vsa_status st = derive(layout, &L, nullptr);
  if (st != VSA_OK) return st;
  if (!q || !k || !v || !out) return fail(VSA_ERR_INVALID, "q, k, v and out must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(VSA_ERR_INVALID, "pointers must be 16-byte aligned");
  if ((kv_idx == nullptr) != (kv_cnt == nullptr))
    return fail(VSA_ERR_INVALID, "kv_idx and kv_cnt must both be set or both be NULL");
  if (kv_idx && max_kv < 1) return fail(VSA_ERR_INVALID, "max_kv must be >= 1");
  if (list_mode < 0 || list_mode > 2) return fail(VSA_ERR_INVALID, "list_mode must be 0, 1 or 2");
  st = check_order(work_order, kv_idx, list_mode);
  if (st != VSA_OK) return st;
  if (!isfinite(softmax_scale)) return fail(VSA_ERR_INVALID, "softmax_scale must be finite");
  if (dtype != VSA_F32 && dtype != VSA_BF16 && dtype != VSA_FP8_E4M3 && dtype != VSA_FP8_E4M3_VOP &&
      dtype != VSA_BF16_VOP)
    return fail(VSA_ERR_INVALID, "unknown dtype %d", dtype);
  if (dtype == VSA_BF16_VOP && L.C != 64)
    return fail(VSA_ERR_UNSUPPORTED, "the bf16 V operand layout needs 64-token tiles");
  if (dtype == VSA_FP8_E4M3 || dtype == VSA_FP8_E4M3_VOP) {
    if (!q_scale || !k_scale || !v_scale) return fail(VSA_ERR_INVALID, "fp8 needs q_scale, k_scale and v_scale");
    if (L.C != 64 || L.d != 128) return fail(VSA_ERR_UNSUPPORTED, "fp8 attention needs 64-token tiles and head_dim 128");
  } else {
    if (L.C != 32 && L.C != 64) return fail(VSA_ERR_UNSUPPORTED, "attention needs 32- or 64-token tiles");
    if (L.d != 64 && L.d != 128) return fail(VSA_ERR_UNSUPPORTED, "attention needs head_dim 64 or 128");
  }
  const long long work = (long long)L.B * L.heads * L.n_tiles;
  if (work > 0x7FFFFFFFll) return fail(VSA_ERR_UNSUPPORTED, "too many query tiles for one launch");
  st = check_slice(L, dtype);
  if (st != VSA_OK) return st;
  vsa::AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.kv_idx = kv_idx;
  a.kv_cnt = kv_cnt;
  a.max_kv = kv_idx ? max_kv : L.n_tiles;
  a.list_mode = list_mode;
  a.work_order = work_order;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.out = out;
  a.lse = lse;
  return hip_status(vsa::launch_attn(L, dtype, a, static_cast<hipStream_t>(stream)),
                    "vsa_block_sparse_attn_fwd");
}

vsa_status vsa_build_transposed_lists(const vsa_layout* layout, const int32_t* kv_idx,
                                      const int32_t* kv_cnt, int32_t max_kv, int32_t list_mode,
                                      int32_t* q_idx, int32_t* q_cnt, void* stream) {
  vsa::DevLayout L;
  vsa_status st = derive(layout, &L, nullptr);
  if (st != VSA_OK) return st;
  if (!kv_idx || !kv_cnt || !q_idx || !q_cnt)
    return fail(VSA_ERR_INVALID, "kv_idx, kv_cnt, q_idx and q_cnt must be non-NULL");
  if (max_kv < 1) return fail(VSA_ERR_INVALID, "max_kv must be >= 1");
  if (list_mode != 0 && list_mode != 1) return fail(VSA_ERR_INVALID, "list_mode must be 0 or 1");
  const long long lh = list_mode ? (long long)L.B * L.heads : 1;
  if (lh > 65535) return fail(VSA_ERR_UNSUPPORTED, "more than 65535 list heads");
  return hip_status(vsa::launch_transpose_lists(L, kv_idx, kv_cnt, max_kv, list_mode, q_idx, q_cnt,
                                                static_cast<hipStream_t>(stream)),
                    "vsa_build_transposed_lists");
}

size_t vsa_block_sparse_attn_bwd_workspace(const vsa_layout* layout) {
  vsa::DevLayout L;
  if (derive(layout, &L, nullptr) != VSA_OK) return 0;
  return vsa::attn_bwd_workspace_bytes(L);
}

// Argument checks and argument block shared by both backward entry points
// (everything but the workspace).
static vsa_status bwd_args(const vsa_layout* layout, int32_t dtype, const void* q, const void* k,
                           const void* v, const void* out, const void* dout, const float* lse,
                           const int32_t* kv_idx, const int32_t* kv_cnt, int32_t max_kv,
                           const int32_t* q_idx, const int32_t* q_cnt, int32_t list_mode,
                           float softmax_scale, void* dq, void* dk, void* dv, vsa::DevLayout* L,
                           vsa::BwdArgs* a) {
  vsa_status st = derive(layout, L, nullptr);
  if (st != VSA_OK) return st;
  if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv)
    return fail(VSA_ERR_INVALID, "q, k, v, out, dout, lse, dq, dk and dv must be non-NULL");
  const void* ptrs[] = {q, k, v, out, dout, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(VSA_ERR_INVALID, "tensor pointers must be 16-byte aligned");
  if (dq == dk || dq == dv || dk == dv) return fail(VSA_ERR_INVALID, "dq, dk and dv must be distinct");
  for (const void* g : {dq, dk, dv})
    for (const void* x : {q, k, v, out, dout})
      if (g == x) return fail(VSA_ERR_INVALID, "gradients must not alias the inputs");
  const bool lists = kv_idx || kv_cnt || q_idx || q_cnt;
  if (lists && !(kv_idx && kv_cnt && q_idx && q_cnt))
    return fail(VSA_ERR_INVALID, "kv_idx, kv_cnt, q_idx and q_cnt must all be set or all be NULL");
  if (lists && max_kv < 1) return fail(VSA_ERR_INVALID, "max_kv must be >= 1");
  if (list_mode != 0 && list_mode != 1) return fail(VSA_ERR_INVALID, "list_mode must be 0 or 1");
  if (!isfinite(softmax_scale)) return fail(VSA_ERR_INVALID, "softmax_scale must be finite");
  if (dtype != VSA_F32 && dtype != VSA_BF16)
    return fail(VSA_ERR_UNSUPPORTED, "the backward pass takes VSA_F32 or VSA_BF16");
  if (L->C != 32 && L->C != 64) return fail(VSA_ERR_UNSUPPORTED, "attention needs 32- or 64-token tiles");
  if (L->d != 64 && L->d != 128) return fail(VSA_ERR_UNSUPPORTED, "attention needs head_dim 64 or 128");
  const long long work = (long long)L->B * L->heads * L->n_tiles;
  if (work > 0x7FFFFFFFll) return fail(VSA_ERR_UNSUPPORTED, "too many tiles for one launch");
  st = check_slice(*L, dtype);
  if (st != VSA_OK) return st;
  *a = vsa::BwdArgs{};
  a->q = q;
  a->k = k;
  a->v = v;
  a->out = out;
  a->dout = dout;
  a->lse = lse;
  a->kv_idx = kv_idx;
  a->kv_cnt = kv_cnt;
  a->max_kv = lists ? max_kv : L->n_tiles;
  a->q_idx = q_idx;
  a->q_cnt = q_cnt;
  a->list_mode = list_mode;
  a->scale = softmax_scale;
  a->scale_log2 = softmax_scale * 1.4426950408889634f;
  a->dq = dq;
  a->dk = dk;
  a->dv = dv;
  return VSA_OK;
}

vsa_status vsa_block_sparse_attn_bwd(const vsa_layout* layout, int32_t dtype, const void* q,
                                     const void* k, const void* v, const void* out,
                                     const void* dout, const float* lse, const int32_t* kv_idx,
                                     const int32_t* kv_cnt, int32_t max_kv, const int32_t* q_idx,
                                     const int32_t* q_cnt, int32_t list_mode, float softmax_scale,
                                     void* dq, void* dk, void* dv, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  vsa::DevLayout L;
  vsa::BwdArgs a;
  vsa_status st = bwd_args(layout, dtype, q, k, v, out, dout, lse, kv_idx, kv_cnt, max_kv, q_idx,
                           q_cnt, list_mode, softmax_scale, dq, dk, dv, &L, &a);
  if (st != VSA_OK) return st;
  const size_t need = vsa::attn_bwd_workspace_bytes(L);
  if (!workspace || workspace_bytes < need)
    return fail(VSA_ERR_WORKSPACE, "workspace of %zu bytes needed", need);
  if (reinterpret_cast<uintptr_t>(workspace) % 8 != 0)
    return fail(VSA_ERR_INVALID, "workspace must be 8-byte aligned");
  a.rowstat = static_cast<float2*>(workspace);
  return hip_status(vsa::launch_attn_bwd(L, dtype, a, static_cast<hipStream_t>(stream)),
                    "vsa_block_sparse_attn_bwd");
}

vsa_status vsa_block_sparse_attn_bwd_noalloc(const vsa_layout* layout, int32_t dtype, const void* q,
                                             const void* k, const void* v, const void* out,
                                             const void* dout, const float* lse,
                                             const int32_t* kv_idx, const int32_t* kv_cnt,
                                             int32_t max_kv, const int32_t* q_idx,
                                             const int32_t* q_cnt, int32_t list_mode,
                                             float softmax_scale, void* dq, void* dk, void* dv,
                                             void* stream) {
  vsa::DevLayout L;
  vsa::BwdArgs a;
  vsa_status st = bwd_args(layout, dtype, q, k, v, out, dout, lse, kv_idx, kv_cnt, max_kv, q_idx,
                           q_cnt, list_mode, softmax_scale, dq, dk, dv, &L, &a);
  if (st != VSA_OK) return st;
  const size_t need = vsa::attn_bwd_workspace_bytes(L);
  if (need > vsa::kBwdScratchBytes)
    return fail(VSA_ERR_UNSUPPORTED,
                "the row statistics need %zu bytes; the built-in scratch holds %zu "
                "(B * heads * n_padded <= %zu rows): call vsa_block_sparse_attn_bwd with a workspace",
                need, vsa::kBwdScratchBytes, vsa::kBwdScratchBytes / 8);
  void* ptr = nullptr;
  const hipError_t e = vsa::attn_bwd_scratch(&ptr);
  if (e != hipSuccess) return hip_status(e, "vsa_block_sparse_attn_bwd_noalloc: scratch address");
  a.rowstat = static_cast<float2*>(ptr);
  return hip_status(vsa::launch_attn_bwd(L, dtype, a, static_cast<hipStream_t>(stream)),
                    "vsa_block_sparse_attn_bwd_noalloc");
}

vsa_status vsa_block_sparse_attn_fwd_fp8_nat(const vsa_layout* layout, int32_t dtype, const void* q,
                                             const void* k, const void* v, const float* q_scale,
                                             const float* k_scale, const float* v_scale,
                                             const int32_t* kv_idx, const int32_t* kv_cnt,
                                             int32_t max_kv, int32_t list_mode,
                                             const int32_t* work_order, float softmax_scale,
                                             void* out, float* lse, void* stream) {
  vsa::DevLayout L;
  vsa_status st = derive(layout, &L, nullptr);
  if (st != VSA_OK) return st;
  if (dtype != VSA_FP8_E4M3 && dtype != VSA_FP8_E4M3_VOP)
    return fail(VSA_ERR_UNSUPPORTED, "vsa_block_sparse_attn_fwd_fp8_nat takes the fp8 dtypes");
  if (!q || !k || !v || !out) return fail(VSA_ERR_INVALID, "q, k, v and out must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(VSA_ERR_INVALID, "pointers must be 16-byte aligned");
  if (!q_scale || !k_scale || !v_scale) return fail(VSA_ERR_INVALID, "fp8 needs q_scale, k_scale and v_scale");
  if ((kv_idx == nullptr) != (kv_cnt == nullptr))
    return fail(VSA_ERR_INVALID, "kv_idx and kv_cnt must both be set or both be NULL");
  if (kv_idx && max_kv < 1) return fail(VSA_ERR_INVALID, "max_kv must be >= 1");
  if (list_mode < 0 || list_mode > 2) return fail(VSA_ERR_INVALID, "list_mode must be 0, 1 or 2");
  st = check_order(work_order, kv_idx, list_mode);
  if (st != VSA_OK) return st;
  if (!isfinite(softmax_scale)) return fail(VSA_ERR_INVALID, "softmax_scale must be finite");
  if (L.C != 64 || L.d != 128) return fail(VSA_ERR_UNSUPPORTED, "fp8 attention needs 64-token tiles and head_dim 128");
  const long long work = (long long)L.B * L.heads * L.n_tiles;
  if (work > 0x7FFFFFFFll) return fail(VSA_ERR_UNSUPPORTED, "too many query tiles for one launch");
  st = check_slice(L, dtype);
  if (st != VSA_OK) return st;
  vsa::AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.kv_idx = kv_idx;
  a.kv_cnt = kv_cnt;
  a.max_kv = kv_idx ? max_kv : L.n_tiles;
  a.list_mode = list_mode;
  a.work_order = work_order;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.out = out;
  a.lse = lse;
  a.natural_io = 1;
  return hip_status(vsa::launch_attn(L, dtype, a, static_cast<hipStream_t>(stream)),
                    "vsa_block_sparse_attn_fwd_fp8_nat");
}

vsa_status vsa_block_sparse_attn_fwd_nat(const vsa_layout* layout, int32_t dtype, const void* q,
                                         const void* k, const void* v, const int32_t* kv_idx,
                                         const int32_t* kv_cnt, int32_t max_kv, int32_t list_mode,
                                         const int32_t* work_order, float softmax_scale, void* out,
                                         float* lse, void* stream) {
  vsa::DevLayout L;
  vsa_status st = derive(layout, &L, nullptr);
  if (st != VSA_OK) return st;
  if (dtype != VSA_F32 && dtype != VSA_BF16 && dtype != VSA_BF16_VOP)
    return fail(VSA_ERR_UNSUPPORTED, "natural-order attention takes VSA_F32, VSA_BF16 or VSA_BF16_VOP");
  if (dtype == VSA_BF16_VOP && L.C != 64)
    return fail(VSA_ERR_UNSUPPORTED, "the bf16 V operand layout needs 64-token tiles");
  const long long es = dtype == VSA_F32 ? 4 : 2;
  if ((long long)L.n_tokens * L.heads * L.d * es > 0x7FFFFFFFll)
    return fail(VSA_ERR_UNSUPPORTED, "one batch of natural Q must stay below 2 GiB");
  if (!q || !k || !v || !out) return fail(VSA_ERR_INVALID, "q, k, v and out must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(VSA_ERR_INVALID, "pointers must be 16-byte aligned");
  if ((kv_idx == nullptr) != (kv_cnt == nullptr))
    return fail(VSA_ERR_INVALID, "kv_idx and kv_cnt must both be set or both be NULL");
  if (kv_idx && max_kv < 1) return fail(VSA_ERR_INVALID, "max_kv must be >= 1");
  if (list_mode < 0 || list_mode > 2) return fail(VSA_ERR_INVALID, "list_mode must be 0, 1 or 2");
  st = check_order(work_order, kv_idx, list_mode);
  if (st != VSA_OK) return st;
  if (!isfinite(softmax_scale)) return fail(VSA_ERR_INVALID, "softmax_scale must be finite");
  if (L.C != 32 && L.C != 64) return fail(VSA_ERR_UNSUPPORTED, "attention needs 32- or 64-token tiles");
  if (L.d != 64 && L.d != 128) return fail(VSA_ERR_UNSUPPORTED, "attention needs head_dim 64 or 128");
  const long long work = (long long)L.B * L.heads * L.n_tiles;
  if (work > 0x7FFFFFFFll) return fail(VSA_ERR_UNSUPPORTED, "too many query tiles for one launch");
  st = check_slice(L, dtype);
  if (st != VSA_OK) return st;
  vsa::AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.kv_idx = kv_idx;
  a.kv_cnt = kv_cnt;
  a.max_kv = kv_idx ? max_kv : L.n_tiles;
  a.list_mode = list_mode;
  a.work_order = work_order;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.out = out;
  a.lse = lse;
  a.natural_io = 1;
  return hip_status(vsa::launch_attn(L, dtype, a, static_cast<hipStream_t>(stream)),
                    "vsa_block_sparse_attn_fwd_nat");
}

const char* vsa_status_string(int32_t status) {
  switch (status) {
    case VSA_OK: return "VSA_OK";
    case VSA_ERR_INVALID: return "VSA_ERR_INVALID";
    case VSA_ERR_UNSUPPORTED: return "VSA_ERR_UNSUPPORTED";
    case VSA_ERR_WORKSPACE: return "VSA_ERR_WORKSPACE";
    case VSA_ERR_HIP: return "VSA_ERR_HIP";
    default: return "unknown status";
  }
}

const char* vsa_last_error(void) { return g_last_error.c_str(); }

const char* vsa_version(void) { return "0.1.0"; }

}  // extern "C"
