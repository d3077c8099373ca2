// S2: fixed block masks as ascending key-tile lists, one per query tile.
// FPSAttention, Approach and window ablation: a sliding window over 3D tiles.
// OSP-Next card, Model Summary: Skiparse-2D (a query sees its residue group)
// mixed with full-attention layers (dense lists).
#include "vsa_internal.h"

namespace vsa {
namespace {

__global__ __launch_bounds__(256) void mask_window_kernel(DevLayout L, int rt, int rh, int rw,
                                                          int max_kv, int32_t* __restrict__ kv_idx,
                                                          int32_t* __restrict__ kv_cnt) {
  const int qt = blockIdx.x * blockDim.x + threadIdx.x;
  if (qt >= L.n_tiles) return;
  int32_t* row = kv_idx + (long long)qt * max_kv;
  int n = 0;
  if (rt < 0 || rh < 0 || rw < 0) {                      // dense
    for (int j = 0; j < L.n_tiles; ++j) row[n++] = j;
  } else if (L.kind == 1) {                               // own residue group
    const int g0 = (qt / L.tiles_per_group) * L.tiles_per_group;
    for (int j = 0; j < L.tiles_per_group; ++j) row[n++] = g0 + j;
  } else {                                                // clipped 3D window
    const int per_a = L.nth * L.ntw;
    const int a = qt / per_a;
    const int b = (qt - a * per_a) / L.ntw;
    const int c = qt - a * per_a - b * L.ntw;
    const int a0 = max(a - rt, 0), a1 = min(a + rt, L.ntt - 1);
    const int b0 = max(b - rh, 0), b1 = min(b + rh, L.nth - 1);
    const int c0 = max(c - rw, 0), c1 = min(c + rw, L.ntw - 1);
    // row-major over (a, b, c) is ascending tile index
    for (int x = a0; x <= a1; ++x)
      for (int y = b0; y <= b1; ++y)
        for (int z = c0; z <= c1; ++z) row[n++] = (x * L.nth + y) * L.ntw + z;
  }
  kv_cnt[qt] = n;
}

// Tiles [lo, hi] along one axis of n tiles covered by the window of extent e
// (in groups of g tiles) around tile x's group: groups X - (e-1)/2 ..
// X - (e-1)/2 + e - 1, clipped at the grid edge.
__device__ __forceinline__ void group_window(int x, int g, int e, int n, int& lo, int& hi) {
  const int ng = (n + g - 1) / g;
  const int X = x / g;
  const int glo = max(X - (e - 1) / 2, 0);
  const int ghi = min(X - (e - 1) / 2 + e - 1, ng - 1);
  lo = glo * g;
  hi = min((ghi + 1) * g, n) - 1;
}

// Big tiles as groups of (gt, gh, gw) layout tiles (FPSAttention, Approach
// and ablation table: (6,8,8) tiles, windows such as (6,6,1)): a query tile
// lists every tile of every group inside the window of its own group.
__global__ __launch_bounds__(256) void mask_window_grouped_kernel(
    DevLayout L, int gt, int gh, int gw, int et, int eh, int ew, int max_kv,
    int32_t* __restrict__ kv_idx, int32_t* __restrict__ kv_cnt) {
  const int qt = blockIdx.x * blockDim.x + threadIdx.x;
  if (qt >= L.n_tiles) return;
  int32_t* row = kv_idx + (long long)qt * max_kv;
  const int per_a = L.nth * L.ntw;
  const int a = qt / per_a;
  const int b = (qt - a * per_a) / L.ntw;
  const int c = qt - a * per_a - b * L.ntw;
  int a0, a1, b0, b1, c0, c1;
  group_window(a, gt, et, L.ntt, a0, a1);
  group_window(b, gh, eh, L.nth, b0, b1);
  group_window(c, gw, ew, L.ntw, c0, c1);
  int n = 0;
  for (int x = a0; x <= a1; ++x)
    for (int y = b0; y <= b1; ++y)
      for (int z = c0; z <= c1; ++z) row[n++] = (x * L.nth + y) * L.ntw + z;
  kv_cnt[qt] = n;
}

}  // namespace

hipError_t launch_mask_window_grouped(const DevLayout& L, int gt, int gh, int gw, int et, int eh,
                                      int ew, int max_kv, int32_t* kv_idx, int32_t* kv_cnt,
                                      hipStream_t s) {
  const int threads = 256;
  dim3 grid((L.n_tiles + threads - 1) / threads);
  hipLaunchKernelGGL(mask_window_grouped_kernel, grid, dim3(threads), 0, s, L, gt, gh, gw, et, eh, ew,
                     max_kv, kv_idx, kv_cnt);
  return hipGetLastError();
}

hipError_t launch_mask_window(const DevLayout& L, int rt, int rh, int rw, int max_kv,
                              int32_t* kv_idx, int32_t* kv_cnt, hipStream_t s) {
  const int threads = 256;
  dim3 grid((L.n_tiles + threads - 1) / threads);
  hipLaunchKernelGGL(mask_window_kernel, grid, dim3(threads), 0, s, L, rt, rh, rw, max_kv, kv_idx,
                     kv_cnt);
  return hipGetLastError();
}

}  // namespace vsa
