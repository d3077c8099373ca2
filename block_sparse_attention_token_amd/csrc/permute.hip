// S1 / S7: natural <-> tiled token permutation (FPSAttention, Approach: one
// shared 3D tile granularity; FVAttn summary: video-aware block organisation;
// OSP-Next card, Model Summary: Skiparse groups along H and W).
//
// One workgroup moves one (batch, tile, head): tile_tokens rows of
// d * esize bytes. Consecutive threads move consecutive 16-byte chunks of a
// row, so both the natural-order side (rows of heads*d elements per token)
// and the tiled side (rows of d elements per (head, token)) are read and
// written in contiguous runs of d * esize bytes.
#include "vsa_internal.h"

namespace vsa {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void permute_kernel(DevLayout L, int row_bytes,
                                                           const uint4* __restrict__ src,
                                                           uint4* __restrict__ dst, int inverse) {
  const int tile = blockIdx.x;
  const int head = blockIdx.y;
  const int b = blockIdx.z;
  const int chunks = row_bytes >> 4;                 // 16-byte chunks per row
  const int total = L.C * chunks;
  const long long tiled_row0 =
      ((long long)(b * L.heads + head) * L.n_padded + (long long)tile * L.C);
  for (int idx = threadIdx.x; idx < total; idx += kThreads) {
    const int r = idx / chunks;
    const int ch = idx - r * chunks;
    const int nat = natural_index(L, tile, r);
    const long long t_off = (tiled_row0 + r) * chunks + ch;
    if (nat < 0) {
      if (!inverse) dst[t_off] = make_uint4(0u, 0u, 0u, 0u);
      continue;
    }
    const long long n_off = (((long long)b * L.n_tokens + nat) * L.heads + head) * chunks + ch;
    if (!inverse) {
      dst[t_off] = src[n_off];
    } else {
      dst[n_off] = src[t_off];
    }
  }
}

}  // namespace

hipError_t launch_permute(const DevLayout& L, int esize, const void* src, void* dst, int inverse,
                          hipStream_t s) {
  const int row_bytes = L.d * esize;
  dim3 grid(L.n_tiles, L.heads, L.B);
  hipLaunchKernelGGL(permute_kernel, grid, dim3(kThreads), 0, s, L, row_bytes,
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), inverse);
  return hipGetLastError();
}

}  // namespace vsa
