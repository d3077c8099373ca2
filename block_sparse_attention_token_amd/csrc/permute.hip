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

// Natural bf16 -> tiled V in the bf16 P.V operand layout (64-token tiles):
// the tile's rows of one head are gathered into LDS (pad rows as zeros), then
// written as two 32-token blocks, each channel-major with the block's tokens
// in the order the P.V product consumes them: position 16 ps + 8 h + i of a
// channel row holds token 16 ps + 8 (i / 4) + 4 h + i % 4 of the block.
// Output chunk q (16 bytes, 8 positions) of the tile is block q / (4 d),
// channel (q / 4) % d, positions 8 (q % 4) .. + 7: consecutive threads write
// consecutive chunks.
__global__ __launch_bounds__(kThreads) void permute_vop_kernel(DevLayout L, const uint4* __restrict__ src,
                                                               uint4* __restrict__ dst) {
  const int tile = blockIdx.x;
  const int head = blockIdx.y;
  const int b = blockIdx.z;
  const int chunks = L.d >> 3;                       // 16-byte chunks per bf16 row
  __shared__ uint4 rows[64 * 32];                    // the tile, token-major (d <= 256)
  for (int idx = threadIdx.x; idx < 64 * chunks; idx += kThreads) {
    const int r = idx / chunks;
    const int ch = idx - r * chunks;
    const int nat = natural_index(L, tile, r);
    rows[idx] = nat < 0 ? make_uint4(0u, 0u, 0u, 0u)
                        : src[(((long long)b * L.n_tokens + nat) * L.heads + head) * chunks + ch];
  }
  __syncthreads();
  const uint16_t* el = reinterpret_cast<const uint16_t*>(rows);
  const long long out0 = ((long long)(b * L.heads + head) * L.n_padded + (long long)tile * 64) * chunks;
  for (int q = threadIdx.x; q < 64 * chunks; q += kThreads) {
    const int kb = q / (4 * L.d);
    const int c = (q >> 2) - kb * L.d;
    const int p0 = 8 * (q & 3);
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t two = 0u;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int p = p0 + 2 * e + k;
        const int t = 16 * (p >> 4) + 8 * ((p >> 2) & 1) + 4 * ((p >> 3) & 1) + (p & 3);
        two |= (uint32_t)el[(32 * kb + t) * L.d + c] << (16 * k);
      }
      w[e] = two;
    }
    dst[out0 + q] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace

hipError_t launch_permute_vop(const DevLayout& L, const void* src, void* dst, hipStream_t s) {
  if (L.C != 64 || L.d % 8 || L.d > 256) return hipErrorInvalidValue;
  dim3 grid(L.n_tiles, L.heads, L.B);
  hipLaunchKernelGGL(permute_vop_kernel, grid, dim3(kThreads), 0, s, L, static_cast<const uint4*>(src),
                     static_cast<uint4*>(dst));
  return hipGetLastError();
}

hipError_t launch_permute(const DevLayout& L, int esize, const void* src, void* dst, int inverse,
                          hipStream_t s) {
  const int row_bytes = L.d * esize;
  dim3 grid(L.n_tiles, L.heads, L.B);
  hipLaunchKernelGGL(permute_kernel, grid, dim3(kThreads), 0, s, L, row_bytes,
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), inverse);
  return hipGetLastError();
}

}  // namespace vsa
