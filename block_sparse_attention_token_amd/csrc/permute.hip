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
// each 32-token block kb of a tile is stored channel-major, position
// 16 A + 8 h + i of a channel row holding token 16 A + 8 (i / 4) + 4 h + i % 4
// of the block. Output chunk (kb, channel c, part) is 16 bytes: positions
// 8 part .. +7 of channel c, i.e. tokens 32 kb + 16 A + 8 (i / 4) + 4 h + i % 4
// (part = 2 A + h, i = 0..7). One thread takes such an octet of tokens for 8
// channels: 8 16-byte loads (pad tokens read as zeros), an 8 x 8 transpose of
// 16-bit values with byte permutes, 8 16-byte stores. Lanes with consecutive
// channel groups read consecutive 16 bytes of a token row; the four parts of
// one channel are adjacent lanes' stores (64 contiguous bytes).
__global__ __launch_bounds__(kThreads) void permute_vop_kernel(DevLayout L, const uint4* __restrict__ src,
                                                               uint4* __restrict__ dst) {
  const int tile = blockIdx.x;
  const int head = blockIdx.y;
  const int b = blockIdx.z;
  const int chunks = L.d >> 3;                       // 16-byte chunks per bf16 row = channel groups
  const long long out0 = ((long long)(b * L.heads + head) * L.n_padded + (long long)tile * 64) * chunks;
  for (int item = threadIdx.x; item < 8 * chunks; item += blockDim.x) {
    const int part = (item / chunks) & 3, kb = item / (4 * chunks), cg = item % chunks;
    const int t0 = 32 * kb + 16 * (part >> 1) + 4 * (part & 1);
    uint4 x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int nat = natural_index(L, tile, t0 + 8 * (i >> 2) + (i & 3));
      x[i] = nat < 0 ? make_uint4(0u, 0u, 0u, 0u)
                     : src[(((long long)b * L.n_tokens + nat) * L.heads + head) * chunks + cg];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // channel 8 cg + j: half j % 2 of word j / 2 of every token; positions
      // 2 k, 2 k + 1 are tokens x[2 k], x[2 k + 1]
      const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t lo = (&x[2 * k].x)[j >> 1], hi = (&x[2 * k + 1].x)[j >> 1];
        w[k] = __builtin_amdgcn_perm(hi, lo, sel);
      }
      dst[out0 + ((long long)(kb * L.d + 8 * cg + j) << 2) + part] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

}  // namespace

hipError_t launch_permute_vop(const DevLayout& L, const void* src, void* dst, hipStream_t s) {
  if (L.C != 64 || L.d % 8 || L.d > 256) return hipErrorInvalidValue;
  dim3 grid(L.n_tiles, L.heads, L.B);
  const int threads = min(kThreads, (L.d + 63) / 64 * 64);     // one thread per (token octet, channel group)
  hipLaunchKernelGGL(permute_vop_kernel, grid, dim3(threads), 0, s, L, static_cast<const uint4*>(src),
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
