// S5: per-tile fp8 e4m3 quantiser (FPSAttention, Approach: FP8 quantisation
// on the same 3D tiles as the block sparsity).
//
// Per (batch, head, tile): a = absmax over real rows and all channels,
// scale = fl32(a / 448), code = RNE_e4m3(fl32(x * fl32(448 / a))) saturating
// at +-448, sign taken from the fp32 sign bit. Every step is a correctly
// rounded fp32 operation, a round-to-nearest-even conversion or exact
// integer work, so codes are reproducible bit for bit.
#include <float.h>

#include "vsa_internal.h"

namespace vsa {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// OCP E4M3 encode of one fp32 value, round to nearest even, saturating.
__device__ __forceinline__ uint32_t e4m3_rne(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a > 0x7F800000u) {
    code = 0x7Fu;                                   // NaN
  } else if (a >= 0x43E00000u) {                    // |y| >= 448 (and inf): saturate
    code = 0x7Eu;
  } else if (a >= 0x3C800000u) {                    // |y| >= 2^-6: normal e4m3
    // keep exponent + 3 mantissa bits, round the 20 dropped bits to nearest even
    const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
    code = r - (120u << 3);                         // rebias 127 -> 7
  } else {                                          // subnormal: multiples of 2^-9
    const float m = rintf(__uint_as_float(a) * 512.0f);   // exact scaling, RNE to integer
    code = (uint32_t)m;                             // 0..8 (8 is the smallest normal)
  }
  return code | sign;
}

// Codes of the 8 bf16 values in ws (4 dwords, low half first) times inv,
// byte i of the result = value i. With a finite, non-zero tile absmax every
// |value * inv| is at most 448 (1 + 2^-23), inside the e4m3 range, and the
// matrix core's conversion (v_cvt_pk_fp8_f32, round to nearest even, sign
// kept) gives the same codes as e4m3_rne at one instruction per pair; a tile
// with an infinite or NaN absmax takes e4m3_rne for its saturation and NaN
// codes.
__device__ __forceinline__ uint2 encode8(const uint32_t (&ws)[4], float inv, bool hw) {
  if (hw) {
    int w0 = 0, w1 = 0;
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(__fmul_rn(bf16_lo(ws[0]), inv), __fmul_rn(bf16_hi(ws[0]), inv), w0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(__fmul_rn(bf16_lo(ws[1]), inv), __fmul_rn(bf16_hi(ws[1]), inv), w0, true);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(__fmul_rn(bf16_lo(ws[2]), inv), __fmul_rn(bf16_hi(ws[2]), inv), w1, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(__fmul_rn(bf16_lo(ws[3]), inv), __fmul_rn(bf16_hi(ws[3]), inv), w1, true);
    return make_uint2((uint32_t)w0, (uint32_t)w1);
  }
  uint32_t packed[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t c0 = e4m3_rne(__fmul_rn(bf16_lo(ws[e]), inv));
    const uint32_t c1 = e4m3_rne(__fmul_rn(bf16_hi(ws[e]), inv));
    packed[e >> 1] |= (c0 | (c1 << 8)) << ((e & 1) * 16);
  }
  return make_uint2(packed[0], packed[1]);
}

// VOP: 64-token tiles of d = 128 only. The tile's codes are gathered in LDS
// and written channel-major, each 64-byte channel row holding the tile's
// tokens in the order the fp8 P.V product takes them: position
// p = 32 h + 16 A + 4 B + r holds token t = 32 A + 8 B + 4 h + r
// (h, r in 0..1 and 0..3, A in 0..1, B in 0..3).
// PRESET: the tile's absmax a was written into scales[] by group_absmax_kernel
// (one a per group of tiles); the kernel reads it, then overwrites the entry
// with the scale, so each entry is touched by its own workgroup only.
template <bool VOP, bool PRESET>
__global__ __launch_bounds__(kThreads) void quant_kernel(DevLayout L, const uint4* __restrict__ x,
                                                         uint2* __restrict__ codes,
                                                         float* __restrict__ scales) {
  const int tile = blockIdx.x;
  const int head = blockIdx.y;
  const int b = blockIdx.z;
  const int chunks = L.d >> 3;                      // 8 bf16 per 16-byte chunk
  const int total = L.C * chunks;
  const long long row0 = (long long)(b * L.heads + head) * L.n_padded + (long long)tile * L.C;
  const TileValid tv = tile_valid(L, tile);

  __shared__ float red[kThreads / 64];
  float amax = 0.0f;
  for (int idx = threadIdx.x; !PRESET && idx < total; idx += kThreads) {
    const int r = idx / chunks;
    if (!row_is_real(L, tv, r)) continue;
    const uint4 w = x[(row0 + r) * chunks + (idx - r * chunks)];
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      amax = fmaxf(amax, fabsf(bf16_lo(ws[e])));
      amax = fmaxf(amax, fabsf(bf16_hi(ws[e])));
    }
  }
  // wavefront then workgroup max (max is order-independent, so exact)
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  float a = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) a = fmaxf(a, red[i]);
  if constexpr (PRESET) a = scales[(long long)(b * L.heads + head) * L.n_tiles + tile];
  __syncthreads();                                   // every thread has read the preset a

  const float inv = (a > 0.0f) ? __fdiv_rn(448.0f, a) : 0.0f;
  if (threadIdx.x == 0) {
    scales[(long long)(b * L.heads + head) * L.n_tiles + tile] =
        (a > 0.0f) ? __fdiv_rn(a, 448.0f) : 0.0f;
  }
  __shared__ uint2 tl[VOP ? 64 * 128 / 8 : 1];       // VOP: the tile's codes, token-major
  for (int idx = threadIdx.x; idx < total; idx += kThreads) {
    const int r = idx / chunks;
    const long long off = (row0 + r) * chunks + (idx - r * chunks);
    uint2 out = make_uint2(0u, 0u);
    if (a != 0.0f && row_is_real(L, tv, r)) {
      const uint4 w = x[off];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
      out = encode8(ws, inv, a <= FLT_MAX);
    }
    if constexpr (VOP) tl[idx] = out;
    else codes[off] = out;
  }
  if constexpr (VOP) {
    __syncthreads();
    const uint8_t* tb = reinterpret_cast<const uint8_t*>(tl);
    uint4* dst = reinterpret_cast<uint4*>(codes + row0 * chunks);
    // 16-byte piece q: channel q / 4, positions 16 (q % 4) .. +15
    for (int q = threadIdx.x; q < 128 * 4; q += kThreads) {
      const int c = q >> 2, p0 = 16 * (q & 3);
      uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int pp = p0 + e;
        const int h = pp >> 5, A = (pp >> 4) & 1, B = (pp >> 2) & 3, rr = pp & 3;
        const int t = 32 * A + 8 * B + 4 * h + rr;
        w[e >> 2] |= (uint32_t)tb[t * 128 + c] << (8 * (e & 3));
      }
      dst[q] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// The quantiser with the tile permute folded in (FVAttn summary: video-aware
// block organisation; FPSAttention, Approach: FP8 on the shared tiles): one
// workgroup per (batch, tile, head) gathers the tile's rows of one head from
// the natural order [B, T*H*W, heads, d] into registers, takes their absmax,
// and writes the codes to the tiled position (VOP: in the P.V operand
// layout) and the scale, exactly as quant_kernel does from the tiled copy.
// POOL: also the tile's fp32 mean over its real rows, with the rows of each
// thread and the order of the sums of the routing's pool pass, so the means
// are bit-identical to it. Thread t takes chunk t % chunks of rows
// t / chunks + groups * m (groups = 256 / chunks), at most kNatRows rows.
constexpr int kNatRows = 8;

// CT, DT: tile tokens and head_dim fixed at compile time (0: taken from L),
// so that the common 64-token, 128-channel tile runs without per-row tests.
template <bool VOP, bool POOL, int CT = 0, int DT = 0>
__global__ __launch_bounds__(kThreads) void quant_nat_kernel(DevLayout L, const uint4* __restrict__ x,
                                                             uint2* __restrict__ codes,
                                                             float* __restrict__ scales,
                                                             float* __restrict__ pooled) {
  const int tile = blockIdx.x;
  const int head = blockIdx.y;
  const int b = blockIdx.z;
  const int C = CT ? CT : L.C, d = DT ? DT : L.d;
  const int chunks = d >> 3;
  const int groups = kThreads / chunks;
  const int ch = threadIdx.x % chunks;
  const int rg = threadIdx.x / chunks;
  const long long bh = (long long)b * L.heads + head;
  const long long row0 = bh * L.n_padded + (long long)tile * C;
  // natural position of each row of the tile, found once per row
  __shared__ int nat_of[kThreads * kNatRows];           // C <= 8 * groups <= 2048 rows
  for (int r = threadIdx.x; r < C; r += kThreads) nat_of[r] = natural_index(L, tile, r);
  __syncthreads();
  uint4 xr[kNatRows];
  float amax = 0.0f;
#pragma unroll
  for (int m = 0; m < kNatRows; ++m) {
    const int r = rg + groups * m;
    xr[m] = make_uint4(0u, 0u, 0u, 0u);
    if (rg < groups && r < C) {
      const int nat = nat_of[r];
      if (nat >= 0) xr[m] = x[(((long long)b * L.n_tokens + nat) * L.heads + head) * chunks + ch];
    }
    const uint32_t ws[4] = {xr[m].x, xr[m].y, xr[m].z, xr[m].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      amax = fmaxf(amax, fabsf(bf16_lo(ws[e])));
      amax = fmaxf(amax, fabsf(bf16_hi(ws[e])));
    }
  }
  __shared__ float red[kThreads / 64];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  float a = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) a = fmaxf(a, red[i]);
  const float inv = (a > 0.0f) ? __fdiv_rn(448.0f, a) : 0.0f;
  if (threadIdx.x == 0) scales[bh * L.n_tiles + tile] = (a > 0.0f) ? __fdiv_rn(a, 448.0f) : 0.0f;

  __shared__ uint2 tl[VOP ? 64 * 128 / 8 : 1];       // VOP: the tile's codes, token-major
#pragma unroll
  for (int m = 0; m < kNatRows; ++m) {
    const int r = rg + groups * m;
    if (rg >= groups || r >= C) continue;
    uint2 out = make_uint2(0u, 0u);
    if (a != 0.0f) {
      const uint32_t ws[4] = {xr[m].x, xr[m].y, xr[m].z, xr[m].w};
      out = encode8(ws, inv, a <= FLT_MAX);
    }
    if constexpr (VOP) tl[r * chunks + ch] = out;
    else codes[(row0 + r) * chunks + ch] = out;
  }
  if constexpr (POOL) {
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int m = 0; m < kNatRows; ++m) {
      const int r = rg + groups * m;
      if (rg >= groups || r >= C || nat_of[r] < 0) continue;
      const uint32_t ws[4] = {xr[m].x, xr[m].y, xr[m].z, xr[m].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += __uint_as_float(ws[e] << 16);
        acc[2 * e + 1] += __uint_as_float(ws[e] & 0xFFFF0000u);
      }
    }
    __shared__ float part[kThreads * 8];
#pragma unroll
    for (int e = 0; e < 8; ++e) part[threadIdx.x * 8 + e] = acc[e];
    __syncthreads();
    const int n = real_rows(L, tile_valid(L, tile));
    for (int c = threadIdx.x; c < d; c += kThreads) {
      const int cch = c >> 3, ce = c & 7;
      float sum = 0.0f;
      for (int g = 0; g < groups; ++g) sum += part[(g * chunks + cch) * 8 + ce];
      pooled[(bh * L.n_tiles + tile) * d + c] = n > 0 ? sum / (float)n : 0.0f;
    }
  }
  if constexpr (VOP) {
    __syncthreads();
    const uint8_t* tb = reinterpret_cast<const uint8_t*>(tl);
    uint4* dst = reinterpret_cast<uint4*>(codes + row0 * chunks);
    for (int q = threadIdx.x; q < 128 * 4; q += kThreads) {
      const int c = q >> 2, p0 = 16 * (q & 3);
      uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int pp = p0 + e;
        const int h = pp >> 5, A = (pp >> 4) & 1, B = (pp >> 2) & 3, rr = pp & 3;
        const int t = 32 * A + 8 * B + 4 * h + rr;
        w[e >> 2] |= (uint32_t)tb[t * 128 + c] << (8 * (e & 3));
      }
      dst[q] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// One workgroup per (batch, head, group of gt x gh x gw tiles): the absmax
// over the real rows of every tile of the group, written to scales[] for
// each member tile (3D tiles only).
__global__ __launch_bounds__(kThreads) void group_absmax_kernel(DevLayout L, int gt, int gh, int gw,
                                                                const uint4* __restrict__ x,
                                                                float* __restrict__ scales) {
  const int ngh = (L.nth + gh - 1) / gh, ngw = (L.ntw + gw - 1) / gw;
  const int grp = blockIdx.x, head = blockIdx.y, b = blockIdx.z;
  const int A = grp / (ngh * ngw), Bg = (grp / ngw) % ngh, Cg = grp % ngw;
  const int a0 = A * gt, a1 = min(a0 + gt, L.ntt);
  const int b0 = Bg * gh, b1 = min(b0 + gh, L.nth);
  const int c0 = Cg * gw, c1 = min(c0 + gw, L.ntw);
  const int chunks = L.d >> 3;
  const int total = L.C * chunks;
  const long long bh = (long long)(b * L.heads + head);
  float amax = 0.0f;
  for (int ta = a0; ta < a1; ++ta)
    for (int tb = b0; tb < b1; ++tb)
      for (int tc = c0; tc < c1; ++tc) {
        const int tile = (ta * L.nth + tb) * L.ntw + tc;
        const TileValid tv = tile_valid(L, tile);
        const long long row0 = bh * L.n_padded + (long long)tile * L.C;
        for (int idx = threadIdx.x; idx < total; idx += kThreads) {
          const int r = idx / chunks;
          if (!row_is_real(L, tv, r)) continue;
          const uint4 w = x[(row0 + r) * chunks + (idx - r * chunks)];
          const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            amax = fmaxf(amax, fabsf(bf16_lo(ws[e])));
            amax = fmaxf(amax, fabsf(bf16_hi(ws[e])));
          }
        }
      }
  __shared__ float red[kThreads / 64];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  float a = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) a = fmaxf(a, red[i]);
  const int members = (a1 - a0) * (b1 - b0) * (c1 - c0);
  for (int m = threadIdx.x; m < members; m += kThreads) {
    const int nb = b1 - b0, nc = c1 - c0;
    const int ta = a0 + m / (nb * nc), tb = b0 + (m / nc) % nb, tc = c0 + m % nc;
    scales[bh * L.n_tiles + (ta * L.nth + tb) * L.ntw + tc] = a;
  }
}

}  // namespace

hipError_t launch_quant_fp8_grouped(const DevLayout& L, int gt, int gh, int gw, const void* x,
                                    uint8_t* codes, float* scales, bool v_operand, hipStream_t s) {
  const int ng = ((L.ntt + gt - 1) / gt) * ((L.nth + gh - 1) / gh) * ((L.ntw + gw - 1) / gw);
  hipLaunchKernelGGL(group_absmax_kernel, dim3(ng, L.heads, L.B), dim3(kThreads), 0, s, L, gt, gh, gw,
                     static_cast<const uint4*>(x), scales);
  dim3 grid(L.n_tiles, L.heads, L.B);
  if (v_operand) {
    if (L.C != 64 || L.d != 128) return hipErrorInvalidValue;
    hipLaunchKernelGGL((quant_kernel<true, true>), grid, dim3(kThreads), 0, s, L,
                       static_cast<const uint4*>(x), reinterpret_cast<uint2*>(codes), scales);
  } else {
    hipLaunchKernelGGL((quant_kernel<false, true>), grid, dim3(kThreads), 0, s, L,
                       static_cast<const uint4*>(x), reinterpret_cast<uint2*>(codes), scales);
  }
  return hipGetLastError();
}

hipError_t launch_quant_fp8(const DevLayout& L, const void* x, uint8_t* codes, float* scales,
                            bool v_operand, hipStream_t s) {
  dim3 grid(L.n_tiles, L.heads, L.B);
  if (v_operand) {
    if (L.C != 64 || L.d != 128) return hipErrorInvalidValue;
    hipLaunchKernelGGL((quant_kernel<true, false>), grid, dim3(kThreads), 0, s, L,
                       static_cast<const uint4*>(x), reinterpret_cast<uint2*>(codes), scales);
  } else {
    hipLaunchKernelGGL((quant_kernel<false, false>), grid, dim3(kThreads), 0, s, L,
                       static_cast<const uint4*>(x), reinterpret_cast<uint2*>(codes), scales);
  }
  return hipGetLastError();
}

hipError_t launch_quant_fp8_nat(const DevLayout& L, const void* x, uint8_t* codes, float* scales,
                                float* pooled, bool v_operand, hipStream_t s) {
  dim3 grid(L.n_tiles, L.heads, L.B);
  const uint4* xs = static_cast<const uint4*>(x);
  uint2* cs = reinterpret_cast<uint2*>(codes);
  const bool c64d128 = L.C == 64 && L.d == 128;
  if (v_operand) {
    if (!c64d128) return hipErrorInvalidValue;
    if (pooled) hipLaunchKernelGGL((quant_nat_kernel<true, true, 64, 128>), grid, dim3(kThreads), 0, s, L, xs, cs, scales, pooled);
    else hipLaunchKernelGGL((quant_nat_kernel<true, false, 64, 128>), grid, dim3(kThreads), 0, s, L, xs, cs, scales, pooled);
  } else if (c64d128) {
    if (pooled) hipLaunchKernelGGL((quant_nat_kernel<false, true, 64, 128>), grid, dim3(kThreads), 0, s, L, xs, cs, scales, pooled);
    else hipLaunchKernelGGL((quant_nat_kernel<false, false, 64, 128>), grid, dim3(kThreads), 0, s, L, xs, cs, scales, pooled);
  } else {
    if (pooled) hipLaunchKernelGGL((quant_nat_kernel<false, true>), grid, dim3(kThreads), 0, s, L, xs, cs, scales, pooled);
    else hipLaunchKernelGGL((quant_nat_kernel<false, false>), grid, dim3(kThreads), 0, s, L, xs, cs, scales, pooled);
  }
  return hipGetLastError();
}

}  // namespace vsa
