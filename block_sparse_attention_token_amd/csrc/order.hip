// Heavy-first work order for per-head (routed) key-tile lists. Top-p
// routing gives each head, and each query tile within a head, a list of its
// own length (FVAttn summary, Summary and Abstract: the per-head work under
// Top-p routing is uneven). The one-tile attention walks deal one query tile
// per workgroup; dealing them in index order leaves long walks that start
// late running alone at the end of the launch. This order deals the heads
// with the most (query tile, key tile) pairs first, and within a head the
// query tiles with the longest lists first, so the launch ends on short
// walks; a head's query tiles stay consecutive, which keeps the workgroups
// that read one head's K and V on the same XCDs.
//
// order[p] = bh * n_tiles + t lists every (b, head, query tile) once:
//   heads by total pairs, descending (equal totals: lower bh first);
//   within a head, by list length, descending (equal lengths: lower t first).
// The keys are max(cnt, 0) clamped to n_tiles, the lengths a walk can have.
// kOrderSplit workgroups per (b, head), each ranking one slice of the head's
// query tiles; each also sums every head's pairs, so a single launch needs no
// scratch memory. Integer sums and ranks: the result
// does not depend on the order of any operation.
#include "vsa_internal.h"

namespace vsa {
namespace {

constexpr int kOrderThreads = 1024;
constexpr int kOrderSplit = 8;

__device__ __forceinline__ int order_key(int c, int n) { return min(max(c, 0), n); }

__global__ __launch_bounds__(kOrderThreads) void work_order_kernel(const int32_t* __restrict__ cnt,
                                                                   int n, int n4, int lh,
                                                                   int32_t* __restrict__ order) {
  extern __shared__ int4 order_sh[];
  int* key = reinterpret_cast<int*>(order_sh);   // n4 entries: this head's keys, -1 past n
  int* tot = key + n4;                           // lh entries: pairs per head
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int per = (n + kOrderSplit - 1) / kOrderSplit;
  const int i0 = blockIdx.y * per, i1 = min(n, i0 + per);
  for (int i = tid; i < n4; i += kOrderThreads) key[i] = i < n ? order_key(cnt[(long long)bh * n + i], n) : -1;
  // pairs of every head: wave w sums heads w, w + 16, ..., a strided partial
  // per lane, then a shuffle reduction (integer sums: any order is exact)
  for (int h = tid >> 6; h < lh; h += kOrderThreads / 64) {
    const int32_t* row = cnt + (long long)h * n;
    int part = 0;
    for (int i = lane; i < n; i += 64) part += order_key(row[i], n);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
    if (lane == 0) tot[h] = part;
  }
  __syncthreads();
  // rank of this head among all heads (every thread computes it; lh is small)
  const int mine = tot[bh];
  int hr = 0;
  for (int h = 0; h < lh; ++h) hr += (tot[h] > mine) | ((tot[h] == mine) & (h < bh));
  // rank of each query tile within the head: one wave per tile, its lanes
  // comparing against interleaved groups of four keys, then a shuffle sum
  const int4* k4 = reinterpret_cast<const int4*>(key);
  for (int i = i0 + (tid >> 6); i < i1; i += kOrderThreads / 64) {
    const int ki = key[i];
    int r = 0;
    for (int j4 = lane; j4 < n4 / 4; j4 += 64) {
      const int4 kj = k4[j4];
      const int j = 4 * j4;
      r += (kj.x > ki) | ((kj.x == ki) & (j < i));
      r += (kj.y > ki) | ((kj.y == ki) & (j + 1 < i));
      r += (kj.z > ki) | ((kj.z == ki) & (j + 2 < i));
      r += (kj.w > ki) | ((kj.w == ki) & (j + 3 < i));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) r += __shfl_xor(r, off);
    if (lane == 0) order[(long long)hr * n + r] = bh * n + i;
  }
}

}  // namespace

size_t work_order_lds_bytes(const DevLayout& L) {
  const long long n4 = (L.n_tiles + 3) / 4 * 4;
  return (size_t)(n4 + (long long)L.B * L.heads) * sizeof(int);
}

hipError_t launch_work_order(const DevLayout& L, const int32_t* kv_cnt, int32_t* order, hipStream_t s) {
  const int lh = L.B * L.heads, n4 = (L.n_tiles + 3) / 4 * 4;
  hipLaunchKernelGGL(work_order_kernel, dim3(lh, kOrderSplit), dim3(kOrderThreads), work_order_lds_bytes(L), s,
                     kv_cnt, L.n_tiles, n4, lh, order);
  return hipGetLastError();
}

}  // namespace vsa
