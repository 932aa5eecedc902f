// Wave- and block-level integer scans for 64-wide wavefronts (internal).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moonep {

__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = __lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o, 64));
  return x;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = __lane_id();
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// In-place exclusive scan of a[0..n) in LDS for any n, by chunks of blockDim.x;
// wsum needs blockDim.x/64 ints of LDS.  Returns the total.  All threads must call it.
__device__ __forceinline__ int block_excl_scan(int32_t* a, int n, int32_t* wsum) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, nw = blockDim.x >> 6;
  int carry = 0;
  for (int i0 = 0; i0 < n; i0 += blockDim.x) {
    const int i = i0 + t;
    const int v = i < n ? a[i] : 0;
    const int incl = wave_incl_scan(v);
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int woff = 0, tot = 0;
    for (int k = 0; k < nw; ++k) {
      if (k < w) woff += wsum[k];
      tot += wsum[k];
    }
    if (i < n) a[i] = carry + woff + incl - v;
    carry += tot;
    __syncthreads();
  }
  return carry;
}

// Stable compaction: writes, in ascending order, every i in [0, n) with pred(i) into out[];
// returns the count.  wsum needs blockDim.x/64 ints of LDS.  All threads must call it.
template <typename Pred>
__device__ __forceinline__ int block_compact(int n, Pred pred, int32_t* out, int32_t* wsum) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, nw = blockDim.x >> 6;
  int base = 0;
  for (int i0 = 0; i0 < n; i0 += blockDim.x) {
    const int i = i0 + t;
    const bool f = i < n && pred(i);
    const uint64_t m = __ballot(f);
    if (lane == 0) wsum[w] = __popcll(m);
    __syncthreads();
    int off = base, tot = 0;
    for (int k = 0; k < nw; ++k) {
      if (k < w) off += wsum[k];
      tot += wsum[k];
    }
    if (f) out[off + __popcll(m & lanemask_lt())] = i;
    base += tot;
    __syncthreads();
  }
  return base;
}

}  // namespace moonep
