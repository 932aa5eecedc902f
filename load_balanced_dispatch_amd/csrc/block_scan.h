// Wave- and block-level integer scans for 64-wide wavefronts (internal).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moonep {

// Inclusive scan across the 64 lanes with DPP moves (no LDS round trips): shifts by 1, 2, 4, 8 inside
// each row of 16 lanes, then row 0's total into rows 1 and 3 (row_bcast:15) and rows 0-1's total into
// rows 2 and 3 (row_bcast:31).  A lane whose source is outside its row, or whose row the mask leaves
// out, adds the `old` operand, 0.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
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

// In-place exclusive scans of up to three LDS arrays together (a[0..na), b[0..nb), c[0..nc); an
// array of length 0 is skipped), sharing the barriers of one pass; wsum needs 3 * blockDim.x/64 ints.
// The totals go to tot[0..2].  All threads must call it.
__device__ __forceinline__ void block_excl_scan3(int32_t* a, int na, int32_t* b, int nb, int32_t* c, int nc,
                                                 int32_t* wsum, int* tot) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, nw = blockDim.x >> 6;
  int32_t* arr[3] = {a, b, c};
  const int len[3] = {na, nb, nc};
  int carry[3] = {0, 0, 0};
  const int n = max(na, max(nb, nc));
  for (int i0 = 0; i0 < n; i0 += blockDim.x) {
    const int i = i0 + t;
    int v[3], incl[3];
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      v[q] = i < len[q] ? arr[q][i] : 0;
      incl[q] = wave_incl_scan(v[q]);
      if (lane == 63) wsum[q * nw + w] = incl[q];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      int woff = 0, all = 0;
      for (int k = 0; k < nw; ++k) {
        const int x = wsum[q * nw + k];
        woff += k < w ? x : 0;
        all += x;
      }
      if (i < len[q]) arr[q][i] = carry[q] + woff + incl[q] - v[q];
      carry[q] += all;
    }
    __syncthreads();
  }
#pragma unroll
  for (int q = 0; q < 3; ++q) tot[q] = carry[q];
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
