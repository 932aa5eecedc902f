// Row-moving kernels of the balanced MoE layer on gfx950: dispatch, prefetch, combine, reduce_grad.
//
// All four are HBM-bound streams of 16-byte vectors ([P2] = "Moonshot open-sources
// MoonEP: an expert-parallel communication library for MoE training",
// umios.umi6.com, sections "Core technique" and "Memory contract and weight
// layout"):
//   dispatch    one wave per 64-element piece of a token's row: read once into
//               registers, stored K times (fused permute into the expert-grouped buffer).
//   prefetch    persistent blocks copy every used slot's [H,Hp] expert matrix, one item ahead.
//   combine     one thread per 16 bytes of input row: K gathers issued together
//               (non-temporal: Yp is read once), fp32 FMA in k order.
//   reduce_grad persistent blocks fold each expert's slot gradients (ranks in
//               ascending order, a batch of slots loaded at once) into the home
//               gradient and zero the slots.
#include "block_scan.h"
#include "moonep_common.h"

namespace moonep {
namespace {

// ------------------------------------------------------------------ dispatch

constexpr int kDispatchThreads = 256;
// Dispatch outputs up to this size use ordinary stores, larger ones non-temporal stores.  Measured
// on 4 KB and 14 KB rows: ordinary stores were 10% faster for a 0.8 GB output and 3% for 3.8 GB,
// non-temporal ones 4% faster for 7.5 GB (the last-level cache holds 256 MB).
constexpr int64_t kStreamStoreBytes = int64_t(4) << 30;

// One wave per 64-element piece of a token's row (1 KB with 16-byte elements): each lane reads its
// element once and stores it K times.  Many short waves keep more rows in flight than one wave
// walking a whole row, which measured ~9% faster on the 4 KB rows of the mid workload.  NT selects
// non-temporal stores, for outputs far larger than the caches (see kStreamStoreBytes); issuing a
// token's K stores back to back (destinations read first) measured no faster than this loop.
template <typename V, bool NT>
__global__ __launch_bounds__(kDispatchThreads) void dispatch_rows(const V* __restrict__ X,
                                                                  const int32_t* __restrict__ dest,
                                                                  V* __restrict__ Xp, int64_t tokens, int K,
                                                                  int nvec, int pieces) {
  const int64_t g = (int64_t)blockIdx.x * (kDispatchThreads / 64) + (threadIdx.x >> 6);
  const int64_t tok = g / pieces;
  const int v = (int)(g % pieces) * 64 + (threadIdx.x & 63);
  if (tok >= tokens || v >= nvec) return;
  const V x = X[tok * nvec + v];
  const int32_t* dk = dest + tok * K;
  for (int k = 0; k < K; ++k) {
    const int32_t d = dk[k];
    if (d < 0) continue;
    if (NT) __builtin_nontemporal_store(x, Xp + (int64_t)d * nvec + v);
    else Xp[(int64_t)d * nvec + v] = x;
  }
}

// ------------------------------------------------------------------ prefetch

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;
constexpr int kCopyBlocksPerCU = 8;  // measured: 8 beat 16 by 5% on the large workload (equal on mid); 4 and 64 slower
constexpr int kMaxSlots = 32768;

// Persistent copy of every used slot, in items of kCopyThreads * kCopyUnroll vectors.  The loads of
// a block's next item are issued before the stores of its current one: on gfx950 one counter
// (vmcnt) tracks loads and stores in issue order, so a wait for loads issued after a store also
// waits for that store to complete; loading one item ahead keeps the stores off that wait.  In the
// whole step this took the large workload's prefetch from 101 / 109 / 121 / 153 us to
// 98 / 108 / 120 / 147 us at maxvio 0.5 / 1 / 2 / 4 and the mid one's from 22.1 to 17.8 us at
// maxvio 0.  Non-temporal slot stores were no faster in the step, and non-temporal loads slower.
template <typename V>
__global__ __launch_bounds__(kCopyThreads) void prefetch_slots(const V* __restrict__ W_home,
                                                               const int32_t* __restrict__ slot_expert,
                                                               V* __restrict__ W_slots, int RB, int E,
                                                               int64_t nvec) {
  extern __shared__ int32_t used[];  // [RB] used slots, ascending
  __shared__ int32_t wsum[kCopyThreads / 64];
  const int n = block_compact(
      RB, [&](int s) {
        const int e = slot_expert[s];
        return e >= 0 && e < E;
      },
      used, wsum);
  const int64_t per_item = (int64_t)kCopyThreads * kCopyUnroll;
  const int64_t chunks = (nvec + per_item - 1) / per_item;
  const int64_t items = (int64_t)n * chunks;
  auto load = [&](int64_t it, V* r) {
    const int s = used[it / chunks];
    const V* src = W_home + (int64_t)slot_expert[s] * nvec;
    const int64_t v0 = (it % chunks) * per_item + threadIdx.x;
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
      if (v0 + u * kCopyThreads < nvec) r[u] = src[v0 + u * kCopyThreads];
  };
  auto store = [&](int64_t it, const V* r) {
    V* dst = W_slots + (int64_t)used[it / chunks] * nvec;
    const int64_t v0 = (it % chunks) * per_item + threadIdx.x;
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
      if (v0 + u * kCopyThreads < nvec) dst[v0 + u * kCopyThreads] = r[u];
  };
  // two register buffers, alternating, so that the indices into them stay compile-time constants
  V a[kCopyUnroll], b[kCopyUnroll];
  int64_t it = blockIdx.x;
  if (it < items) load(it, a);
  while (it < items) {
    int64_t nx = it + gridDim.x;
    if (nx < items) load(nx, b);
    store(it, a);
    it = nx;
    if (it >= items) break;
    nx = it + gridDim.x;
    if (nx < items) load(nx, a);
    store(it, b);
    it = nx;
  }
}

// ------------------------------------------------------------------ combine

template <int VEC>
struct InVec;
template <>
struct InVec<8> {  // 8 bf16
  static __device__ __forceinline__ void load(const void* p, float* f) {
    const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(q[i] << 16);
      f[2 * i + 1] = __uint_as_float(q[i] & 0xffff0000u);
    }
  }
};
template <>
struct InVec<4> {  // 4 f32
  static __device__ __forceinline__ void load(const void* p, float* f) {
    const f32x4 q = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = q[i];
  }
};

constexpr int kCombineThreads = 256;
constexpr int kBatch = 8;  // gathers a combine thread keeps in flight

// VEC elements of 16 bytes per thread; ESZ = element bytes of Yp.  With GATED false every gate is 1
// and gates is not read (the gradient of dispatch: dX[r,s] = sum_k dXp[dest]); fma(1, y, acc)
// rounds as y + acc.  The gathers of a batch of k are all issued before the first is used, so a
// thread keeps up to kBatch 16-byte loads in flight; they are summed in ascending k as before.  A
// dropped pair (dest < 0) loads row 0 and is discarded by a select rather than a branch, which
// would make the compiler wait for each gather in turn.  IDX is the index type of the thread's item
// (32 bits when tokens * D / VEC fits); KC > 0 fixes K at compile time (KC = 0: K from the call).
template <int VEC, int ESZ, bool GATED, typename IDX, int KC>
__global__ __launch_bounds__(kCombineThreads) void combine_vec(const char* __restrict__ Yp,
                                                               const int32_t* __restrict__ dest,
                                                               const float* __restrict__ gates,
                                                               float* __restrict__ out, int64_t tokens, int K_arg,
                                                               int D) {
  const int K = KC > 0 ? KC : K_arg;
  const int nchunk = D / VEC;
  const IDX item = (IDX)blockIdx.x * kCombineThreads + threadIdx.x;
  if ((int64_t)item >= tokens * nchunk) return;
  const IDX tq = item / (IDX)nchunk;
  const int c = (int)(item - tq * (IDX)nchunk);
  const int64_t tok = (int64_t)tq;
  const int32_t* dk = dest + tok * K;
  const float* gk = GATED ? gates + tok * K : nullptr;
  float acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
  for (int k0 = 0; k0 < K; k0 += kBatch) {
    int32_t d[kBatch];
    float g[kBatch], y[kBatch][VEC];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      d[u] = k0 + u < K ? dk[k0 + u] : -1;
      g[u] = GATED && k0 + u < K ? gk[k0 + u] : 1.f;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (k0 + u < K) InVec<VEC>::load(Yp + ((int64_t)max(d[u], 0) * D + (int64_t)c * VEC) * ESZ, y[u]);
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (k0 + u < K) {
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          const float f = __builtin_fmaf(g[u], y[u][i], acc[i]);
          acc[i] = d[u] >= 0 ? f : acc[i];
        }
      }
  }
  f32x4* o = reinterpret_cast<f32x4*>(out + tok * D + (int64_t)c * VEC);
#pragma unroll
  for (int i = 0; i < VEC / 4; ++i) {
    const f32x4 q = {acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]};
    if (GATED) o[i] = q;
    else __builtin_nontemporal_store(q, o + i);
  }
}

// Scalar fallback for widths that are not a multiple of 16 bytes.
template <typename T, bool GATED>
__global__ __launch_bounds__(kCombineThreads) void combine_scalar(const T* __restrict__ Yp,
                                                                  const int32_t* __restrict__ dest,
                                                                  const float* __restrict__ gates,
                                                                  float* __restrict__ out, int64_t tokens, int K,
                                                                  int D) {
  const int64_t item = (int64_t)blockIdx.x * kCombineThreads + threadIdx.x;
  if (item >= tokens * D) return;
  const int64_t tok = item / D;
  const int c = (int)(item % D);
  float acc = 0.f;
  for (int k = 0; k < K; ++k) {
    const int32_t d = dest[tok * K + k];
    if (d < 0) continue;
    float y;
    if constexpr (sizeof(T) == 2)
      y = bf16_to_f32(reinterpret_cast<const uint16_t*>(Yp)[(int64_t)d * D + c]);
    else
      y = reinterpret_cast<const float*>(Yp)[(int64_t)d * D + c];
    acc = __builtin_fmaf(GATED ? gates[tok * K + k] : 1.f, y, acc);
  }
  out[tok * D + c] = acc;
}

// ------------------------------------------------------------------ combine backward

__device__ __forceinline__ float wave_sum_f(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

template <int ESZ>
__device__ __forceinline__ void store_scaled(char* p, float g, const float* o);
template <>
__device__ __forceinline__ void store_scaled<2>(char* p, float g, const float* o) {  // 8 bf16, rounded to nearest even
  u32x4 q;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    q[i] = (uint32_t)f32_to_bf16(g * o[2 * i]) | ((uint32_t)f32_to_bf16(g * o[2 * i + 1]) << 16);
  *reinterpret_cast<u32x4*>(p) = q;
}
template <>
__device__ __forceinline__ void store_scaled<4>(char* p, float g, const float* o) {  // 4 f32
  *reinterpret_cast<f32x4*>(p) = f32x4{g * o[0], g * o[1], g * o[2], g * o[3]};
}

// One wave per token; lane c handles 16-byte chunks c, c+64, ... of the Yp row (VEC elements of
// ESZ bytes).  The lane's part of the dout row is read once into registers (CPL chunks at most;
// CPL = 0: rows too wide for that, read again for every k).  For each k in ascending order:
// dYp[dest] = gate * dout (rounded to Yp's type), and dgate = <dout, Yp[dest]> as a float32 FMA
// chain per lane followed by a fixed butterfly across the wave, so the result does not depend on
// timing.
template <int VEC, int ESZ, int CPL>
__global__ __launch_bounds__(256) void combine_bwd_vec(const float* __restrict__ dout, const char* __restrict__ Yp,
                                                       const int32_t* __restrict__ dest,
                                                       const float* __restrict__ gates, char* __restrict__ dYp,
                                                       float* __restrict__ dgates, int64_t tokens, int K, int D) {
  const int lane = threadIdx.x & 63;
  const int64_t tok = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tok >= tokens) return;
  const int nchunk = D / VEC;
  const float* drow = dout + tok * D;
  auto load_dout = [&](int c, float (&o)[VEC]) {
#pragma unroll
    for (int h = 0; h < VEC / 4; ++h) {
      const f32x4 q = *reinterpret_cast<const f32x4*>(drow + c * VEC + 4 * h);
      o[4 * h] = q[0];
      o[4 * h + 1] = q[1];
      o[4 * h + 2] = q[2];
      o[4 * h + 3] = q[3];
    }
  };
  constexpr int NR = CPL > 0 ? CPL : 1;
  float o_reg[NR][VEC];
  if constexpr (CPL > 0) {
#pragma unroll
    for (int i = 0; i < CPL; ++i)
      if (lane + 64 * i < nchunk) load_dout(lane + 64 * i, o_reg[i]);
  }
  for (int k = 0; k < K; ++k) {
    const int32_t d = dest[tok * K + k];
    const float g = gates[tok * K + k];
    float part = 0.f;
    if (d >= 0) {
      auto chunk = [&](int c, const float (&o)[VEC]) {
        float y[VEC];
        const int64_t at = ((int64_t)d * D + (int64_t)c * VEC) * ESZ;
        InVec<VEC>::load(Yp + at, y);
#pragma unroll
        for (int i = 0; i < VEC; ++i) part = __builtin_fmaf(o[i], y[i], part);
        store_scaled<ESZ>(dYp + at, g, o);
      };
      if constexpr (CPL > 0) {
#pragma unroll
        for (int i = 0; i < CPL; ++i)
          if (lane + 64 * i < nchunk) chunk(lane + 64 * i, o_reg[i]);
      } else {
        for (int c = lane; c < nchunk; c += 64) {
          float o[VEC];
          load_dout(c, o);
          chunk(c, o);
        }
      }
    }
    part = wave_sum_f(part);
    if (lane == 0) dgates[tok * K + k] = part;
  }
}

// Scalar fallback (rows that are not a whole number of 16-byte chunks): same order of work.
template <typename T>
__global__ __launch_bounds__(256) void combine_bwd_scalar(const float* __restrict__ dout, const T* __restrict__ Yp,
                                                          const int32_t* __restrict__ dest,
                                                          const float* __restrict__ gates, T* __restrict__ dYp,
                                                          float* __restrict__ dgates, int64_t tokens, int K, int D) {
  const int lane = threadIdx.x & 63;
  const int64_t tok = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tok >= tokens) return;
  const float* drow = dout + tok * D;
  for (int k = 0; k < K; ++k) {
    const int32_t d = dest[tok * K + k];
    const float g = gates[tok * K + k];
    float part = 0.f;
    if (d >= 0) {
      for (int c = lane; c < D; c += 64) {
        const float o = drow[c];
        const int64_t at = (int64_t)d * D + c;
        float y;
        if constexpr (sizeof(T) == 2) {
          y = bf16_to_f32(Yp[at]);
          dYp[at] = f32_to_bf16(g * o);
        } else {
          y = Yp[at];
          dYp[at] = g * o;
        }
        part = __builtin_fmaf(o, y, part);
      }
    }
    part = wave_sum_f(part);
    if (lane == 0) dgates[tok * K + k] = part;
  }
}

// ------------------------------------------------------------------ reduce_grad

constexpr int kReduceThreads = 256;
// Measured in the whole step (bitwise-identical results): 2 vectors per thread, slots in batches
// of 4 and 4 blocks per CU took the mid workload's reduce_grad from 54.6 / 51.4 / 73.9 us to
// 48.9 / 46.6 / 63.3 us at maxvio 0 / 2 / 3 (equal at maxvio 1 and within 3% on the large one)
// against 4 vectors, one slot at a time and 16 blocks per CU.  Each block first lists every
// expert's slots: counting them with LDS atomics and placing them with one wave's ballots (instead
// of a loop over all slots per expert) cut that setup from about 6.5 to 0.7 us.
constexpr int kReduceUnroll = 2;
constexpr int kReduceBatch = 4;
constexpr int kReduceBlocksPerCU = 4;
constexpr size_t kMaxDynLds = 160 * 1024 - 1024;

__device__ __forceinline__ void add4(f32x4& a, const f32x4& x) {
  a[0] = a[0] + x[0];
  a[1] = a[1] + x[1];
  a[2] = a[2] + x[2];
  a[3] = a[3] + x[3];
}

__global__ __launch_bounds__(kReduceThreads) void reduce_grad_kernel(const int32_t* __restrict__ slot_expert,
                                                                     f32x4* __restrict__ dW_home,
                                                                     f32x4* __restrict__ dW_slots, int R, int B,
                                                                     int E, int64_t nvec) {
  extern __shared__ int32_t sh[];
  const int RB = R * B;
  int32_t* sslot = sh;          // [RB] expert held by each slot, -1 unused
  int32_t* cnt = sslot + RB;    // [E]  copies of each expert
  int32_t* eoff = cnt + E;      // [E]  start of expert e's slots in lslot
  int32_t* elist = eoff + E;    // [E]  experts with copies, ascending
  int32_t* lslot = elist + E;   // [RB] the slots of each listed expert, ranks ascending
  __shared__ int32_t wsum[kReduceThreads / 64];
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  for (int s = threadIdx.x; s < RB; s += blockDim.x) {
    const int e = slot_expert[s];
    const bool ok = e >= 0 && e < E;
    sslot[s] = ok ? e : -1;
    if (ok) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  const int n = block_compact(E, [&](int e) { return cnt[e] > 0; }, elist, wsum);
  for (int e = threadIdx.x; e < E; e += blockDim.x) eoff[e] = cnt[e];
  __syncthreads();
  block_excl_scan(eoff, E, wsum);
  // each used slot's place in its expert's list, slots in ascending order: wave 0 takes the slots
  // 64 at a time; a lane's rank among the lanes holding the same expert comes from ballots, the
  // slots of earlier rounds from cnt, reused as a running count that ends at the total again
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    for (int e = lane; e < E; e += 64) cnt[e] = 0;
    for (int s0 = 0; s0 < RB; s0 += 64) {
      const int sl = s0 + lane;
      const int e = sl < RB ? sslot[sl] : -1;
      int before = 0, group = 0;
      uint64_t todo = __ballot(e >= 0);
      while (todo) {
        const int el = __shfl(e, __builtin_ctzll(todo), 64);
        const uint64_t m = __ballot(e == el);
        if (e == el) {
          before = __popcll(m & lanemask_lt());
          group = __popcll(m);
        }
        todo &= ~m;
      }
      if (e >= 0) lslot[eoff[e] + cnt[e] + before] = sl;
      if (e >= 0 && before == 0) cnt[e] += group;  // read above by every lane of the group first
    }
  }
  __syncthreads();
  constexpr int U = kReduceUnroll, CB = kReduceBatch, T = kReduceThreads;
  const int64_t per_item = (int64_t)T * U;
  const int64_t chunks = (nvec + per_item - 1) / per_item;
  const int64_t items = (int64_t)n * chunks;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int e = elist[(int)(it / chunks)];
    const int64_t v0 = (it % chunks) * per_item + threadIdx.x;
    f32x4* home = dW_home + (int64_t)e * nvec;
    f32x4 acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (v0 + u * T < nvec) acc[u] = home[v0 + u * T];
    // slots in batches of CB: every load of a batch is issued before its adds (which stay in rank
    // order) and before its stores, so the batch's loads wait on one memory latency together
    const int pa = eoff[e], pe = pa + cnt[e];
    for (int p0 = pa; p0 < pe; p0 += CB) {
      f32x4 x[CB][U];
      f32x4* sl[CB];
#pragma unroll
      for (int q = 0; q < CB; ++q) {
        sl[q] = dW_slots + (int64_t)lslot[min(p0 + q, pe - 1)] * nvec;
        if (p0 + q < pe) {
#pragma unroll
          for (int u = 0; u < U; ++u)
            if (v0 + u * T < nvec)
              x[q][u] = __builtin_nontemporal_load(sl[q] + v0 + u * T);
        }
      }
#pragma unroll
      for (int q = 0; q < CB; ++q)
        if (p0 + q < pe) {
#pragma unroll
          for (int u = 0; u < U; ++u) add4(acc[u], x[q][u]);
        }
      // a slot is read once and cleared: the zeros are stored non-temporally, so they leave no
      // dirty lines behind for the next kernels to write back
#pragma unroll
      for (int q = 0; q < CB; ++q)
        if (p0 + q < pe) {
#pragma unroll
          for (int u = 0; u < U; ++u)
            if (v0 + u * T < nvec) __builtin_nontemporal_store(f32x4{0.f, 0.f, 0.f, 0.f}, sl[q] + v0 + u * T);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (v0 + u * T < nvec) home[v0 + u * T] = acc[u];
  }
}

// scalar fallback: one thread per element (H*Hp not a multiple of 4)
__global__ __launch_bounds__(kReduceThreads) void reduce_grad_scalar(const int32_t* __restrict__ slot_expert,
                                                                     float* __restrict__ dW_home,
                                                                     float* __restrict__ dW_slots, int R, int B,
                                                                     int E, int64_t nel) {
  const int64_t item = (int64_t)blockIdx.x * kReduceThreads + threadIdx.x;
  if (item >= (int64_t)E * nel) return;
  const int e = (int)(item / nel);
  const int64_t x = item % nel;
  bool any = false;
  float acc = 0.f;
  for (int r = 0; r < R; ++r)
    for (int j = 0; j < B; ++j)
      if (slot_expert[r * B + j] == e) {
        if (!any) acc = dW_home[(int64_t)e * nel + x];
        any = true;
        float* sl = dW_slots + ((int64_t)r * B + j) * nel + x;
        acc = acc + *sl;
        *sl = 0.f;
      }
  if (any) dW_home[(int64_t)e * nel + x] = acc;
}

}  // namespace
}  // namespace moonep

using namespace moonep;

extern "C" int moonep_dispatch(moonep_dims d, int32_t H, moonep_dtype t, const void* X, const int32_t* dest_idx,
                               void* Xp, moonep_stream stream) {
  if (int rc = check_dims(d, "moonep_dispatch")) return rc;
  MOONEP_REQUIRE(t == MOONEP_F32 || t == MOONEP_BF16, "moonep_dispatch: bad dtype %d", (int)t);
  MOONEP_REQUIRE(H >= 1, "moonep_dispatch: H must be >= 1");
  const int64_t tokens = (int64_t)d.R * d.S;
  if (tokens == 0) return MOONEP_OK;
  MOONEP_REQUIRE(X && dest_idx && Xp, "moonep_dispatch: null pointer");
  const size_t row = (size_t)H * elem_bytes(t);
  hipStream_t s = as_stream(stream);
  clear_stale_error();
  const bool vec = row % 16 == 0;
  const int nvec = vec ? (int)(row / 16) : H;
  const int pieces = (nvec + 63) / 64;
  const int64_t waves = tokens * pieces;
  MOONEP_REQUIRE(waves / (kDispatchThreads / 64) < (int64_t(1) << 31), "moonep_dispatch: grid too large");
  const unsigned grid = ceil_div_u(waves, kDispatchThreads / 64);
  const bool nt = n_pairs(d) * (int64_t)row > kStreamStoreBytes;
  if (vec) {
    MOONEP_REQUIRE(aligned16(X) && aligned16(Xp), "moonep_dispatch: X and Xp must be 16-byte aligned");
    const u32x4* x = static_cast<const u32x4*>(X);
    u32x4* xp = static_cast<u32x4*>(Xp);
    if (nt)
      hipLaunchKernelGGL((dispatch_rows<u32x4, true>), dim3(grid), dim3(kDispatchThreads), 0, s, x, dest_idx, xp,
                         tokens, d.K, nvec, pieces);
    else
      hipLaunchKernelGGL((dispatch_rows<u32x4, false>), dim3(grid), dim3(kDispatchThreads), 0, s, x, dest_idx, xp,
                         tokens, d.K, nvec, pieces);
  } else if (t == MOONEP_F32) {
    hipLaunchKernelGGL((dispatch_rows<float, false>), dim3(grid), dim3(kDispatchThreads), 0, s,
                       static_cast<const float*>(X), dest_idx, static_cast<float*>(Xp), tokens, d.K, nvec, pieces);
  } else {
    hipLaunchKernelGGL((dispatch_rows<uint16_t, false>), dim3(grid), dim3(kDispatchThreads), 0, s,
                       static_cast<const uint16_t*>(X), dest_idx, static_cast<uint16_t*>(Xp), tokens, d.K, nvec,
                       pieces);
  }
  MOONEP_LAUNCH_CHECK("moonep_dispatch");
  return MOONEP_OK;
}

extern "C" int moonep_prefetch(moonep_dims d, int32_t H, int32_t Hp, moonep_dtype t, const void* W_home,
                               const int32_t* slot_expert, void* W_slots, moonep_stream stream) {
  if (int rc = check_dims(d, "moonep_prefetch")) return rc;
  MOONEP_REQUIRE(t == MOONEP_F32 || t == MOONEP_BF16, "moonep_prefetch: bad dtype %d", (int)t);
  MOONEP_REQUIRE(H >= 1 && Hp >= 1, "moonep_prefetch: H and Hp must be >= 1");
  if (d.B == 0) return MOONEP_OK;
  MOONEP_REQUIRE((int64_t)d.R * d.B <= kMaxSlots, "moonep_prefetch: R*B exceeds %d", kMaxSlots);
  MOONEP_REQUIRE(W_home && slot_expert && W_slots, "moonep_prefetch: null pointer");
  const size_t mat = (size_t)H * Hp * elem_bytes(t);
  hipStream_t s = as_stream(stream);
  clear_stale_error();
  const unsigned grid = (unsigned)device_cu_count() * kCopyBlocksPerCU;
  const size_t lds = (size_t)d.R * d.B * sizeof(int32_t);
  if (lds > 65536) {
    (void)hipFuncSetAttribute((const void*)prefetch_slots<u32x4>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    (void)hipFuncSetAttribute((const void*)prefetch_slots<uint16_t>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  }
  if (mat % 16 == 0) {
    MOONEP_REQUIRE(aligned16(W_home) && aligned16(W_slots), "moonep_prefetch: weights must be 16-byte aligned");
    hipLaunchKernelGGL(prefetch_slots<u32x4>, dim3(grid), dim3(kCopyThreads), lds, s,
                       static_cast<const u32x4*>(W_home), slot_expert, static_cast<u32x4*>(W_slots), d.R * d.B, d.E,
                       (int64_t)(mat / 16));
  } else {
    hipLaunchKernelGGL(prefetch_slots<uint16_t>, dim3(grid), dim3(kCopyThreads), lds, s,
                       static_cast<const uint16_t*>(W_home), slot_expert, static_cast<uint16_t*>(W_slots), d.R * d.B,
                       d.E, (int64_t)(mat / 2));
  }
  MOONEP_LAUNCH_CHECK("moonep_prefetch");
  return MOONEP_OK;
}

namespace {

template <int VEC, int ESZ, bool GATED, int KC>
void combine_vec_k(unsigned grid, hipStream_t s, const char* y, const int32_t* dest, const float* gates, float* out,
                   int64_t tokens, int K, int D) {
  hipLaunchKernelGGL((combine_vec<VEC, ESZ, GATED, uint32_t, KC>), dim3(grid), dim3(kCombineThreads), 0, s, y, dest,
                     gates, out, tokens, K, D);
}

// K up to kBatch gets its own instantiation (the batch then has no branches); 64-bit item indices
// or a larger K take the kernel with K from the call.
template <int VEC, int ESZ, bool GATED>
void combine_vec_launch(bool idx32, int K, unsigned grid, hipStream_t s, const char* y, const int32_t* dest,
                        const float* gates, float* out, int64_t tokens, int D) {
  static_assert(kBatch == 8, "one case per K up to kBatch");
  if (!idx32) {
    hipLaunchKernelGGL((combine_vec<VEC, ESZ, GATED, int64_t, 0>), dim3(grid), dim3(kCombineThreads), 0, s, y, dest,
                       gates, out, tokens, K, D);
    return;
  }
  switch (K) {
    case 1: combine_vec_k<VEC, ESZ, GATED, 1>(grid, s, y, dest, gates, out, tokens, K, D); break;
    case 2: combine_vec_k<VEC, ESZ, GATED, 2>(grid, s, y, dest, gates, out, tokens, K, D); break;
    case 3: combine_vec_k<VEC, ESZ, GATED, 3>(grid, s, y, dest, gates, out, tokens, K, D); break;
    case 4: combine_vec_k<VEC, ESZ, GATED, 4>(grid, s, y, dest, gates, out, tokens, K, D); break;
    case 5: combine_vec_k<VEC, ESZ, GATED, 5>(grid, s, y, dest, gates, out, tokens, K, D); break;
    case 6: combine_vec_k<VEC, ESZ, GATED, 6>(grid, s, y, dest, gates, out, tokens, K, D); break;
    case 7: combine_vec_k<VEC, ESZ, GATED, 7>(grid, s, y, dest, gates, out, tokens, K, D); break;
    case 8: combine_vec_k<VEC, ESZ, GATED, 8>(grid, s, y, dest, gates, out, tokens, K, D); break;
    default: combine_vec_k<VEC, ESZ, GATED, 0>(grid, s, y, dest, gates, out, tokens, K, D); break;
  }
}

// combine (GATED) and dispatch backward (unit gates)
template <bool GATED>
int combine_launch(const char* name, moonep_dims d, int32_t D, moonep_dtype t, const void* Yp,
                   const int32_t* dest_idx, const float* gates, float* out, hipStream_t s) {
  const int64_t tokens = (int64_t)d.R * d.S;
  clear_stale_error();
  const int vec = t == MOONEP_BF16 ? 8 : 4;
  if (D % vec == 0 && aligned16(Yp) && aligned16(out)) {
    const int64_t items = tokens * (D / vec);
    const unsigned grid = ceil_div_u(items, kCombineThreads);
    const bool idx32 = (int64_t)grid * kCombineThreads < (int64_t(1) << 32);
    const char* y = static_cast<const char*>(Yp);
    if (t == MOONEP_BF16)
      combine_vec_launch<8, 2, GATED>(idx32, d.K, grid, s, y, dest_idx, gates, out, tokens, (int)D);
    else
      combine_vec_launch<4, 4, GATED>(idx32, d.K, grid, s, y, dest_idx, gates, out, tokens, (int)D);
  } else {
    const unsigned grid = ceil_div_u(tokens * D, kCombineThreads);
    if (t == MOONEP_BF16)
      hipLaunchKernelGGL((combine_scalar<uint16_t, GATED>), dim3(grid), dim3(kCombineThreads), 0, s,
                         static_cast<const uint16_t*>(Yp), dest_idx, gates, out, tokens, d.K, (int)D);
    else
      hipLaunchKernelGGL((combine_scalar<float, GATED>), dim3(grid), dim3(kCombineThreads), 0, s,
                         static_cast<const float*>(Yp), dest_idx, gates, out, tokens, d.K, (int)D);
  }
  MOONEP_LAUNCH_CHECK(name);
  return MOONEP_OK;
}

}  // namespace

extern "C" int moonep_combine(moonep_dims d, int32_t D, moonep_dtype t, const void* Yp, const int32_t* dest_idx,
                              const float* gates, float* out, moonep_stream stream) {
  if (int rc = check_dims(d, "moonep_combine")) return rc;
  MOONEP_REQUIRE(t == MOONEP_F32 || t == MOONEP_BF16, "moonep_combine: bad dtype %d", (int)t);
  MOONEP_REQUIRE(D >= 1, "moonep_combine: D must be >= 1");
  const int64_t tokens = (int64_t)d.R * d.S;
  if (tokens == 0) return MOONEP_OK;
  MOONEP_REQUIRE(Yp && dest_idx && gates && out, "moonep_combine: null pointer");
  return combine_launch<true>("moonep_combine", d, D, t, Yp, dest_idx, gates, out, as_stream(stream));
}

extern "C" int moonep_reduce_grad(moonep_dims d, int32_t H, int32_t Hp, const int32_t* slot_expert, float* dW_home,
                                  float* dW_slots, moonep_stream stream) {
  if (int rc = check_dims(d, "moonep_reduce_grad")) return rc;
  MOONEP_REQUIRE(H >= 1 && Hp >= 1, "moonep_reduce_grad: H and Hp must be >= 1");
  if (d.B == 0) return MOONEP_OK;
  MOONEP_REQUIRE(slot_expert && dW_home && dW_slots, "moonep_reduce_grad: null pointer");
  hipStream_t s = as_stream(stream);
  clear_stale_error();
  const int64_t nel = (int64_t)H * Hp;
  const size_t lds = ((size_t)2 * d.R * d.B + 3 * (size_t)d.E) * sizeof(int32_t);
  if (nel % 4 == 0 && lds <= kMaxDynLds && aligned16(dW_home) && aligned16(dW_slots)) {
    if (lds > 65536)
      (void)hipFuncSetAttribute((const void*)reduce_grad_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    const unsigned grid = (unsigned)device_cu_count() * kReduceBlocksPerCU;
    hipLaunchKernelGGL(reduce_grad_kernel, dim3(grid), dim3(kReduceThreads), lds, s, slot_expert,
                       reinterpret_cast<f32x4*>(dW_home), reinterpret_cast<f32x4*>(dW_slots), d.R, d.B, d.E, nel / 4);
  } else {
    hipLaunchKernelGGL(reduce_grad_scalar, dim3(ceil_div_u((int64_t)d.E * nel, kReduceThreads)), dim3(kReduceThreads),
                       0, s, slot_expert, dW_home, dW_slots, d.R, d.B, d.E, nel);
  }
  MOONEP_LAUNCH_CHECK("moonep_reduce_grad");
  return MOONEP_OK;
}

extern "C" int moonep_combine_backward(moonep_dims d, int32_t D, moonep_dtype t, const float* dout, const void* Yp,
                                       const int32_t* dest_idx, const float* gates, void* dYp, float* dgates,
                                       moonep_stream stream) {
  if (int rc = check_dims(d, "moonep_combine_backward")) return rc;
  MOONEP_REQUIRE(t == MOONEP_F32 || t == MOONEP_BF16, "moonep_combine_backward: bad dtype %d", (int)t);
  MOONEP_REQUIRE(D >= 1, "moonep_combine_backward: D must be >= 1");
  const int64_t tokens = (int64_t)d.R * d.S;
  if (tokens == 0) return MOONEP_OK;
  MOONEP_REQUIRE(dout && Yp && dest_idx && gates && dYp && dgates, "moonep_combine_backward: null pointer");
  hipStream_t s = as_stream(stream);
  clear_stale_error();
  const unsigned grid = ceil_div_u(tokens, 4);
  const int vec = t == MOONEP_BF16 ? 8 : 4;
  if (D % vec == 0 && aligned16(dout) && aligned16(Yp) && aligned16(dYp)) {
    const int cpl = (D / vec + 63) / 64;  // 16-byte chunks per lane
    const char* y = static_cast<const char*>(Yp);
    char* dy = static_cast<char*>(dYp);
#define MOONEP_CBWD(V, ES, C)                                                                                  \
  hipLaunchKernelGGL((combine_bwd_vec<V, ES, C>), dim3(grid), dim3(256), 0, s, dout, y, dest_idx, gates, dy, dgates, \
                     tokens, d.K, (int)D)
    if (t == MOONEP_BF16) {
      if (cpl <= 1) MOONEP_CBWD(8, 2, 1);
      else if (cpl == 2) MOONEP_CBWD(8, 2, 2);
      else if (cpl <= 4) MOONEP_CBWD(8, 2, 4);
      else MOONEP_CBWD(8, 2, 0);
    } else {
      if (cpl <= 1) MOONEP_CBWD(4, 4, 1);
      else if (cpl == 2) MOONEP_CBWD(4, 4, 2);
      else if (cpl <= 4) MOONEP_CBWD(4, 4, 4);
      else MOONEP_CBWD(4, 4, 0);
    }
#undef MOONEP_CBWD
  } else if (t == MOONEP_BF16) {
    hipLaunchKernelGGL(combine_bwd_scalar<uint16_t>, dim3(grid), dim3(256), 0, s, dout,
                       static_cast<const uint16_t*>(Yp), dest_idx, gates, static_cast<uint16_t*>(dYp), dgates, tokens,
                       d.K, (int)D);
  } else {
    hipLaunchKernelGGL(combine_bwd_scalar<float>, dim3(grid), dim3(256), 0, s, dout, static_cast<const float*>(Yp),
                       dest_idx, gates, static_cast<float*>(dYp), dgates, tokens, d.K, (int)D);
  }
  MOONEP_LAUNCH_CHECK("moonep_combine_backward");
  return MOONEP_OK;
}

extern "C" int moonep_dispatch_backward(moonep_dims d, int32_t H, moonep_dtype t, const void* dXp,
                                        const int32_t* dest_idx, float* dX, moonep_stream stream) {
  if (int rc = check_dims(d, "moonep_dispatch_backward")) return rc;
  MOONEP_REQUIRE(t == MOONEP_F32 || t == MOONEP_BF16, "moonep_dispatch_backward: bad dtype %d", (int)t);
  MOONEP_REQUIRE(H >= 1, "moonep_dispatch_backward: H must be >= 1");
  const int64_t tokens = (int64_t)d.R * d.S;
  if (tokens == 0) return MOONEP_OK;
  MOONEP_REQUIRE(dXp && dest_idx && dX, "moonep_dispatch_backward: null pointer");
  return combine_launch<false>("moonep_dispatch_backward", d, H, t, dXp, dest_idx, nullptr, dX, as_stream(stream));
}
