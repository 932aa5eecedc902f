// moonep_group_gemm: the VM group GEMM over each rank's logical [E+B, H, Hp] weight tensor.
//
// [P2] = "Moonshot open-sources MoonEP: an expert-parallel communication library
// for MoE training" (umios.umi6.com), section "Memory contract and weight
// layout": one [E+B, H, H'] weight tensor per projection, groups delimited by
// the planner's cu_seqlens; rows [0,E) are home experts, rows [E,E+B) the
// rank's prefetched slots.
//
// Design on gfx950:
//   * ggemm_tiles (one block) turns cu_seqlens into a prefix of M-tiles per
//     (rank, group), in device memory, so the GEMM needs no host sync.
//   * ggemm_bf16<BN> is persistent: one 256-thread block per CU walks the
//     (m-tile, n-tile) list; tile ids are remapped so the blocks of one XCD
//     (workgroups are dealt to the 8 XCDs round-robin) take consecutive tiles,
//     which share the same expert weights and token rows in that XCD's L2.
//     Block tile 256 x 128 x 32, four waves of 128 x 64, MFMA 32x32x16 bf16,
//     two blocks per CU so one block's global loads overlap the other's MFMAs.
//     Tiles go global -> registers -> LDS (double-buffered); the activation
//     operand is read with ds_read_b128 (k contiguous), the weight operand --
//     whose k runs along LDS rows -- with ds_read_b64_tr_b16.  A wave skips
//     MFMAs of 32-row strips past the end of its group.
//   * ggemm_generic<T> is a plain LDS-tiled FMA kernel for float32 and for
//     bf16 shapes the MFMA kernel does not tile (H % 64 or Hp % 128 != 0).
//   The epilogue rounds each 32-row strip to bf16 in LDS and writes whole
//   16-byte row chunks.
#include "block_scan.h"
#include "mfma_tile.h"
#include "moonep_common.h"

namespace moonep {
namespace {

constexpr int kMfmaBM = 256;
constexpr int kGenBM = 64;
constexpr int kGenBN = 64;
constexpr int kGenBK = 16;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int64_t n_groups(const moonep_dims& d) { return (int64_t)d.R * (d.E + d.B); }

// workspace: tiles for BM = 256 then for BM = 64, each [NG + 1] ints
size_t ggemm_ws_bytes(const moonep_dims& d) { return 2 * align256((size_t)(n_groups(d) + 1) * sizeof(int32_t)); }

__global__ __launch_bounds__(1024) void ggemm_tiles(const int32_t* __restrict__ cu, int R, int E, int B,
                                                   int32_t* __restrict__ t256, int32_t* __restrict__ t64) {
  __shared__ int32_t wsum[16];
  const int G = E + B, NG = R * G;
  int carry256 = 0, carry64 = 0;
  for (int i0 = 0; i0 < NG; i0 += blockDim.x) {
    const int i = i0 + threadIdx.x;
    int m = 0;
    if (i < NG) {
      const int r = i / G, g = i % G;
      m = cu[(int64_t)r * (G + 1) + g + 1] - cu[(int64_t)r * (G + 1) + g];
    }
    const int a = (m + kMfmaBM - 1) / kMfmaBM, b = (m + kGenBM - 1) / kGenBM;
    // two scans of this chunk
    const int ia = wave_incl_scan(a), ib = wave_incl_scan(b);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    if (lane == 63) wsum[w] = ia;
    __syncthreads();
    int offa = 0, tota = 0;
    for (int k = 0; k < nw; ++k) {
      if (k < w) offa += wsum[k];
      tota += wsum[k];
    }
    __syncthreads();
    if (lane == 63) wsum[w] = ib;
    __syncthreads();
    int offb = 0, totb = 0;
    for (int k = 0; k < nw; ++k) {
      if (k < w) offb += wsum[k];
      totb += wsum[k];
    }
    __syncthreads();
    if (i < NG) {
      t256[i] = carry256 + offa + ia - a;
      t64[i] = carry64 + offb + ib - b;
    }
    carry256 += tota;
    carry64 += totb;
  }
  if (threadIdx.x == 0) {
    t256[NG] = carry256;
    t64[NG] = carry64;
  }
}

// Last group G in [0, NG) with tstart[G] <= mt (tstart[NG] > mt).
__device__ __forceinline__ int find_group(const int32_t* tstart, int NG, int mt) {
  int lo = 0, hi = NG;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tstart[mid] <= mt) lo = mid; else hi = mid;
  }
  return lo;
}

// ------------------------------------------------------------------ bf16 MFMA kernel

template <int BN, int BK>
struct FwdCfg {
  static constexpr int BM = kMfmaBM;
  static constexpr int LDA = BK + 8;   // row pitch 16 mod 64 bytes: conflict-free ds_read_b128 over 16 rows
  static constexpr int LDB = BN + 32;  // row pitch = 64 mod 256 bytes for the transpose reads
  static constexpr int WN = BN / 2;
  static constexpr int TM = 4;         // 128 rows per wave / 32
  static constexpr int TN = WN / 32;
  static constexpr int KK = BK / 16;   // MFMA k-steps per stage
  static constexpr int A_CPR = BK / 8;  // 16-byte chunks per A row
  static constexpr int B_CPR = BN / 8;  // 16-byte chunks per B row
  static constexpr int A_VEC = BM * BK / 8 / 256;  // 16-byte vectors per thread per stage
  static constexpr int B_VEC = BK * BN / 8 / 256;
  static constexpr int A_ROWS = 256 / A_CPR;  // rows covered by one pass of the block
  static constexpr int B_ROWS = 256 / B_CPR;
  static constexpr int A_STAGE = BM * LDA;   // elements per A stage
  static constexpr int B_STAGE = BK * LDB;
  static constexpr int SP = WN + 8;          // epilogue staging pitch (elements)
  static constexpr int LDS_ELEMS = 2 * (A_STAGE + B_STAGE);
  static_assert(4 * 32 * SP <= LDS_ELEMS, "epilogue staging must fit in the stage buffers");
};

// Two blocks per CU (about 60 KB of LDS and <= 256 registers each), so one
// block's global-load wait overlaps the other's MFMAs.
template <int BN, int BK>
__global__ __launch_bounds__(256, 2) void ggemm_bf16(const uint16_t* __restrict__ Xp,
                                                     const uint16_t* __restrict__ W_home,
                                                     const uint16_t* __restrict__ W_slots,
                                                     const int32_t* __restrict__ cu,
                                                     const int32_t* __restrict__ tstart, uint16_t* __restrict__ Yp,
                                                     int R, int E, int B, int P, int H, int Hp) {
  using C = FwdCfg<BN, BK>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int G = E + B, G1 = G + 1, NG = R * G;
  const int NT = Hp / BN;
  const int total = tstart[NG] * NT;
  const int nblk = gridDim.x;
  const int vb = (nblk % 8 == 0) ? (int)(blockIdx.x % 8) * (nblk / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
  const int KT = H / BK;
  // this thread's slice of each stage: A row a_r + i*A_ROWS, chunk a_c; B row b_r + i*B_ROWS, chunk b_c
  const int a_r = t / C::A_CPR, a_c = t % C::A_CPR;
  const int b_r = t / C::B_CPR, b_c = t % C::B_CPR;
  uint16_t* const a_st = lds + a_r * C::LDA + a_c * 8;                  // + buf*A_STAGE + i*A_ROWS*LDA
  uint16_t* const b_st = lds + 2 * C::A_STAGE + b_r * C::LDB + b_c * 8;  // + buf*B_STAGE + i*B_ROWS*LDB

  for (int tile = vb; tile < total; tile += nblk) {
    const int mt = tile / NT, nt = tile % NT;
    const int grp = find_group(tstart, NG, mt);
    const int r = grp / G, g = grp % G;
    const int c0 = cu[(int64_t)r * G1 + g], c1 = cu[(int64_t)r * G1 + g + 1];
    const int mo = (mt - tstart[grp]) * C::BM;
    const int rows = min(C::BM, c1 - c0 - mo);
    const int64_t row0 = (int64_t)r * P + c0 + mo;
    const uint16_t* Wg = g < E ? W_home + (int64_t)g * H * Hp : W_slots + ((int64_t)r * B + (g - E)) * H * Hp;
    const int n0 = nt * BN;
    const int strips = min(C::TM, max(0, (rows - wm * 128 + 31) / 32));  // valid 32-row strips of this wave

    // global sources; rows past the group end repeat the last valid row (their results are dropped)
    const uint16_t* a_base = Xp + row0 * H + a_c * 8;
    int a_off[C::A_VEC];
#pragma unroll
    for (int i = 0; i < C::A_VEC; ++i) a_off[i] = min(a_r + i * C::A_ROWS, rows - 1) * H;
    const uint16_t* b_src = Wg + (int64_t)b_r * Hp + n0 + b_c * 8;

    u32x4 ra[C::A_VEC], rb[C::B_VEC];
    auto gload = [&](int kt) {
#pragma unroll
      for (int i = 0; i < C::A_VEC; ++i) ra[i] = *reinterpret_cast<const u32x4*>(a_base + a_off[i] + kt * BK);
#pragma unroll
      for (int i = 0; i < C::B_VEC; ++i)
        rb[i] = *reinterpret_cast<const u32x4*>(b_src + ((int64_t)kt * BK + i * C::B_ROWS) * Hp);
    };
    auto sstore = [&](int buf) {
#pragma unroll
      for (int i = 0; i < C::A_VEC; ++i)
        *reinterpret_cast<u32x4*>(a_st + buf * C::A_STAGE + i * C::A_ROWS * C::LDA) = ra[i];
#pragma unroll
      for (int i = 0; i < C::B_VEC; ++i)
        *reinterpret_cast<u32x4*>(b_st + buf * C::B_STAGE + i * C::B_ROWS * C::LDB) = rb[i];
    };
    auto frags = [&](int buf, int kk, bf16x8 (&a)[C::TM], bf16x8 (&b)[C::TN]) {
      const uint16_t* As = lds + buf * C::A_STAGE;
      const uint16_t* Bs = lds + 2 * C::A_STAGE + buf * C::B_STAGE;
#pragma unroll
      for (int j = 0; j < C::TN; ++j) b[j] = operand_rows_k(Bs, C::LDB, kk * 16, wn * C::WN + j * 32, lane);
#pragma unroll
      for (int i = 0; i < C::TM; ++i) a[i] = operand_cols_k(As, C::LDA, wm * 128 + i * 32, kk * 16, lane);
    };

    f32x16 acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j) acc[i][j] = (f32x16)(0.f);

    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk) {
        bf16x8 a[C::TM], b[C::TN];
        frags(buf, kk, a, b);
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
          if (i < strips)
#pragma unroll
            for (int j = 0; j < C::TN; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
      }
      if (kt + 1 < KT) sstore(buf ^ 1);
      __syncthreads();
    }

    // epilogue, one 32-row strip at a time: round to bf16 into this wave's LDS
    // region (accumulator layout), then 16-byte stores of the valid rows.
    uint16_t* stage = lds + w * 32 * C::SP;
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      if (i < strips) {
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            stage[acc_row(v, lane) * C::SP + j * 32 + (lane & 31)] = f32_to_bf16(acc[i][j][v]);
      }
      __syncthreads();
      if (i < strips) {
        constexpr int CPR = C::WN / 8;  // 16-byte chunks per staged row
#pragma unroll
        for (int q = lane; q < 32 * CPR; q += 64) {
          const int rr = q / CPR, cc = q % CPR;
          const int row = wm * 128 + i * 32 + rr;
          if (row < rows)
            *reinterpret_cast<u32x4*>(Yp + (row0 + row) * Hp + n0 + wn * C::WN + cc * 8) =
                *reinterpret_cast<const u32x4*>(stage + rr * C::SP + cc * 8);
        }
      }
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------------ generic kernel

template <typename T>
__device__ __forceinline__ float load_elem(const T* p);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

template <typename T>
__device__ __forceinline__ void store_elem(T* p, float v);
template <>
__device__ __forceinline__ void store_elem<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_elem<uint16_t>(uint16_t* p, float v) { *p = f32_to_bf16(v); }

template <typename T>
__global__ __launch_bounds__(256) void ggemm_generic(const T* __restrict__ Xp, const T* __restrict__ W_home,
                                                     const T* __restrict__ W_slots, const int32_t* __restrict__ cu,
                                                     const int32_t* __restrict__ tstart, T* __restrict__ Yp, int R,
                                                     int E, int B, int P, int H, int Hp) {
  __shared__ float As[kGenBK][kGenBM + 4];
  __shared__ float Bs[kGenBK][kGenBN + 4];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int G = E + B, G1 = G + 1, NG = R * G;
  const int NT = (Hp + kGenBN - 1) / kGenBN;
  const int total = tstart[NG] * NT;
  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const int mt = tile / NT, nt = tile % NT;
    const int grp = find_group(tstart, NG, mt);
    const int r = grp / G, g = grp % G;
    const int c0 = cu[(int64_t)r * G1 + g], c1 = cu[(int64_t)r * G1 + g + 1];
    const int mo = (mt - tstart[grp]) * kGenBM;
    const int rows = min(kGenBM, c1 - c0 - mo);
    const int64_t row0 = (int64_t)r * P + c0 + mo;
    const T* Wg = g < E ? W_home + (int64_t)g * H * Hp : W_slots + ((int64_t)r * B + (g - E)) * H * Hp;
    const int n0 = nt * kGenBN;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < H; k0 += kGenBK) {
      for (int i = threadIdx.x; i < kGenBK * kGenBM; i += 256) {
        const int m = i / kGenBK, k = i % kGenBK;
        As[k][m] = (m < rows && k0 + k < H) ? load_elem(Xp + (row0 + m) * H + k0 + k) : 0.f;
      }
      for (int i = threadIdx.x; i < kGenBK * kGenBN; i += 256) {
        const int k = i / kGenBN, n = i % kGenBN;
        Bs[k][n] = (k0 + k < H && n0 + n < Hp) ? load_elem(Wg + (int64_t)(k0 + k) * Hp + n0 + n) : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kGenBK; ++k) {
        float a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = As[k][ty * 4 + i];
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = Bs[k][tx * 4 + j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
      }
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = ty * 4 + i;
      if (m >= rows) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + tx * 4 + j;
        if (n < Hp) store_elem(Yp + (row0 + m) * Hp + n, acc[i][j]);
      }
    }
  }
}

}  // namespace
}  // namespace moonep

using namespace moonep;

extern "C" size_t moonep_group_gemm_workspace_bytes(moonep_dims d) {
  if (check_dims(d, "moonep_group_gemm_workspace_bytes") != MOONEP_OK) return 0;
  return ggemm_ws_bytes(d);
}

extern "C" int moonep_group_gemm(moonep_dims d, int32_t H, int32_t Hp, moonep_dtype t, const void* Xp,
                                 const void* W_home, const void* W_slots, const int32_t* cu_seqlens, void* Yp,
                                 void* workspace, moonep_stream stream) {
  if (int rc = check_dims(d, "moonep_group_gemm")) return rc;
  MOONEP_REQUIRE(t == MOONEP_F32 || t == MOONEP_BF16, "moonep_group_gemm: bad dtype %d", (int)t);
  MOONEP_REQUIRE(H >= 1 && Hp >= 1, "moonep_group_gemm: H and Hp must be >= 1");
  if (n_pairs(d) == 0) return MOONEP_OK;
  MOONEP_REQUIRE(Xp && W_home && cu_seqlens && Yp && workspace, "moonep_group_gemm: null pointer");
  MOONEP_REQUIRE(d.B == 0 || W_slots, "moonep_group_gemm: W_slots is null with B > 0");
  MOONEP_REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0,
                 "moonep_group_gemm: workspace must be 256-byte aligned");
  MOONEP_REQUIRE(n_groups(d) < (int64_t(1) << 30), "moonep_group_gemm: too many groups");
  hipStream_t s = as_stream(stream);
  clear_stale_error();
  int32_t* t256 = static_cast<int32_t*>(workspace);
  int32_t* t64 = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                            align256((size_t)(n_groups(d) + 1) * sizeof(int32_t)));
  hipLaunchKernelGGL(ggemm_tiles, dim3(1), dim3(1024), 0, s, cu_seqlens, d.R, d.E, d.B, t256, t64);
  MOONEP_LAUNCH_CHECK("moonep_group_gemm/tiles");
  const int cus = device_cu_count();
  const bool mfma = t == MOONEP_BF16 && H % 32 == 0 && Hp % 128 == 0 && aligned16(Xp) &&
                    aligned16(W_home) && (d.B == 0 || aligned16(W_slots));
  if (mfma) {
    const auto* x = static_cast<const uint16_t*>(Xp);
    const auto* wh = static_cast<const uint16_t*>(W_home);
    const auto* ws = static_cast<const uint16_t*>(W_slots);
    auto* y = static_cast<uint16_t*>(Yp);
    const int P = d.S * d.K;
    hipLaunchKernelGGL((ggemm_bf16<128, 32>), dim3(2 * cus), dim3(256), 0, s, x, wh, ws, cu_seqlens, t256, y, d.R,
                       d.E, d.B, P, H, Hp);
  } else if (t == MOONEP_BF16) {
    hipLaunchKernelGGL(ggemm_generic<uint16_t>, dim3(cus * 4), dim3(256), 0, s, static_cast<const uint16_t*>(Xp),
                       static_cast<const uint16_t*>(W_home), static_cast<const uint16_t*>(W_slots), cu_seqlens, t64,
                       static_cast<uint16_t*>(Yp), d.R, d.E, d.B, d.S * d.K, H, Hp);
  } else {
    hipLaunchKernelGGL(ggemm_generic<float>, dim3(cus * 4), dim3(256), 0, s, static_cast<const float*>(Xp),
                       static_cast<const float*>(W_home), static_cast<const float*>(W_slots), cu_seqlens, t64,
                       static_cast<float*>(Yp), d.R, d.E, d.B, d.S * d.K, H, Hp);
  }
  MOONEP_LAUNCH_CHECK("moonep_group_gemm");
  return MOONEP_OK;
}
