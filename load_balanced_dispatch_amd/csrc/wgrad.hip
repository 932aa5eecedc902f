// moonep_wgrad: weight-gradient group GEMM into the float32 gradient buffers.
//
// [P2] = "Moonshot open-sources MoonEP: an expert-parallel communication library
// for MoE training" (umios.umi6.com), section "Memory contract and weight
// layout": training keeps an fp32 [E+B, H, H'] gradient per projection; rows
// [E, E+B) are separate reduce buffers (viewed as [R, B, H, H'] across ranks).
//
// Work is split by OUTPUT, so the float32 result is deterministic without
// atomics: job e < E owns dW_home[e] and sums, in ascending rank order, the
// rows every rank holds in its home-row group e (the home rank's kept rows and
// other ranks' direct reads); job E + r*B + j owns slot j of rank r.  An output
// tile is 256 (H) x 128 (H'), reduced over 32-row chunks of the job's rows with
// MFMA 32x32x16 bf16.  Both operands reduce along LDS rows (token rows), so both
// are read with ds_read_b64_tr_b16 from row-major tiles; rows past a segment
// end are zero-filled.  A job without rows writes nothing.  The float32
// read-modify-write of dW goes through LDS so it moves whole 16-byte row chunks.
#include "mfma_tile.h"
#include "moonep_common.h"

namespace moonep {
namespace {

constexpr int kWgBH = 256;
constexpr int kGenBH = 64, kGenBN = 64, kGenBK = 16;

// Walks the row segments of one job, ranks ascending, in chunks of `step` rows.
struct SegWalk {
  const int32_t* cu;
  int R, G1, P, col;  // col = group column in cu (e for home jobs)
  bool home;          // home job: every rank may contribute; slot job: one rank
  int r, r_end;       // current rank, one past the last rank
  int m, end;         // current row and end of the current segment (global rows)

  __device__ bool seek(int from_rank) {
    for (r = from_rank; r < r_end; ++r) {
      const int a = cu[(int64_t)r * G1 + col], b = cu[(int64_t)r * G1 + col + 1];
      if (b > a) {
        m = r * P + a;
        end = r * P + b;
        return true;
      }
    }
    return false;
  }
  __device__ bool next(int step) {
    m += step;
    if (m < end) return true;
    return seek(r + 1);
  }
};

__device__ __forceinline__ SegWalk make_walk(const int32_t* cu, int job, int R, int E, int B, int P) {
  SegWalk s;
  s.cu = cu;
  s.R = R;
  s.G1 = E + B + 1;
  s.P = P;
  if (job < E) {
    s.home = true;
    s.col = job;
    s.r = 0;
    s.r_end = R;
  } else {
    const int sj = job - E;
    s.home = false;
    s.col = E + sj % B;
    s.r = sj / B;
    s.r_end = s.r + 1;
  }
  s.m = s.end = 0;
  return s;
}

template <int BN, int BK>
struct WgCfg {
  static constexpr int BH = kWgBH;
  static constexpr int LDX = BH + 32;  // row pitch = 64 mod 256 bytes for the transpose reads
  static constexpr int LDD = BN + 32;
  static constexpr int WN = BN / 2;
  static constexpr int TM = 4;  // 128 rows of dW per wave / 32
  static constexpr int TN = WN / 32;
  static constexpr int KK = BK / 16;
  static constexpr int X_CPR = BH / 8, D_CPR = BN / 8;  // 16-byte chunks per staged row
  static constexpr int X_VEC = BK * BH / 8 / 256;
  static constexpr int D_VEC = BK * BN / 8 / 256;
  static constexpr int X_ROWS = 256 / X_CPR, D_ROWS = 256 / D_CPR;
  static constexpr int X_STAGE = BK * LDX, D_STAGE = BK * LDD;
  static constexpr int LDS_ELEMS = 2 * (X_STAGE + D_STAGE);
  static constexpr int SP = WN + 4;  // float32 epilogue staging pitch (floats)
  static_assert(4 * 32 * SP * 2 <= LDS_ELEMS, "epilogue staging must fit in the stage buffers");
};

// Two blocks per CU (about 57 KB of LDS and <= 256 registers each).
template <int BN, int BK>
__global__ __launch_bounds__(256, 2) void wgrad_bf16(const uint16_t* __restrict__ Xp, const uint16_t* __restrict__ dY,
                                                     const int32_t* __restrict__ cu, float* __restrict__ dW_home,
                                                     float* __restrict__ dW_slots, int R, int E, int B, int P, int H,
                                                     int Hp) {
  using C = WgCfg<BN, BK>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int HT = H / C::BH, NT = Hp / BN;
  const int per_job = HT * NT;
  const int nblk = gridDim.x;
  // XCD-aware: consecutive tiles of one job on one XCD share its rows in L2
  const int bid = (nblk % 8 == 0) ? (int)(blockIdx.x % 8) * (nblk / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
  const int job = bid / per_job, rem = bid % per_job;
  const int ht = rem / NT, nt = rem % NT;
  const int h0 = ht * C::BH, n0 = nt * BN;

  SegWalk walk = make_walk(cu, job, R, E, B, P);
  if (!walk.seek(walk.r)) return;  // no rows: gradient untouched
  float* out = job < E ? dW_home + (int64_t)job * H * Hp : dW_slots + (int64_t)(job - E) * H * Hp;

  const int x_r = t / C::X_CPR, x_c = t % C::X_CPR;
  const int d_r = t / C::D_CPR, d_c = t % C::D_CPR;
  const uint16_t* x_src = Xp + h0 + x_c * 8;
  const uint16_t* d_src = dY + n0 + d_c * 8;
  uint16_t* const x_st = lds + x_r * C::LDX + x_c * 8;
  uint16_t* const d_st = lds + 2 * C::X_STAGE + d_r * C::LDD + d_c * 8;

  u32x4 rx[C::X_VEC], rd[C::D_VEC];
  auto gload = [&](int m, int end) {  // rows past the segment end load as zeros
#pragma unroll
    for (int i = 0; i < C::X_VEC; ++i) {
      const int row = m + x_r + i * C::X_ROWS;
      rx[i] = row < end ? *reinterpret_cast<const u32x4*>(x_src + (int64_t)row * H) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < C::D_VEC; ++i) {
      const int row = m + d_r + i * C::D_ROWS;
      rd[i] = row < end ? *reinterpret_cast<const u32x4*>(d_src + (int64_t)row * Hp) : u32x4{0, 0, 0, 0};
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::X_VEC; ++i)
      *reinterpret_cast<u32x4*>(x_st + buf * C::X_STAGE + i * C::X_ROWS * C::LDX) = rx[i];
#pragma unroll
    for (int i = 0; i < C::D_VEC; ++i)
      *reinterpret_cast<u32x4*>(d_st + buf * C::D_STAGE + i * C::D_ROWS * C::LDD) = rd[i];
  };

  f32x16 acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j) acc[i][j] = (f32x16)(0.f);

  gload(walk.m, walk.end);
  sstore(0);
  __syncthreads();
  int buf = 0;
  for (;;) {
    const bool more = walk.next(BK);
    if (more) gload(walk.m, walk.end);
    const uint16_t* Xs = lds + buf * C::X_STAGE;
    const uint16_t* Ds = lds + 2 * C::X_STAGE + buf * C::D_STAGE;
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      bf16x8 a[C::TM], b[C::TN];
#pragma unroll
      for (int j = 0; j < C::TN; ++j) b[j] = operand_rows_k(Ds, C::LDD, kk * 16, wn * C::WN + j * 32, lane);
#pragma unroll
      for (int i = 0; i < C::TM; ++i) a[i] = operand_rows_k(Xs, C::LDX, kk * 16, wm * 128 + i * 32, lane);
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
    }
    if (more) sstore(buf ^ 1);
    __syncthreads();
    if (!more) break;
    buf ^= 1;
  }

  // epilogue, one 32-row strip at a time: stage the float32 strip in this wave's
  // LDS region, then dW += strip with 16-byte read-modify-writes of whole rows.
  float* stage = reinterpret_cast<float*>(lds) + w * 32 * C::SP;
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) stage[acc_row(v, lane) * C::SP + j * 32 + (lane & 31)] = acc[i][j][v];
    __syncthreads();
    constexpr int CPR = C::WN / 4;  // 16-byte chunks per staged row
#pragma unroll
    for (int q = lane; q < 32 * CPR; q += 64) {
      const int rr = q / CPR, cc = q % CPR;
      f32x4* p = reinterpret_cast<f32x4*>(out + (int64_t)(h0 + wm * 128 + i * 32 + rr) * Hp + n0 + wn * C::WN + cc * 4);
      const f32x4 s = *reinterpret_cast<const f32x4*>(stage + rr * C::SP + cc * 4);
      f32x4 v = *p;
      v[0] = v[0] + s[0];
      v[1] = v[1] + s[1];
      v[2] = v[2] + s[2];
      v[3] = v[3] + s[3];
      *p = v;
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ generic kernel

template <typename T>
__device__ __forceinline__ float ld(const T* p);
template <>
__device__ __forceinline__ float ld<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

template <typename T>
__global__ __launch_bounds__(256) void wgrad_generic(const T* __restrict__ Xp, const T* __restrict__ dY,
                                                     const int32_t* __restrict__ cu, float* __restrict__ dW_home,
                                                     float* __restrict__ dW_slots, int R, int E, int B, int P, int H,
                                                     int Hp) {
  __shared__ float Xs[kGenBK][kGenBH + 4];
  __shared__ float Ds[kGenBK][kGenBN + 4];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int HT = (H + kGenBH - 1) / kGenBH, NT = (Hp + kGenBN - 1) / kGenBN;
  const int job = blockIdx.x / (HT * NT), rem = blockIdx.x % (HT * NT);
  const int h0 = (rem / NT) * kGenBH, n0 = (rem % NT) * kGenBN;
  SegWalk walk = make_walk(cu, job, R, E, B, P);
  if (!walk.seek(walk.r)) return;
  float* out = job < E ? dW_home + (int64_t)job * H * Hp : dW_slots + (int64_t)(job - E) * H * Hp;
  float acc[4][4] = {};
  do {
    for (int i = threadIdx.x; i < kGenBK * kGenBH; i += 256) {
      const int mr = i / kGenBH, h = i % kGenBH;
      Xs[mr][h] = (walk.m + mr < walk.end && h0 + h < H) ? ld(Xp + (int64_t)(walk.m + mr) * H + h0 + h) : 0.f;
    }
    for (int i = threadIdx.x; i < kGenBK * kGenBN; i += 256) {
      const int mr = i / kGenBN, n = i % kGenBN;
      Ds[mr][n] = (walk.m + mr < walk.end && n0 + n < Hp) ? ld(dY + (int64_t)(walk.m + mr) * Hp + n0 + n) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kGenBK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = Xs[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Ds[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  } while (walk.next(kGenBK));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = h0 + ty * 4 + i;
    if (h >= H) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n < Hp) {
        float* p = out + (int64_t)h * Hp + n;
        *p = *p + acc[i][j];
      }
    }
  }
}

}  // namespace
}  // namespace moonep

using namespace moonep;

extern "C" int moonep_wgrad(moonep_dims d, int32_t H, int32_t Hp, moonep_dtype t, const void* Xp, const void* dY,
                            const int32_t* cu_seqlens, float* dW_home, float* dW_slots, moonep_stream stream) {
  if (int rc = check_dims(d, "moonep_wgrad")) return rc;
  MOONEP_REQUIRE(t == MOONEP_F32 || t == MOONEP_BF16, "moonep_wgrad: bad dtype %d", (int)t);
  MOONEP_REQUIRE(H >= 1 && Hp >= 1, "moonep_wgrad: H and Hp must be >= 1");
  if (n_pairs(d) == 0) return MOONEP_OK;
  MOONEP_REQUIRE(Xp && dY && cu_seqlens && dW_home, "moonep_wgrad: null pointer");
  MOONEP_REQUIRE(d.B == 0 || dW_slots, "moonep_wgrad: dW_slots is null with B > 0");
  hipStream_t s = as_stream(stream);
  clear_stale_error();
  const int64_t jobs = (int64_t)d.E + (int64_t)d.R * d.B;
  const int P = d.S * d.K;
  const bool mfma = t == MOONEP_BF16 && H % kWgBH == 0 && Hp % 128 == 0 && aligned16(Xp) && aligned16(dY) &&
                    aligned16(dW_home) && (d.B == 0 || aligned16(dW_slots));
  if (mfma) {
    const int BN = 128;
    const int64_t blocks = jobs * (H / kWgBH) * (Hp / BN);
    MOONEP_REQUIRE(blocks < (int64_t(1) << 31), "moonep_wgrad: grid too large");
    const auto* x = static_cast<const uint16_t*>(Xp);
    const auto* dy = static_cast<const uint16_t*>(dY);
    hipLaunchKernelGGL((wgrad_bf16<128, 32>), dim3((unsigned)blocks), dim3(256), 0, s, x, dy, cu_seqlens, dW_home,
                       dW_slots, d.R, d.E, d.B, P, H, Hp);
  } else {
    const int64_t blocks = jobs * ((H + kGenBH - 1) / kGenBH) * ((Hp + kGenBN - 1) / kGenBN);
    MOONEP_REQUIRE(blocks < (int64_t(1) << 31), "moonep_wgrad: grid too large");
    if (t == MOONEP_BF16)
      hipLaunchKernelGGL(wgrad_generic<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, s,
                         static_cast<const uint16_t*>(Xp), static_cast<const uint16_t*>(dY), cu_seqlens, dW_home,
                         dW_slots, d.R, d.E, d.B, P, H, Hp);
    else
      hipLaunchKernelGGL(wgrad_generic<float>, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<const float*>(Xp),
                         static_cast<const float*>(dY), cu_seqlens, dW_home, dW_slots, d.R, d.E, d.B, P, H, Hp);
  }
  MOONEP_LAUNCH_CHECK("moonep_wgrad");
  return MOONEP_OK;
}
