// moonep_group_gemm: the VM group GEMM over each rank's logical [E+B, H, Hp] weight tensor.
//
// [P2] = "Moonshot open-sources MoonEP: an expert-parallel communication library
// for MoE training" (umios.umi6.com), section "Memory contract and weight
// layout": one [E+B, H, H'] weight tensor per projection, groups delimited by
// the planner's cu_seqlens; rows [0,E) are home experts, rows [E,E+B) the
// rank's prefetched slots.
//
// Design on gfx950:
//   * ggemm_tiles (one block) turns cu_seqlens into a prefix of 256-row M-tiles per
//     (rank, group), in device memory, so the GEMM needs no host sync.
//   * fwd::ggemm_bf16 is persistent (one 512-thread block per CU), 256 x 256 x 32 block tiles,
//     eight waves of 128 x 64 with MFMA 32x32x16 bf16 in two ping-pong groups (one computes while
//     the other loads).  Operands stream global -> LDS with
//     global_load_lds_dwordx4 into a 4-stage ring; the activation operand (k contiguous) is read
//     with ds_read_b128, the weight operand (k along LDS rows, as the [H, H'] layout stores it)
//     with ds_read_b64_tr_b16; both LDS layouts are XOR-swizzled against bank conflicts.  The
//     epilogue rounds one 32-row strip at a time to bf16 in LDS and writes whole 16-byte chunks.
//     Where N is a multiple of 512, a group's last m-tile of at most 128 rows runs as 128 x 512
//     tiles, so that fewer rows past the group end are computed.
//   * ggemm_generic<T> is a plain LDS-tiled kernel for float32 and for bf16 shapes the bf16 MFMA
//     kernel does not tile (H % 32 or H' % 64 != 0): 64 x 64 x 16 block tiles held as float32 in
//     LDS, four waves of 32 x 32, each a chain of float32 MFMA 32x32x2 steps.
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

// workspace: tiles of the bf16 kernel, then 64-row tiles of the generic kernel, each [NG + 1] ints
size_t ggemm_ws_bytes(const moonep_dims& d) { return 2 * align256((size_t)(n_groups(d) + 1) * sizeof(int32_t)); }

// With tail tiles, a group of m rows runs as full-height (256-row) m-tiles times the 256-wide n-tiles,
// except that a last m-tile of at most 128 rows runs as a 128-row m-tile times 512-wide n-tiles.
__device__ __forceinline__ int full_mtiles(int m) {
  const int rem = m & (kMfmaBM - 1);
  return m / kMfmaBM + (rem > kMfmaBM / 2 ? 1 : 0);
}

// Per group, in t256: the bf16 kernel's tiles (with tail tiles: every tile of the group, N being a
// multiple of 512; without: its 256-row m-tiles); in t64: the generic kernel's 64-row m-tiles.
__global__ __launch_bounds__(1024) void ggemm_tiles(const int32_t* __restrict__ cu, int R, int E, int B, int N,
                                                   int tails, int32_t* __restrict__ t256,
                                                   int32_t* __restrict__ t64) {
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
    int a = (m + kMfmaBM - 1) / kMfmaBM;
    if (tails) {
      const int f = full_mtiles(m);
      a = f * (N / kMfmaBM) + (m > f * kMfmaBM ? N / (2 * kMfmaBM) : 0);
    }
    const int b = (m + kGenBM - 1) / kGenBM;
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

namespace fwd {
constexpr int BM = 256, BN = 256, BK = 32, STAGES = 4, NWAVES = 8;
constexpr int OPS = 4;  // DMA instructions per wave per stage (2 for A, 2 for B)
constexpr int kBandM = 4;  // m-tiles per band of the tile raster
constexpr int A_STAGE = BM * BK;  // 64-byte rows; 16-byte chunks XOR-swizzled by row
constexpr int B_STAGE = BK * BN;  // 512-byte rows; 64-byte blocks XOR-swizzled by row
constexpr int A_TAIL = BM / 2 * BK;  // a 128 x 512 tail tile's A stage
// a ring slot holds a full tile's stage (A, then B) or, with tail tiles, a tail tile's (its 128-row
// A, then B as two 256-column parts, each laid out like a full tile's B)
template <bool TAILS>
constexpr int STAGE = TAILS ? A_TAIL + 2 * B_STAGE : A_STAGE + B_STAGE;
constexpr int WN = 64, TM = 4, TN = 2, KK = BK / 16;
constexpr int SP = WN + 8;  // epilogue staging pitch (elements)
template <bool TAILS>
constexpr int LDS_ELEMS = STAGES * STAGE<TAILS>;
static_assert(NWAVES * 32 * SP <= LDS_ELEMS<false>, "epilogue staging must fit in the ring");
static_assert(A_STAGE + B_STAGE <= STAGE<true> && LDS_ELEMS<true> * 2 <= 160 * 1024, "slot sizes");

// A stage (rows = tokens, 4 chunks of 8 k-values per row): the chunk order is permuted per row so
// that the 16-byte operand reads of 16 consecutive rows, and of the two k-halves of 8 rows, hit
// distinct LDS banks.
__device__ __forceinline__ int a_swz(int row) { return (((row >> 2) & 1) << 1) | ((row >> 3) & 1); }
__device__ __forceinline__ int a_off(int row, int c) { return row * BK + 8 * (c ^ a_swz(row)); }
// B stage (rows = k, 256 output columns): the 64-byte blocks of row k are permuted by k % 4 so the
// four rows a transpose read touches land in different banks.
__device__ __forceinline__ int b_off(int k, int n) { return k * BN + ((((n >> 5) ^ (k & 3)) << 5) | (n & 31)); }

// C[rows of (r, g)] = A[those rows] @ op(W_r[g]), every W_r[g] an [H, H'] row-major matrix:
//   forward (BT = false): A = Xp [N, H], op(W) = W, C = Yp [N, H']  (K = H,  N = H')
//   dgrad   (BT = true):  A = dYp [N, H'], op(W) = W^T, C = dXp [N, H] (K = H', N = H)
// With BT the weight tile is stored n-major (each output column's k-run is 64 contiguous bytes of a
// W row), so it is staged and read exactly like the activation tile; otherwise it is k-major and
// read with the transpose read.
//
// Persistent: one 512-thread block per CU; block ids are remapped so the blocks of one XCD
// (workgroups are dealt to the 8 XCDs round-robin) take consecutive tile ids, and tile ids follow
// a banded raster (4 m-tiles x all n-tiles per band, n-major inside), so those tiles share token
// rows and expert weights in that XCD's L2.  Block tile 256 x 256 x 32; eight waves of 128 x 64
// (MFMA 32x32x16 bf16, two waves per SIMD).  Operand tiles stream global -> LDS with
// global_load_lds_dwordx4 into a 4-stage ring, three stages ahead of the MFMAs, with no
// register staging.  The last n-tile may be narrower than 256 (H' % 256 != 0): its missing
// columns load a repeated valid column and their waves skip MFMAs and stores.
//
// TAILS (N a multiple of 512): a group whose last m-tile would hold at most 128 rows runs that tail
// as 128 x 512 tiles (one row of eight 128 x 64 waves), which halves the rows computed past the group
// end, and tiles are numbered group by group (each group's full m-tiles in bands, then its tail).
template <bool BT, bool TAILS>
__global__ __launch_bounds__(512, 1) void ggemm_bf16(const uint16_t* __restrict__ Xp,
                                                     const uint16_t* __restrict__ W_home,
                                                     const uint16_t* __restrict__ W_slots,
                                                     const int32_t* __restrict__ cu,
                                                     const int32_t* __restrict__ tstart, uint16_t* __restrict__ Yp,
                                                     int R, int E, int B, int P, int H, int Hp) {
  constexpr int kStage = STAGE<TAILS>;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[LDS_ELEMS<TAILS>];
  const int K = BT ? Hp : H, N = BT ? H : Hp;  // reduction length and output width
  const uint32_t lds0 = lds_addr(lds);                            // LDS byte address of the ring
  const int wu = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index, uniform
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wn = w & 3;  // the wave's 64-column strip inside a 256-column B part
  const int G = E + B, G1 = G + 1, NG = R * G;
  const int NT = (N + BN - 1) / BN;
  const int total = TAILS ? tstart[NG] : tstart[NG] * NT;
  const int nblk = gridDim.x;
  const int vb = (nblk % 8 == 0) ? (int)(blockIdx.x % 8) * (nblk / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
  const int KT = K / BK;
  const int a_lr = lane >> 2, a_ls = lane & 3;   // A: one wave instruction fills 16 rows
  const int b_lr = lane >> 5, b_ls = lane & 31;  // B: one wave instruction fills 2 rows

  for (int tile = vb; tile < total; tile += nblk) {
    // banded raster: bands of kBandM consecutive m-tiles, n-tile-major inside a band, so the 32
    // tiles one XCD runs at once cover a kBandM x 8 block and reuse both operands in its L2 (with
    // tail tiles the bands are a group's own m-tiles, and its tail tiles follow them)
    int grp, mt, nt;
    bool tail = false;
    if constexpr (TAILS) {
      grp = find_group(tstart, NG, tile);
      const int r_ = grp / G, g_ = grp % G;
      const int mts = full_mtiles(cu[(int64_t)r_ * G1 + g_ + 1] - cu[(int64_t)r_ * G1 + g_]);
      const int local = tile - tstart[grp];
      if (local < mts * NT) {
        const int band = local / (kBandM * NT), m0b = band * kBandM;
        const int sb = min(kBandM, mts - m0b), rb = local - band * kBandM * NT;
        mt = m0b + rb % sb;
        nt = rb / sb;
      } else {
        mt = mts;
        nt = local - mts * NT;
        tail = true;
      }
    } else {
      const int MT = tstart[NG];
      const int band = tile / (kBandM * NT), m0b = band * kBandM;
      const int sb = min(kBandM, MT - m0b), rb = tile - band * kBandM * NT;
      const int mtg = m0b + rb % sb;
      nt = rb / sb;
      grp = find_group(tstart, NG, mtg);
      mt = mtg - tstart[grp];
    }
    const int r = grp / G, g = grp % G;
    const int c0 = cu[(int64_t)r * G1 + g], c1 = cu[(int64_t)r * G1 + g + 1];
    const int mo = mt * BM;
    const int rows = min(tail ? BM / 2 : BM, c1 - c0 - mo);
    const int64_t row0 = (int64_t)r * P + c0 + mo;
    const uint16_t* Wg = g < E ? W_home + (int64_t)g * H * Hp : W_slots + ((int64_t)r * B + (g - E)) * H * Hp;
    const int n0 = nt * (tail ? 2 * BN : BN);
    const int width = min(tail ? 2 * BN : BN, N - n0);
    // wave tile origin: 2 x 4 waves of 128 x 64 in a full tile, 1 x 8 in a tail tile, whose waves 4-7
    // read the second B part
    const int wr0 = tail ? 0 : (w >> 2) * 128, wc0 = tail ? w * WN : wn * WN;
    const int b_at = tail ? A_TAIL + (w >> 2) * B_STAGE : A_STAGE;  // this wave's B part, elements into a slot
    const int strips = min(TM, max(0, (rows - wr0 + 31) / 32));  // valid 32-row strips of this wave
    const bool wave_cols = wc0 < width;

    // global sources of this wave's DMA instructions per stage: 2 for A and 2 for B in a full tile,
    // 1 for A and 2 for each B part in a tail tile
    const uint16_t* a_src[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = tail ? w * 16 + a_lr : (2 * w + i) * 16 + a_lr;  // rows past the group end repeat its last row
      a_src[i] = Xp + (row0 + min(row, rows - 1)) * K + 8 * (a_ls ^ a_swz(row));
    }
    const uint16_t* b_src[TAILS ? 4 : 2];
#pragma unroll
    for (int i = 0; i < (TAILS ? 4 : 2); ++i) {
      const int nb = n0 + (i >> 1) * BN;  // first column of B part i / 2
      if (BT) {  // output columns past N repeat the last one
        const int row = (2 * w + (i & 1)) * 16 + a_lr;
        b_src[i] = Wg + (int64_t)min(nb + row, N - 1) * Hp + 8 * (a_ls ^ a_swz(row));
      } else {
        const int k = (2 * w + (i & 1)) * 2 + b_lr;
        const int q = (b_ls >> 2) ^ (k & 3);
        b_src[i] = Wg + (int64_t)k * Hp + min(nb + (q * 4 + (b_ls & 3)) * 8, Hp - 8);
      }
    }
    const int64_t b_step = BT ? BK : (int64_t)BK * Hp;  // one stage along k
    auto issue = [&](int kt) {  // this wave's 1 KB pieces of stage kt
      const uint32_t sl = lds0 + (uint32_t)((kt % STAGES) * kStage * 2);
      if constexpr (TAILS) {
        if (tail) {
          dma16(a_src[0] + kt * BK, sl + wu * 1024);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            dma16(b_src[i] + kt * b_step, sl + (A_TAIL + (i >> 1) * B_STAGE) * 2 + wu * 2 * 1024 + (i & 1) * 1024);
          return;
        }
      }
      const uint32_t st = sl + wu * 2 * 1024;  // slot byte base + (2w + i) KB
#pragma unroll
      for (int i = 0; i < 2; ++i) dma16(a_src[i] + kt * BK, st + i * 1024);
#pragma unroll
      for (int i = 0; i < 2; ++i) dma16(b_src[i] + kt * b_step, st + A_STAGE * 2 + i * 1024);
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = (f32x16)(0.f);

    for (int st = 0; st < STAGES - 1 && st < KT; ++st) issue(st);
    auto frag = [&](int kt, int kk, bf16x8 (&a)[TM], bf16x8 (&b)[TN]) {
      const uint16_t* As = lds + (kt % STAGES) * kStage;
      const uint16_t* Bs = As + b_at;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if (BT) {
          const int n = wn * WN + j * 32 + (lane & 31);
          b[j] = *reinterpret_cast<const bf16x8*>(Bs + a_off(n, kk * 2 + (lane >> 5)));
        } else {
          const int grp4 = lane >> 4, c = lane & 15;
          const int n = wn * WN + j * 32 + 16 * (grp4 & 1) + 4 * (c & 3);
          const int k = kk * 16 + 8 * (grp4 >> 1) + (c >> 2);
          const bf16x4 lo = lds_tr4(Bs + b_off(k, n));
          const bf16x4 hi = lds_tr4(Bs + b_off(k + 4, n));
          b[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wr0 + i * 32 + (lane & 31);
        a[i] = *reinterpret_cast<const bf16x8*>(As + a_off(row, kk * 2 + (lane >> 5)));
      }
    };
    auto mma = [&](const bf16x8 (&a)[TM], const bf16x8 (&b)[TN]) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
    };
    // Ping-pong: waves 0-3 (group A, one per SIMD) and 4-7 (group B, the other wave of each SIMD)
    // alternate between a memory phase (the operands of one stage, LDS -> registers, plus this
    // wave's share of the DMA three stages ahead) and a compute phase (that stage's 16 MFMAs), half
    // a stage apart, so while one wave of a SIMD waits on LDS the other keeps the MFMA pipe busy.
    // Phase q opens with a barrier.  A: memory(t) in phase 2t, compute(t) in 2t+1; B: memory(t) in
    // 2t+1, compute(t) in 2t+2; 2*KT + 1 phases.  memory(t) refills the slot of stage t-1, which B
    // read in phase 2t-1.  A tile at a group's end computes all its strips (rows past the end load
    // the group's last row); the epilogue stores only the valid rows.
    bf16x8 fa[KK][TM], fb[KK][TN];
    auto mem = [&](int t) {
      if (wave_cols) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) frag(t, kk, fa[kk], fb[kk]);
      }
      if (t + STAGES - 1 < KT) issue(t + STAGES - 1);
    };
    // the computing wave of a SIMD runs at raised priority, so the arbiter keeps its MFMAs issuing
    // ahead of the other wave's LDS reads (measured ~2% on the mid workload; no gain in wgrad)
    auto comp = [&]() {
      if (wave_cols) {
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) mma(fa[kk], fb[kk]);
        __builtin_amdgcn_s_setprio(0);
      }
    };
    // barrier opening phase 2t: this wave has issued the stages up to min(t + 2, KT - 1), so
    // waiting until only the later ones are in flight means its share of stage t has landed, and
    // the barrier extends that to every wave's share (a tail tile's stage is 5 DMAs per wave)
    auto even_barrier = [&](int t) {
      if (t + 2 < KT) {
        if (tail) wait_vmcnt<2 * (OPS + 1)>();
        else wait_vmcnt<2 * OPS>();
      } else if (t + 1 < KT) {
        if (tail) wait_vmcnt<OPS + 1>();
        else wait_vmcnt<OPS>();
      } else {
        wait_vmcnt<0>();
      }
      lds_barrier();
    };
    if (w < 4) {
      for (int t = 0; t < KT; ++t) {
        even_barrier(t);
        mem(t);
        plain_barrier();  // slot t is next refilled in phase 2t + 2, after comp() has consumed these reads
        comp();
      }
      even_barrier(KT);
    } else {
      even_barrier(0);
      for (int t = 0; t < KT; ++t) {
        lds_barrier();
        mem(t);
        even_barrier(t + 1);
        comp();
      }
    }
    lds_barrier();  // the ring is free: every wave has read its last stage

    // epilogue, one 32-row strip at a time: round to bf16 into this wave's LDS region
    // (accumulator layout), then 16-byte stores of whole row chunks of the valid rows.
    uint16_t* stage = lds + w * 32 * SP;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      const bool live = i < strips && wave_cols;
      if (live) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            stage[acc_row(v, lane) * SP + j * 32 + (lane & 31)] = f32_to_bf16(acc[i][j][v]);
      }
      __syncthreads();
      if (live) {
        constexpr int CPR = WN / 8;
#pragma unroll
        for (int q = lane; q < 32 * CPR; q += 64) {
          const int rr = q / CPR, cc = q % CPR;
          const int row = wr0 + i * 32 + rr;
          if (row < rows)
            *reinterpret_cast<u32x4*>(Yp + (row0 + row) * N + n0 + wc0 + cc * 8) =
                *reinterpret_cast<const u32x4*>(stage + rr * SP + cc * 8);
        }
      }
      __syncthreads();
    }
  }
}
}  // namespace fwd

// ------------------------------------------------------------------ generic kernel
//
// One 256-thread block per 64 x 64 output tile (grid-stride over the 64-row tile prefix), K in steps
// of 16 staged as float32 in LDS (bf16 widened exactly), zeros past a group's rows and past K;
// four waves of 32 x 32 reduce with v_mfma_f32_32x32x2_f32.

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

template <typename T, bool BT>
__global__ __launch_bounds__(256) void ggemm_generic(const T* __restrict__ Xp, const T* __restrict__ W_home,
                                                     const T* __restrict__ W_slots, const int32_t* __restrict__ cu,
                                                     const int32_t* __restrict__ tstart, T* __restrict__ Yp, int R,
                                                     int E, int B, int P, int H, int Hp) {
  __shared__ float As[kGenBK][kGenBM + 4];
  __shared__ float Bs[kGenBK][kGenBN + 4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;  // 2 x 2 waves of 32 x 32
  const int K = BT ? Hp : H, N = BT ? H : Hp;  // reduction length and output width (as in ggemm_bf16)
  const int G = E + B, G1 = G + 1, NG = R * G;
  const int NT = (N + kGenBN - 1) / kGenBN;
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
    f32x16 acc = (f32x16)(0.f);
    for (int k0 = 0; k0 < K; k0 += kGenBK) {
      for (int i = threadIdx.x; i < kGenBK * kGenBM; i += 256) {
        const int m = i / kGenBK, k = i % kGenBK;
        As[k][m] = (m < rows && k0 + k < K) ? load_elem(Xp + (row0 + m) * K + k0 + k) : 0.f;
      }
      for (int i = threadIdx.x; i < kGenBK * kGenBN; i += 256) {
        const int k = i / kGenBN, n = i % kGenBN;
        const int64_t at = BT ? (int64_t)(n0 + n) * Hp + k0 + k : (int64_t)(k0 + k) * Hp + n0 + n;
        Bs[k][n] = (k0 + k < K && n0 + n < N) ? load_elem(Wg + at) : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kGenBK; k += 2)
        acc = mfma32_f32(As[k + (lane >> 5)][wm * 32 + (lane & 31)], Bs[k + (lane >> 5)][wn * 32 + (lane & 31)], acc);
      __syncthreads();
    }
    const int n = n0 + wn * 32 + (lane & 31);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = wm * 32 + acc_row(v, lane);
      if (m < rows && n < N) store_elem(Yp + (row0 + m) * N + n, acc[v]);
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

namespace {

// Shared by the forward GEMM and dgrad: BT selects op(W) = W^T (see ggemm_bf16).
template <bool BT>
int group_gemm_launch(const char* name, moonep_dims d, int32_t H, int32_t Hp, moonep_dtype t, const void* A,
                      const void* W_home, const void* W_slots, const int32_t* cu_seqlens, void* C, void* workspace,
                      moonep_stream stream) {
  if (int rc = check_dims(d, name)) return rc;
  MOONEP_REQUIRE(t == MOONEP_F32 || t == MOONEP_BF16, "%s: bad dtype %d", name, (int)t);
  MOONEP_REQUIRE(H >= 1 && Hp >= 1, "%s: H and Hp must be >= 1", name);
  if (n_pairs(d) == 0) return MOONEP_OK;
  MOONEP_REQUIRE(A && W_home && cu_seqlens && C && workspace, "%s: null pointer", name);
  MOONEP_REQUIRE(d.B == 0 || W_slots, "%s: W_slots is null with B > 0", name);
  MOONEP_REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, "%s: workspace must be 256-byte aligned",
                 name);
  MOONEP_REQUIRE(n_groups(d) < (int64_t(1) << 30), "%s: too many groups", name);
  {
    // rows of 16-byte multiples move as 16-byte vectors: their base pointers must be 16-byte aligned
    const int64_t eb = (int64_t)elem_bytes(t);
    const int64_t a_row = (BT ? Hp : H) * eb, c_row = (BT ? H : Hp) * eb, w_row = (int64_t)Hp * eb;
    MOONEP_REQUIRE(a_row % 16 || aligned16(A), "%s: the input rows must be 16-byte aligned", name);
    MOONEP_REQUIRE(c_row % 16 || aligned16(C), "%s: the output rows must be 16-byte aligned", name);
    MOONEP_REQUIRE(w_row % 16 || (aligned16(W_home) && (d.B == 0 || aligned16(W_slots))),
                   "%s: the weight rows must be 16-byte aligned", name);
  }
  hipStream_t s = as_stream(stream);
  clear_stale_error();
  int32_t* t256 = static_cast<int32_t*>(workspace);
  int32_t* t64 = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                            align256((size_t)(n_groups(d) + 1) * sizeof(int32_t)));
  const int cus = device_cu_count();
  const int K = BT ? Hp : H, N = BT ? H : Hp;
  const bool mfma = t == MOONEP_BF16 && K % 32 == 0 && N % 64 == 0 && aligned16(A) && aligned16(W_home) &&
                    (d.B == 0 || aligned16(W_slots));
  // tail tiles only where every 512-wide tail n-tile is whole (measured: on the 1408-wide output
  // the kernel built with them ran 2-3% slower, tail tiles or not)
  const bool tails = mfma && N % 512 == 0;
  hipLaunchKernelGGL(ggemm_tiles, dim3(1), dim3(1024), 0, s, cu_seqlens, d.R, d.E, d.B, N, tails ? 1 : 0, t256, t64);
  MOONEP_LAUNCH_CHECK(name);
  const int P = d.S * d.K;
  if (tails) {
    hipLaunchKernelGGL((fwd::ggemm_bf16<BT, true>), dim3(cus), dim3(512), 0, s, static_cast<const uint16_t*>(A),
                       static_cast<const uint16_t*>(W_home), static_cast<const uint16_t*>(W_slots), cu_seqlens, t256,
                       static_cast<uint16_t*>(C), d.R, d.E, d.B, P, H, Hp);
  } else if (mfma) {
    hipLaunchKernelGGL((fwd::ggemm_bf16<BT, false>), dim3(cus), dim3(512), 0, s, static_cast<const uint16_t*>(A),
                       static_cast<const uint16_t*>(W_home), static_cast<const uint16_t*>(W_slots), cu_seqlens, t256,
                       static_cast<uint16_t*>(C), d.R, d.E, d.B, P, H, Hp);
  } else if (t == MOONEP_BF16) {
    hipLaunchKernelGGL((ggemm_generic<uint16_t, BT>), dim3(cus * 4), dim3(256), 0, s, static_cast<const uint16_t*>(A),
                       static_cast<const uint16_t*>(W_home), static_cast<const uint16_t*>(W_slots), cu_seqlens, t64,
                       static_cast<uint16_t*>(C), d.R, d.E, d.B, P, H, Hp);
  } else {
    hipLaunchKernelGGL((ggemm_generic<float, BT>), dim3(cus * 4), dim3(256), 0, s, static_cast<const float*>(A),
                       static_cast<const float*>(W_home), static_cast<const float*>(W_slots), cu_seqlens, t64,
                       static_cast<float*>(C), d.R, d.E, d.B, P, H, Hp);
  }
  MOONEP_LAUNCH_CHECK(name);
  return MOONEP_OK;
}

}  // namespace

extern "C" int moonep_group_gemm(moonep_dims d, int32_t H, int32_t Hp, moonep_dtype t, const void* Xp,
                                 const void* W_home, const void* W_slots, const int32_t* cu_seqlens, void* Yp,
                                 void* workspace, moonep_stream stream) {
  return group_gemm_launch<false>("moonep_group_gemm", d, H, Hp, t, Xp, W_home, W_slots, cu_seqlens, Yp, workspace,
                                  stream);
}

extern "C" int moonep_group_gemm_dgrad(moonep_dims d, int32_t H, int32_t Hp, moonep_dtype t, const void* dYp,
                                       const void* W_home, const void* W_slots, const int32_t* cu_seqlens, void* dXp,
                                       void* workspace, moonep_stream stream) {
  return group_gemm_launch<true>("moonep_group_gemm_dgrad", d, H, Hp, t, dYp, W_home, W_slots, cu_seqlens, dXp,
                                 workspace, stream);
}
