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
// tile is 256 (H) x 256 (H'), reduced over 32-row chunks of the job's rows with
// MFMA 32x32x16 bf16 by eight waves; both operands reduce along token rows, so
// both are read from LDS with ds_read_b64_tr_b16.  A job without rows writes
// nothing.  The float32 read-modify-write of dW goes through LDS so it moves
// whole 16-byte row chunks.  float32 inputs, and bf16 shapes that kernel does not
// tile (H % 128 or H' % 64 != 0), take wgrad_generic: 64 x 64 output tiles per
// block, 16-row chunks staged as float32 in LDS, four waves of 32 x 32 reducing
// with v_mfma_f32_32x32x2_f32.
#include "block_scan.h"
#include "mfma_tile.h"
#include "moonep_common.h"

namespace moonep {
namespace {

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

// Work list of the MFMA kernel, in the workspace (int32 words; J = E + R*B jobs):
//   [0]                       n, the number of jobs that have rows
//   [32 * (1 + x)]            next unclaimed unit of queue x, x = 0..7 (one 128-byte line each)
//   [kSchedHdr + p]           job at position p of the size order (p < n)
//   [kSchedHdr + J + p]       its number of 32-row chunks
//   [kSchedHdr + 2J + job]    chunk count of every job (scratch)
//   [zero_row_word(J) ...]    512 zero bytes (128 words, 256-byte aligned): the source of the rows
//                             past a segment's end, which must add nothing
constexpr int kQueues = 8, kSchedHdr = 32 * (1 + kQueues), kBuckets = 512;
__host__ __device__ constexpr int64_t zero_row_word(int64_t J) { return (kSchedHdr + 3 * J + 63) / 64 * 64; }

// 32-row chunks of a job: each contributing rank's segment rounded up, as the kernel walks them.
__device__ __forceinline__ int job_chunks(const int32_t* cu, int job, int R, int E, int B) {
  const int G1 = E + B + 1;
  if (job < E) {
    int c = 0;
    for (int r = 0; r < R; ++r) c += (max(0, cu[(int64_t)r * G1 + job + 1] - cu[(int64_t)r * G1 + job]) + 31) >> 5;
    return c;
  }
  const int sj = job - E, r = sj / B, col = E + sj % B;
  return (max(0, cu[(int64_t)r * G1 + col + 1] - cu[(int64_t)r * G1 + col]) + 31) >> 5;
}

// Size class of a job with c >= 1 chunks: 16 classes per octave (the float's exponent and top four
// mantissa bits), numbered so that larger jobs get smaller classes; always in [0, kBuckets).
__device__ __forceinline__ int size_class(int c) {
  return kBuckets - 1 - ((int)(__float_as_uint((float)c) >> 19) - (127 << 4));
}

// One block of 1024: orders the jobs that have rows by size class, larger first, ties by job id
// (a stable counting sort, so the order is deterministic), and clears the queue counters.
__global__ __launch_bounds__(1024) void wgrad_schedule(const int32_t* __restrict__ cu, int R, int E, int B,
                                                       int32_t* __restrict__ ws) {
  __shared__ int32_t off[kBuckets];
  __shared__ int32_t wsum[16];
  const int J = E + R * B, t = threadIdx.x, w = t >> 6, nw = blockDim.x >> 6;
  int32_t* sorted_job = ws + kSchedHdr;
  int32_t* sorted_chunks = sorted_job + J;
  int32_t* chunks = sorted_chunks + J;
  for (int i = t; i < kBuckets; i += blockDim.x) off[i] = 0;
  __syncthreads();
  for (int j = t; j < J; j += blockDim.x) {  // thread t handles jobs t, t + 1024, ... in both passes
    const int c = job_chunks(cu, j, R, E, B);
    chunks[j] = c;
    if (c > 0) atomicAdd(&off[size_class(c)], 1);
  }
  __syncthreads();
  const int n = block_excl_scan(off, kBuckets, wsum);
  for (int i0 = 0; i0 < J; i0 += blockDim.x) {
    const int j = i0 + t;
    const int c = j < J ? chunks[j] : 0;
    const int b = c > 0 ? size_class(c) : -1;
    // rank among the lanes of this wave in the same class, and the size of that group
    int before = 0, group = 0;
    uint64_t todo = __ballot(b >= 0);
    while (todo) {
      const int bl = __shfl(b, __builtin_ctzll(todo), 64);
      const uint64_t m = __ballot(b == bl);
      if (b == bl) {
        before = __popcll(m & lanemask_lt());
        group = __popcll(m);
      }
      todo &= ~m;
    }
    for (int ww = 0; ww < nw; ++ww) {  // waves in order keep equal classes in job order
      if (w == ww && b >= 0) {
        const int pos = off[b] + before;
        sorted_job[pos] = j;
        sorted_chunks[pos] = c;
        if (before == 0) off[b] = pos + group;
      }
      __syncthreads();
    }
  }
  if (t == 0) ws[0] = n;
  if (t < kQueues) ws[32 * (1 + t)] = 0;
  if (t < 128) ws[zero_row_word(J) + t] = 0;
}

namespace wg {
constexpr int BH = 256, BN = 256, BK = 32, STAGES = 4, NWAVES = 8;
constexpr int kMaxRanks = 4096;             // the MFMA kernel's limit on R (one bit per rank in LDS)
constexpr int kMaskWords = kMaxRanks / 64;
constexpr int kLdsRanks = 512;              // ranks whose segment bounds are also kept in LDS

// Walks the row segments of one job like SegWalk, but from a per-unit table in LDS: a bit per rank
// whose segment of this job is non-empty, and the bounds of the first kLdsRanks ranks' segments.
// Inside the chunk loop a compiler-visible global load would make the compiler wait for every
// load the wave has in flight, the DMA of the next chunks included (it cannot count the DMA
// issued from asm); the table keeps the walk off global memory there for R <= kLdsRanks.
struct LdsWalk {
  const int32_t* cu;
  const uint64_t* mask;
  const int32_t *lo, *hi;
  int G1, P, col;
  int r, r_end;  // current rank, one past the last rank
  int m, end;    // current row and end of the current segment (global rows)

  __device__ bool seek(int from) {
    from = __builtin_amdgcn_readfirstlane(from);  // uniform, so the walk branches on scalars
    const int nwords = (r_end + 63) >> 6;
    for (int wi = from >> 6; wi < nwords; ++wi) {
      uint64_t bits = mask[wi];
      bits = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(bits >> 32)) << 32) |
             (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)bits);
      if (wi == (from >> 6)) bits &= ~uint64_t(0) << (from & 63);
      if (bits) {
        r = __builtin_amdgcn_readfirstlane((wi << 6) + __builtin_ctzll(bits));
        if (r >= r_end) break;
        if (r < kLdsRanks) {
          m = __builtin_amdgcn_readfirstlane(lo[r]);
          end = __builtin_amdgcn_readfirstlane(hi[r]);
        } else {
          m = r * P + cu[(int64_t)r * G1 + col];
          end = r * P + cu[(int64_t)r * G1 + col + 1];
        }
        return true;
      }
    }
    r = r_end;
    return false;
  }
  __device__ bool next(int step) {
    m += step;
    if (m < end) return true;
    return seek(r + 1);
  }
};
constexpr int X_STAGE = BK * BH;  // 32 token rows x 256 h; 64-byte blocks XOR-swizzled by row
constexpr int D_STAGE = BK * BN;  // 32 token rows x 256 n; same layout
constexpr int STAGE = X_STAGE + D_STAGE;
constexpr int WN = 64, TM = 4, TN = 2, KK = BK / 16;
constexpr int SP = WN + 4;  // float32 epilogue staging pitch (floats)
constexpr int LDS_ELEMS = STAGES * STAGE;
static_assert(NWAVES * 32 * SP * 2 <= LDS_ELEMS, "epilogue staging must fit in the ring");

__device__ __forceinline__ int blk_off(int k, int n) { return k * 256 + ((((n >> 5) ^ (k & 3)) << 5) | (n & 31)); }

__device__ __forceinline__ bf16x8 operand_rows(const uint16_t* T, int k0, int c0, int lane) {
  const int grp = lane >> 4, c = lane & 15;
  const int col = c0 + 16 * (grp & 1) + 4 * (c & 3);
  const int row = k0 + 8 * (grp >> 1) + (c >> 2);
  const bf16x4 lo = lds_tr4(T + blk_off(row, col));
  const bf16x4 hi = lds_tr4(T + blk_off(row + 4, col));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Persistent: one block of 512 per CU.  A unit is one output tile of one job; the jobs, larger
// first, are dealt to 8 queues in snake order (queue slot q of queue x holds sorted position
// 8q + x for even q, 8q + 7 - x for odd q) and a job's tiles follow one another in its queue.
// Block b drains queue b % 8 first -- workgroups are dealt to the 8 XCDs round-robin, so that is
// its own XCD's queue and a job's tiles share its rows in one L2 -- then takes what is left in
// the other queues.  Units are claimed with an atomic counter per queue, so every unit runs
// exactly once and every block stops once all 8 queues are empty.  Eight waves of 128 (h) x 64
// (n); both operands stream global -> LDS with global_load_lds_dwordx4 into a 4-stage ring of
// 32-row chunks and are read with ds_read_b64_tr_b16 (the reduction runs along token rows).
__global__ __launch_bounds__(512, 1) void wgrad_bf16(const uint16_t* __restrict__ Xp, const uint16_t* __restrict__ dY,
                                                     const int32_t* __restrict__ cu, int32_t* ws,
                                                     float* __restrict__ dW_home, float* __restrict__ dW_slots, int R,
                                                     int E, int B, int P, int H, int Hp) {
  __shared__ __attribute__((aligned(1024))) uint16_t lds[LDS_ELEMS];
  __shared__ int32_t s_unit[2];
  __shared__ uint64_t s_mask[kMaskWords];           // this unit's job: ranks with a non-empty segment
  __shared__ int32_t s_lo[kLdsRanks], s_hi[kLdsRanks];  // their global row bounds (ranks < kLdsRanks)
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w >> 2, wn = w & 3;
  const int HT = (H + BH - 1) / BH, NT = (Hp + BN - 1) / BN;  // H % 128 == 0, H' % 64 == 0
  const int per_job = HT * NT;
  const int J = E + R * B;
  const int n = ws[0];
  const int32_t* sorted_job = ws + kSchedHdr;
  const int32_t* sorted_chunks = sorted_job + J;
  const int home_q = blockIdx.x % kQueues;
  // rows past a segment's end are loaded from the workspace's zero row (addressed from a kernel
  // argument: a global symbol's address would be reloaded from memory at every DMA issue, and that
  // scalar load's wait would also wait for the wave's LDS reads in flight)
  const uint16_t* zero_row = reinterpret_cast<const uint16_t*>(ws + zero_row_word(J));
  const uint32_t lds0 = lds_addr(lds);                            // LDS byte address of the ring
  const int wu = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index, uniform
  int qd = 0;  // thread 0: queues home_q .. home_q + qd - 1 (mod 8) are known to be empty

  for (;;) {
    if (t == 0) {
      int pos = -1, tile = 0;
      for (; qd < kQueues; ++qd) {
        const int x = (home_q + qd) % kQueues;
        const int u = atomicAdd(ws + 32 * (1 + x), 1);
        const int q = u / per_job;
        const int pp = 8 * q + ((q & 1) ? kQueues - 1 - x : x);
        if (pp < n) {  // positions grow with u, so a queue that once came up empty stays empty
          pos = pp;
          tile = u % per_job;
          break;
        }
      }
      s_unit[0] = pos;
      s_unit[1] = tile;
    }
    __syncthreads();
    const int pos = s_unit[0], tile = s_unit[1];
    if (pos < 0) break;  // uniform: every thread read the same s_unit
    const int job = __builtin_amdgcn_readfirstlane(sorted_job[pos]);
    const int nchunks = __builtin_amdgcn_readfirstlane(sorted_chunks[pos]);
    const int col = job < E ? job : E + (job - E) % B;
    const int only = job < E ? -1 : (job - E) / B;  // a slot job reads one rank's group
    for (int r0 = 0; r0 < R; r0 += 512) {
      const int r = r0 + t;
      int a = 0, b = 0;
      if (r < R && (only < 0 || r == only)) {
        a = cu[(int64_t)r * (E + B + 1) + col];
        b = cu[(int64_t)r * (E + B + 1) + col + 1];
      }
      const uint64_t bits = __ballot(b > a);
      if (lane == 0 && (r0 >> 6) + w < ((R + 63) >> 6)) s_mask[(r0 >> 6) + w] = bits;
      if (r < kLdsRanks) {
        s_lo[r] = r * P + a;
        s_hi[r] = r * P + b;
      }
    }
    __syncthreads();  // the walk table is complete, and every wave holds the unit before thread 0 may
                      // claim the next one
    const int h0 = (tile / NT) * BH, n0 = (tile % NT) * BN;
    const int width = min(BN, Hp - n0);
    // a partial tile (H % 256 or H' % 256 != 0) leaves whole 128-row or 64-column wave strips idle;
    // they still issue their share of the DMA and take every barrier
    const bool wave_cols = wn * WN < width && wm * 128 < min(BH, H - h0);
    float* out = job < E ? dW_home + (int64_t)job * H * Hp : dW_slots + (int64_t)(job - E) * H * Hp;

    // DMA slices: instruction j = 2w+i fills rows 2j, 2j+1 of the X stage, then of the D stage
    const int r_l = lane >> 5, s_l = lane & 31;
    int src_row[2], x_col[2], d_col[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      src_row[i] = (2 * w + i) * 2 + r_l;
      const int q = (s_l >> 2) ^ (src_row[i] & 3);
      x_col[i] = (q * 4 + (s_l & 3)) * 8;
      d_col[i] = x_col[i];
    }
    LdsWalk walk;
    walk.cu = cu;
    walk.mask = s_mask;
    walk.lo = s_lo;
    walk.hi = s_hi;
    walk.G1 = E + B + 1;
    walk.P = P;
    walk.col = col;
    walk.r_end = only < 0 ? R : only + 1;
    walk.m = walk.end = 0;
    walk.seek(only < 0 ? 0 : only);
    int issued = 0;
    auto issue_next = [&]() {  // DMA of chunk `issued` into its ring slot, then advance the walker
      const uint32_t st = lds0 + (uint32_t)((issued % STAGES) * STAGE * 2 + wu * 2 * 1024);  // + (2w + i) KB
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = walk.m + src_row[i];
        const bool ok = row < walk.end;
        const uint16_t* xs = ok ? Xp + (int64_t)row * H + min(h0 + x_col[i], H - 8) : zero_row + x_col[i];
        const int dc = min(n0 + d_col[i], Hp - 8);
        const uint16_t* ds = ok ? dY + (int64_t)row * Hp + dc : zero_row + d_col[i];
        dma16(xs, st + i * 1024);
        dma16(ds, st + X_STAGE * 2 + i * 1024);
      }
      ++issued;
      walk.next(BK);
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = (f32x16)(0.f);

    for (int st = 0; st < STAGES - 1 && st < nchunks; ++st) issue_next();
    // Ping-pong, as in the forward group GEMM: waves 0-3 and 4-7 (one of each per SIMD) alternate
    // half a chunk apart between a memory phase (one chunk's operands LDS -> registers, plus this
    // wave's share of the DMA three chunks ahead) and a compute phase (that chunk's 16 MFMAs).
    // Phase q opens with a barrier; A: memory(t) in phase 2t, compute(t) in 2t+1; B: memory(t) in
    // 2t+1, compute(t) in 2t+2.  memory(t) refills the slot of chunk t-1, which B read in 2t-1.
    const int KT = nchunks;
    bf16x8 fa[KK][TM], fb[KK][TN];
    auto mem = [&](int t) {
      const uint16_t* Xs = lds + (t % STAGES) * STAGE;
      const uint16_t* Ds = Xs + X_STAGE;
      if (wave_cols) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
          for (int j = 0; j < TN; ++j) fb[kk][j] = operand_rows(Ds, kk * 16, wn * WN + j * 32, lane);
#pragma unroll
          for (int i = 0; i < TM; ++i) fa[kk][i] = operand_rows(Xs, kk * 16, wm * 128 + i * 32, lane);
        }
      }
      if (issued < nchunks) issue_next();
    };
    auto comp = [&]() {
      if (wave_cols) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(fa[kk][i], fb[kk][j], acc[i][j]);
      }
    };
    // barrier opening phase 2t: this wave has issued chunks up to min(t + 2, KT - 1); waiting until
    // only the later ones are in flight means its share of chunk t has landed, and the barrier
    // extends that to every wave's share
    auto even_barrier = [&](int t) {
      if (t + 2 < KT) wait_vmcnt<8>();
      else if (t + 1 < KT) wait_vmcnt<4>();
      else wait_vmcnt<0>();
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
    lds_barrier();

    // epilogue, one 32-row strip at a time: stage the float32 strip in this wave's LDS region, then
    // dW += strip with 16-byte read-modify-writes of whole row chunks
    float* stage = reinterpret_cast<float*>(lds) + w * 32 * SP;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      if (wave_cols) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) stage[acc_row(v, lane) * SP + j * 32 + (lane & 31)] = acc[i][j][v];
      }
      __syncthreads();
      if (wave_cols) {
        // all eight 16-byte reads of this wave's part of the strip are issued before any write,
        // so they are in flight together instead of one read-modify-write round trip at a time
        constexpr int CPR = WN / 4, NQ = 32 * CPR / 64;
        f32x4* p[NQ];
        f32x4 v[NQ];
#pragma unroll
        for (int u = 0; u < NQ; ++u) {
          const int q = lane + 64 * u, rr = q / CPR, cc = q % CPR;
          p[u] = reinterpret_cast<f32x4*>(out + (int64_t)(h0 + wm * 128 + i * 32 + rr) * Hp + n0 + wn * WN + cc * 4);
          v[u] = *p[u];
        }
#pragma unroll
        for (int u = 0; u < NQ; ++u) {
          const int q = lane + 64 * u, rr = q / CPR, cc = q % CPR;
          const f32x4 s = *reinterpret_cast<const f32x4*>(stage + rr * SP + cc * 4);
          v[u][0] = v[u][0] + s[0];
          v[u][1] = v[u][1] + s[1];
          v[u][2] = v[u][2] + s[2];
          v[u][3] = v[u][3] + s[3];
          *p[u] = v[u];
        }
      }
      __syncthreads();
    }
  }
}
}  // namespace wg

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
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;  // 2 x 2 waves of 32 x 32
  const int HT = (H + kGenBH - 1) / kGenBH, NT = (Hp + kGenBN - 1) / kGenBN;
  const int job = blockIdx.x / (HT * NT), rem = blockIdx.x % (HT * NT);
  const int h0 = (rem / NT) * kGenBH, n0 = (rem % NT) * kGenBN;
  SegWalk walk = make_walk(cu, job, R, E, B, P);
  if (!walk.seek(walk.r)) return;
  float* out = job < E ? dW_home + (int64_t)job * H * Hp : dW_slots + (int64_t)(job - E) * H * Hp;
  f32x16 acc = (f32x16)(0.f);
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
    for (int k = 0; k < kGenBK; k += 2)
      acc = mfma32_f32(Xs[k + (lane >> 5)][wm * 32 + (lane & 31)], Ds[k + (lane >> 5)][wn * 32 + (lane & 31)], acc);
    __syncthreads();
  } while (walk.next(kGenBK));
  const int n = n0 + wn * 32 + (lane & 31);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int h = h0 + wm * 32 + acc_row(v, lane);
    if (h < H && n < Hp) {
      float* p = out + (int64_t)h * Hp + n;
      *p = *p + acc[v];
    }
  }
}

}  // namespace
}  // namespace moonep

using namespace moonep;

extern "C" size_t moonep_wgrad_workspace_bytes(moonep_dims d) {
  if (check_dims(d, "moonep_wgrad_workspace_bytes") != MOONEP_OK) return 0;
  const size_t jobs = (size_t)d.E + (size_t)d.R * d.B;
  return (((size_t)zero_row_word((int64_t)jobs) + 128) * sizeof(int32_t) + 255) & ~size_t(255);
}

extern "C" int moonep_wgrad(moonep_dims d, int32_t H, int32_t Hp, moonep_dtype t, const void* Xp, const void* dY,
                            const int32_t* cu_seqlens, float* dW_home, float* dW_slots, void* workspace,
                            moonep_stream stream) {
  if (int rc = check_dims(d, "moonep_wgrad")) return rc;
  MOONEP_REQUIRE(t == MOONEP_F32 || t == MOONEP_BF16, "moonep_wgrad: bad dtype %d", (int)t);
  MOONEP_REQUIRE(H >= 1 && Hp >= 1, "moonep_wgrad: H and Hp must be >= 1");
  if (n_pairs(d) == 0) return MOONEP_OK;
  MOONEP_REQUIRE(Xp && dY && cu_seqlens && dW_home && workspace, "moonep_wgrad: null pointer");
  MOONEP_REQUIRE(d.B == 0 || dW_slots, "moonep_wgrad: dW_slots is null with B > 0");
  MOONEP_REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, "moonep_wgrad: workspace must be 256-byte aligned");
  hipStream_t s = as_stream(stream);
  clear_stale_error();
  const int64_t jobs = (int64_t)d.E + (int64_t)d.R * d.B;
  MOONEP_REQUIRE(jobs < (int64_t(1) << 28), "moonep_wgrad: too many jobs");
  const int P = d.S * d.K;
  const bool mfma = t == MOONEP_BF16 && H % 128 == 0 && Hp % 64 == 0 && d.R <= wg::kMaxRanks && aligned16(Xp) &&
                    aligned16(dY) && aligned16(dW_home) && (d.B == 0 || aligned16(dW_slots));
  if (mfma) {
    const int cus = device_cu_count();
    const int64_t units = jobs * ((H + wg::BH - 1) / wg::BH) * ((Hp + wg::BN - 1) / wg::BN);
    MOONEP_REQUIRE(units + 8 * (int64_t)cus < (int64_t(1) << 30), "moonep_wgrad: too many output tiles");
    int32_t* ws = static_cast<int32_t*>(workspace);
    hipLaunchKernelGGL(wgrad_schedule, dim3(1), dim3(1024), 0, s, cu_seqlens, d.R, d.E, d.B, ws);
    MOONEP_LAUNCH_CHECK("moonep_wgrad/schedule");
    const auto* x = static_cast<const uint16_t*>(Xp);
    const auto* dy = static_cast<const uint16_t*>(dY);
    hipLaunchKernelGGL(wg::wgrad_bf16, dim3((unsigned)cus), dim3(512), 0, s, x, dy, cu_seqlens, ws,
                       dW_home, dW_slots, d.R, d.E, d.B, P, H, Hp);
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
