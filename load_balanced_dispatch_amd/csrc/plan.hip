// moonep_plan: expert histogram, maxvio and the home-first prefix-sum plan on gfx950.
//
// What is computed ([P2] = "Moonshot open-sources MoonEP: an expert-parallel
// communication library for MoE training", umios.umi6.com):
//   * maxvio = max_e(T_e / Tbar) - 1 ([P2] "Core problem").
//   * every rank receives exactly P = S*K pairs ([P2] "Core technique"): rank r
//     keeps the first P pairs of its home experts' (expert, src, token, k)-ordered
//     list; the overflow of all ranks, in ascending (expert, order), is cut
//     contiguously into the deficits of the underloaded ranks in rank order.
//     The fewest-copies planner differs only in the keep counts: an overloaded
//     rank's excess leaves through its largest experts (the pages' planner keeps
//     the number of redundant experts small; its program is not printed).
//   * arriving experts take slots E+j (j < B), beyond that they read their home
//     row; cu_seqlens delimits the E+B groups ([P2] "Memory contract and weight
//     layout").
//
// Kernels (all on the caller's stream, no host synchronisation):
//   plan_count  grid = U blocks of TPB whole tokens: LDS histogram of the block's
//               pairs, invalid / repeated ids counted.
//   plan_scan   column-wise exclusive scan of the U x E block histograms (64
//               experts per block, 16 waves split the U rows), totals = T_e.
//   plan_solve  one 1024-thread block: keep counts (home-first prefix, or the
//               fewest-copies choice of overflowing experts), overflow/deficit
//               prefix sums, slot assignment, cu_seqlens, stats, maxvio.
//               O(E + R + R*(E+B)), plus O(E*E/R) for the fewest-copies keep;
//               a handful of block-wide scans, each a few DPP steps per wave.
//   plan_emit   grid = U: stable rank of every pair inside its expert (wave
//               ballot match + per-wave LDS counters, tiles processed in order),
//               then its destination row.
#include <algorithm>
#include <mutex>

#include "block_scan.h"
#include "moonep_common.h"

namespace moonep {
namespace {

constexpr int kCountThreads = 256;
constexpr int kSolveThreads = 1024;
// pairs per count/emit block: 1024 gives the mid workload (196608 pairs) 192 blocks; measured
// against 512, 2048 and 4096, it was fastest there (36 us for the whole plan, 60 us at 4096) and
// within 4% of the best on a 1M-pair routing workload
constexpr int kPairsPerBlock = 1024;
constexpr int kMaxExperts = 4096;
constexpr int64_t kPlanMaxDynLds = 160 * 1024 - 2048;  // LDS per block left for the dynamic tables
constexpr int kMaxRanks = 4096;

struct PlanGeom {
  int64_t tokens;  // R*S
  int tpb;         // whole tokens per count/emit block
  int units;       // number of count/emit blocks
};

PlanGeom plan_geom(const moonep_dims& d) {
  PlanGeom g;
  g.tokens = (int64_t)d.R * d.S;
  g.tpb = kPairsPerBlock / d.K > 0 ? kPairsPerBlock / d.K : 1;
  g.units = (int)((g.tokens + g.tpb - 1) / g.tpb);
  return g;
}

struct PlanWs {
  int32_t* cnt;      // [U, E]  block histograms, then exclusive bases
  int32_t* err;      // [U]
  int32_t* keep;     // [E]
  int32_t* ovstart;  // [E]
  int32_t* npos;     // [E]  experts with overflow before e
  int32_t* defstart; // [R]
  int32_t* defend;   // [R]
  int32_t* efirst;   // [R]  first expert cut into rank d
  size_t bytes;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

PlanWs plan_ws(const moonep_dims& d, void* base) {
  PlanGeom g = plan_geom(d);
  char* p = static_cast<char*>(base);
  size_t off = 0;
  PlanWs w;
  auto take = [&](size_t n_ints) {
    int32_t* q = reinterpret_cast<int32_t*>(p ? p + off : nullptr);
    off = align256(off + n_ints * sizeof(int32_t));
    return q;
  };
  w.cnt = take((size_t)g.units * d.E);
  w.err = take((size_t)g.units + 1);
  w.keep = take(d.E);
  w.ovstart = take(d.E);
  w.npos = take(d.E);
  w.defstart = take(d.R);
  w.defend = take(d.R);
  w.efirst = take(d.R);
  w.bytes = off;
  return w;
}

// ------------------------------------------------------------------ plan_count

__global__ __launch_bounds__(kCountThreads) void plan_count(const int32_t* __restrict__ ids, int E, int K,
                                                           int64_t tokens, int tpb, int32_t* __restrict__ cnt,
                                                           int32_t* __restrict__ err) {
  extern __shared__ int32_t sh[];
  int32_t* hist = sh;      // [E]
  int32_t* sid = sh + E;   // [tpb*K]
  __shared__ int32_t werr[kCountThreads / 64];
  const int u = blockIdx.x;
  const int64_t tok0 = (int64_t)u * tpb;
  const int ntok = (int)min<int64_t>(tpb, tokens - tok0);
  const int np = ntok * K;
  const int64_t base = tok0 * K;
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  for (int i = threadIdx.x; i < np; i += blockDim.x) sid[i] = ids[base + i];
  __syncthreads();
  int bad = 0;
  for (int i = threadIdx.x; i < np; i += blockDim.x) {
    const int v = sid[i];
    if (v >= 0 && v < E) {
      atomicAdd(&hist[v], 1);
      const int t0 = i - i % K;
      for (int j = t0; j < i; ++j)
        if (sid[j] == v) { ++bad; break; }  // repeated expert within one token
    } else {
      ++bad;
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[(int64_t)u * E + e] = hist[e];
  bad = wave_sum(bad);
  if (__lane_id() == 0) werr[threadIdx.x >> 6] = bad;
  __syncthreads();
  if (threadIdx.x == 0) {
    int s = 0;
    for (int w = 0; w < kCountThreads / 64; ++w) s += werr[w];
    err[u] = s;
  }
}

// ------------------------------------------------------------------ plan_scan

constexpr int kScanWaves = 16;

__global__ __launch_bounds__(kScanWaves * 64) void plan_scan(int32_t* __restrict__ cnt, int U, int E,
                                                            int32_t* __restrict__ counts) {
  __shared__ int32_t seg[kScanWaves][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + lane;
  const int cs = (U + kScanWaves - 1) / kScanWaves;
  const int u0 = min(U, w * cs), u1 = min(U, u0 + cs);
  int s = 0;
  if (e < E) {
#pragma unroll 8  // several rows' loads in flight per lane (measured: stress-routing plan 91 -> 75 us)
    for (int u = u0; u < u1; ++u) s += cnt[(int64_t)u * E + e];
  }
  seg[w][lane] = s;
  __syncthreads();
  int start = 0, total = 0;
  for (int i = 0; i < kScanWaves; ++i) {
    if (i < w) start += seg[i][lane];
    total += seg[i][lane];
  }
  if (e < E) {
    int run = start;
#pragma unroll 8
    for (int u = u0; u < u1; ++u) {
      const int64_t at = (int64_t)u * E + e;
      const int c = cnt[at];
      cnt[at] = run;
      run += c;
    }
    if (w == 0) counts[e] = total;
  }
}

// ------------------------------------------------------------------ plan_solve

__device__ __forceinline__ int overlap(int a0, int a1, int b0, int b1) {
  return max(0, min(a1, b1) - max(a0, b0));
}

__global__ __launch_bounds__(kSolveThreads) void plan_solve(
    int R, int E, int B, int P, int64_t N, int U, int planner, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ err, double* __restrict__ maxvio, int32_t* __restrict__ cu,
    int32_t* __restrict__ slot_expert, int32_t* __restrict__ stats, int32_t* __restrict__ g_keep,
    int32_t* __restrict__ g_ovstart, int32_t* __restrict__ g_npos, int32_t* __restrict__ g_defstart,
    int32_t* __restrict__ g_defend, int32_t* __restrict__ g_efirst) {
  extern __shared__ int32_t sh[];
  int32_t* sT = sh;             // [E]
  int32_t* skeep = sT + E;      // [E]
  int32_t* sover = skeep + E;   // [E]
  int32_t* sovs = sover + E;    // [E] exclusive scan of over
  int32_t* snpos = sovs + E;    // [E] exclusive scan of (over > 0)
  int32_t* sdef = snpos + E;    // [R]
  int32_t* sdefs = sdef + R;    // [R] exclusive scan of def
  int32_t* sefirst = sdefs + R; // [R]
  int32_t* sncopy = sefirst + R;// [R]
  int32_t* solist = sT;         // [E] the overflowing experts, ascending (sT is dead by then)
  __shared__ int32_t wsum[3 * (kSolveThreads / 64)];
  __shared__ int32_t red[3][kSolveThreads / 64];
  const int t = threadIdx.x, nt = blockDim.x, lane = t & 63, w = t >> 6, nw = nt >> 6;
  const int per = E / R;

  // the first count and error word of each thread are loaded together, so that their round trips overlap
  int mx = t < E ? counts[t] : 0, bad = t < U ? err[t] : 0;
  if (t < E) sT[t] = mx;
  for (int e = t + nt; e < E; e += nt) {
    sT[e] = counts[e];
    mx = max(mx, sT[e]);
  }
  for (int u = t + nt; u < U; u += nt) bad += err[u];
  mx = wave_max(mx);
  bad = wave_sum(bad);
  if (lane == 0) {
    red[0][w] = mx;
    red[1][w] = bad;
  }
  __syncthreads();
  if (t == 0) {
    int m = 0, b = 0;
    for (int i = 0; i < nw; ++i) {
      m = max(m, red[0][i]);
      b += red[1][i];
    }
    *maxvio = N > 0 ? (double)((int64_t)E * m) / (double)N - 1.0 : 0.0;
    stats[3] = b;
  }

  // exclusive prefix of T over all experts (a rank's home experts are contiguous), in sovs for now:
  // the pairs routed to rank r's experts before e are pre[e] - pre[r * per], its load
  // pre[(r + 1) * per] - pre[r * per] (the total for the last rank)
  for (int e = t; e < E; e += nt) sovs[e] = sT[e];
  __syncthreads();
  int tot3[3];
  block_excl_scan3(sovs, E, nullptr, 0, nullptr, 0, wsum, tot3);
  const int32_t* pre = sovs;
  const int totT = tot3[0];
  auto rank_load = [&](int r) { return (r + 1 < R ? pre[(r + 1) * per] : totT) - pre[r * per]; };
  if (planner == MOONEP_PLAN_PREFIX) {
    // home-first keep counts: each rank keeps the first P pairs of its experts in ascending order
    for (int e = t; e < E; e += nt) {
      const int before = pre[e] - pre[(e / per) * per];
      const int k = min(max(P - before, 0), sT[e]);
      skeep[e] = k;
      sover[e] = sT[e] - k;
    }
    for (int r = t; r < R; r += nt) sdef[r] = max(0, P - rank_load(r));
  } else {
    // fewest copies: an overloaded rank's excess x leaves through its experts taken largest first
    // (equal counts: lower id first).  Expert e overflows what x still needs after the experts ahead
    // of it in that order, clamped to [0, T_e]; one thread per expert, O(E/R) each.
    for (int r = t; r < R; r += nt) sdef[r] = P - rank_load(r);  // signed for now: minus the excess
    __syncthreads();
    for (int e = t; e < E; e += nt) {
      const int r = e / per, te = sT[e], x = -sdef[r];
      int moved = 0;
      if (x > 0 && te > 0) {
        int ahead = 0;
        for (int f = r * per; f < (r + 1) * per; ++f) {
          const int tf = sT[f];
          ahead += (tf > te || (tf == te && f < e)) ? tf : 0;
        }
        moved = min(max(x - ahead, 0), te);
      }
      skeep[e] = te - moved;
      sover[e] = moved;
    }
    __syncthreads();
    for (int r = t; r < R; r += nt) sdef[r] = max(0, sdef[r]);
  }
  __syncthreads();
  for (int e = t; e < E; e += nt) {
    sovs[e] = sover[e];
    snpos[e] = sover[e] > 0 ? 1 : 0;
  }
  for (int r = t; r < R; r += nt) sdefs[r] = sdef[r];
  __syncthreads();
  block_excl_scan3(sovs, E, snpos, E, sdefs, R, wsum, tot3);

  // contiguous cut.  Deficit rank d's interval [lo, hi) of the overflow list overlaps the experts
  // e in [a, z) with over[e] > 0, where a is the first e with ovstart + over > lo and z the first
  // e >= a with ovstart >= hi (ovstart is non-decreasing); they are its copies, ascending, and the
  // j-th of them is the (npos[a] + j)-th overflowing expert overall.
  for (int e = t; e < E; e += nt)
    if (sover[e] > 0) solist[snpos[e]] = e;
  for (int d = t; d < R; d += nt) {
    int j = 0, ef = 0;
    if (sdef[d] > 0) {
      const int lo = sdefs[d], hi = lo + sdef[d];
      int a = 0, b = E;
      while (a < b) {
        const int m = (a + b) >> 1;
        if (sovs[m] + sover[m] > lo) b = m; else a = m + 1;
      }
      int z = a, y = E;
      while (z < y) {
        const int m = (z + y) >> 1;
        if (sovs[m] >= hi) y = m; else z = m + 1;
      }
      const auto npos_at = [&](int e) { return e < E ? snpos[e] : snpos[E - 1] + (sover[E - 1] > 0); };
      ef = a < E ? a : 0;  // a == E only when invalid ids left the deficits larger than the overflow
      j = npos_at(z) - npos_at(a);
    }
    sefirst[d] = ef;
    sncopy[d] = j;
  }
  __syncthreads();
  for (int i = t; i < R * B; i += nt) {
    const int d = i / B, jj = i % B;
    slot_expert[i] = jj < sncopy[d] ? solist[snpos[sefirst[d]] + jj] : -1;
  }

  // cu_seqlens: one wave per rank, 64 groups at a time
  const int G = E + B;
  for (int d = w; d < R; d += nw) {
    const int d0 = sdefs[d], d1 = d0 + sdef[d];
    const int nf = snpos[sefirst[d]], ncp = sncopy[d];
    int carry = 0;
    if (lane == 0) cu[(int64_t)d * (G + 1)] = 0;
    for (int g0 = 0; g0 < G; g0 += 64) {
      const int g = g0 + lane;
      int c = 0;
      if (g < E) {
        if (g / per == d) {
          c = skeep[g];
        } else if (sover[g] > 0 && d1 > d0) {
          const int f = overlap(sovs[g], sovs[g] + sover[g], d0, d1);
          if (f > 0 && snpos[g] - nf >= B) c = f;  // direct read of home row g
        }
      } else if (g < G) {
        const int jj = g - E;  // slot jj < B of rank d, from the LDS tables (not the global output)
        const int e = jj < ncp ? solist[nf + jj] : -1;
        if (e >= 0) c = overlap(sovs[e], sovs[e] + sover[e], d0, d1);
      }
      const int incl = wave_incl_scan(c);
      if (g < G) cu[(int64_t)d * (G + 1) + g + 1] = carry + incl;
      carry += __shfl(incl, 63, 64);
    }
  }

  // tables for plan_emit, stats
  for (int e = t; e < E; e += nt) {
    g_keep[e] = skeep[e];
    g_ovstart[e] = sovs[e];
    g_npos[e] = snpos[e];
  }
  int cp = 0, sl = 0;
  for (int d = t; d < R; d += nt) {
    g_defstart[d] = sdefs[d];
    g_defend[d] = sdefs[d] + sdef[d];
    g_efirst[d] = sefirst[d];
    cp += sncopy[d];
    sl += min(sncopy[d], B);
  }
  cp = wave_sum(cp);
  sl = wave_sum(sl);
  if (lane == 0) {
    red[0][w] = cp;
    red[2][w] = sl;
  }
  __syncthreads();
  if (t == 0) {
    int a = 0, b = 0;
    for (int i = 0; i < nw; ++i) {
      a += red[0][i];
      b += red[2][i];
    }
    stats[0] = a;
    stats[1] = b;
    stats[2] = a - b;
  }
}

// ------------------------------------------------------------------ plan_emit

constexpr int kEmitThreads = 256;
constexpr int kEmitWaves = kEmitThreads / 64;

__global__ __launch_bounds__(kEmitThreads) void plan_emit(
    const int32_t* __restrict__ ids, int R, int E, int B, int K, int P, int64_t tokens, int tpb,
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ g_keep, const int32_t* __restrict__ g_ovstart,
    const int32_t* __restrict__ g_npos, const int32_t* __restrict__ g_defstart,
    const int32_t* __restrict__ g_defend, const int32_t* __restrict__ g_efirst, const int32_t* __restrict__ cu,
    int32_t* __restrict__ dest_idx, int32_t* __restrict__ src_of_row) {
  extern __shared__ int32_t sh[];
  int32_t* run = sh;                    // [E]  pairs of e seen before the current tile
  int32_t* tcnt = run + E;              // [kEmitWaves][E]
  int32_t* keep = tcnt + kEmitWaves * E;// [E]
  int32_t* ovs = keep + E;              // [E]
  int32_t* npos = ovs + E;              // [E]
  int32_t* defs = npos + E;             // [R]
  int32_t* defe = defs + R;             // [R]
  int32_t* efirst = defe + R;           // [R]
  const int u = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  for (int e = t; e < E; e += blockDim.x) {
    run[e] = cnt[(int64_t)u * E + e];
    keep[e] = g_keep[e];
    ovs[e] = g_ovstart[e];
    npos[e] = g_npos[e];
    for (int i = 0; i < kEmitWaves; ++i) tcnt[i * E + e] = 0;
  }
  for (int r = t; r < R; r += blockDim.x) {
    defs[r] = g_defstart[r];
    defe[r] = g_defend[r];
    efirst[r] = g_efirst[r];
  }
  __syncthreads();
  const int per = E / R, G1 = E + B + 1;
  const int64_t tok0 = (int64_t)u * tpb;
  const int np = (int)min<int64_t>(tpb, tokens - tok0) * K;
  const int64_t base = tok0 * K;
  const int nbits = 32 - __clz(E);  // enough bits for the sentinel value E
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int tile = 0; tile < np; tile += kEmitThreads) {
    const int i = tile + t;
    const bool valid = i < np;
    const int v = valid ? ids[base + i] : -1;
    const bool good = valid && v >= 0 && v < E;
    const int key = good ? v : E;
    uint64_t mask = ~0ull;
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (key >> b) & 1;
      const uint64_t bb = __ballot(bit);
      mask &= bit ? bb : ~bb;
    }
    const int wrank = __popcll(mask & lt);
    const int wcnt = __popcll(mask);
    const bool leader = wrank == 0;
    if (good && leader) tcnt[w * E + key] = wcnt;
    __syncthreads();
    int ord = 0;
    if (good) {
      ord = run[key] + wrank;
      for (int i2 = 0; i2 < w; ++i2) ord += tcnt[i2 * E + key];
    }
    __syncthreads();
    if (good && leader) {
      tcnt[w * E + key] = 0;
      atomicAdd(&run[key], wcnt);
    }
    if (valid) {
      int dst = -1;
      if (good) {
        const int e = key;
        int d, g, pos;
        if (ord < keep[e]) {
          d = e / per;
          g = e;
          pos = ord;
        } else {
          const int vpos = ovs[e] + ord - keep[e];
          int a = 0, b = R;  // first d whose deficit interval ends after vpos
          while (a < b) {
            const int m = (a + b) >> 1;
            if (defe[m] > vpos) b = m; else a = m + 1;
          }
          d = min(a, R - 1);
          const int j = npos[e] - npos[efirst[d]];
          g = j < B ? E + j : e;
          pos = vpos - max(ovs[e], defs[d]);
        }
        dst = d * P + cu[(int64_t)d * G1 + g] + pos;
        if (src_of_row != nullptr) src_of_row[dst] = (int32_t)(base + i);
      }
      dest_idx[base + i] = dst;
    }
  }
}

}  // namespace
}  // namespace moonep

using namespace moonep;

extern "C" size_t moonep_plan_workspace_bytes(moonep_dims d) {
  if (check_dims(d, "moonep_plan_workspace_bytes") != MOONEP_OK) return 0;
  return plan_ws(d, nullptr).bytes;
}

extern "C" int moonep_plan(moonep_dims d, const int32_t* topk_idx, int32_t* expert_counts, double* maxvio,
                           int32_t* cu_seqlens, int32_t* slot_expert, int32_t* dest_idx, int32_t* src_of_row,
                           int32_t* stats, void* workspace, moonep_stream stream) {
  return moonep_plan_ex(d, MOONEP_PLAN_PREFIX, topk_idx, expert_counts, maxvio, cu_seqlens, slot_expert, dest_idx,
                        src_of_row, stats, workspace, stream);
}

extern "C" int moonep_plan_ex(moonep_dims d, int32_t planner, const int32_t* topk_idx, int32_t* expert_counts,
                              double* maxvio, int32_t* cu_seqlens, int32_t* slot_expert, int32_t* dest_idx,
                              int32_t* src_of_row, int32_t* stats, void* workspace, moonep_stream stream) {
  if (int rc = check_dims(d, "moonep_plan")) return rc;
  MOONEP_REQUIRE(planner == MOONEP_PLAN_PREFIX || planner == MOONEP_PLAN_MINCOPY, "moonep_plan: unknown planner %d",
                 (int)planner);
  const int64_t N = n_pairs(d);
  MOONEP_REQUIRE(d.E <= kMaxExperts, "moonep_plan: E=%d exceeds the supported %d", d.E, kMaxExperts);
  MOONEP_REQUIRE(d.R <= kMaxRanks, "moonep_plan: R=%d exceeds the supported %d", d.R, kMaxRanks);
  const PlanGeom geo = plan_geom(d);
  // per-block LDS tables of the three kernels, in ints: count E + tpb*K, solve 5E + 4R, emit
  // (4 + waves)E + 3R; the largest must fit beside the kernels' static arrays
  const int64_t lds_ints = std::max<int64_t>({(int64_t)d.E + (int64_t)geo.tpb * d.K, 5 * (int64_t)d.E + 4 * (int64_t)d.R,
                                              (4 + kEmitWaves) * (int64_t)d.E + 3 * (int64_t)d.R});
  MOONEP_REQUIRE(lds_ints * (int64_t)sizeof(int32_t) <= kPlanMaxDynLds,
                 "moonep_plan: E=%d with R=%d needs %lld bytes of LDS tables per block, more than %lld", d.E, d.R,
                 (long long)(lds_ints * (int64_t)sizeof(int32_t)), (long long)kPlanMaxDynLds);
  MOONEP_REQUIRE(expert_counts && maxvio && cu_seqlens && stats && workspace,
                 "moonep_plan: null output or workspace pointer");
  MOONEP_REQUIRE(d.B == 0 || slot_expert, "moonep_plan: slot_expert is null with B > 0");
  MOONEP_REQUIRE(N == 0 || (topk_idx && dest_idx), "moonep_plan: null topk_idx or dest_idx");
  MOONEP_REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, "moonep_plan: workspace must be 256-byte aligned");
  hipStream_t s = as_stream(stream);
  clear_stale_error();
  const PlanWs ws = plan_ws(d, workspace);
  const int P = d.S * d.K;

  if (geo.units > 0) {
    const size_t lds = (size_t)(d.E + geo.tpb * d.K) * sizeof(int32_t);
    hipLaunchKernelGGL(plan_count, dim3(geo.units), dim3(kCountThreads), lds, s, topk_idx, d.E, d.K,
                       geo.tokens, geo.tpb, ws.cnt, ws.err);
    MOONEP_LAUNCH_CHECK("moonep_plan/count");
  }
  hipLaunchKernelGGL(plan_scan, dim3(ceil_div_u(d.E, 64)), dim3(kScanWaves * 64), 0, s, ws.cnt, geo.units, d.E,
                     expert_counts);
  MOONEP_LAUNCH_CHECK("moonep_plan/scan");
  {
    const size_t lds = (size_t)(5 * d.E + 4 * d.R) * sizeof(int32_t);
    if (lds > 65536)
      (void)hipFuncSetAttribute((const void*)plan_solve, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(plan_solve, dim3(1), dim3(kSolveThreads), lds, s, d.R, d.E, d.B, P, N, geo.units,
                       (int)planner, expert_counts, ws.err, maxvio, cu_seqlens, slot_expert, stats, ws.keep, ws.ovstart, ws.npos,
                       ws.defstart, ws.defend, ws.efirst);
    MOONEP_LAUNCH_CHECK("moonep_plan/solve");
  }
  if (geo.units > 0) {
    const size_t lds = (size_t)((4 + kEmitWaves) * d.E + 3 * d.R) * sizeof(int32_t);
    if (lds > 65536)
      (void)hipFuncSetAttribute((const void*)plan_emit, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(plan_emit, dim3(geo.units), dim3(kEmitThreads), lds, s, topk_idx, d.R, d.E, d.B, d.K, P,
                       geo.tokens, geo.tpb, ws.cnt, ws.keep, ws.ovstart, ws.npos, ws.defstart, ws.defend, ws.efirst,
                       cu_seqlens, dest_idx, src_of_row);
    MOONEP_LAUNCH_CHECK("moonep_plan/emit");
  }
  return MOONEP_OK;
}

// ------------------------------------------------------------------ allocation-free planning

namespace {

// Scratch of moonep_plan_static: the planner's workspace in a device array the library owns.  Every GPU
// the library runs on holds its own copy (a __device__ variable exists once per device) until the
// process ends.  Host code never passes `scratch` itself to a kernel -- in host code the name is a
// host-side stand-in -- but the device address hipGetSymbolAddress returns for the current device.
constexpr size_t kStaticScratchBytes = size_t(8) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array, looked up once per device (with that device
// current); nullptr and a message on failure.
void* static_scratch() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    moonep::set_error("moonep_plan_static: no usable current device (%s)", hipGetErrorString(e));
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      moonep::set_error("moonep_plan_static: hipGetSymbolAddress of the scratch array failed on device %d: %s", dev,
                        hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" size_t moonep_plan_static_scratch_bytes(void) { return kStaticScratchBytes; }

extern "C" int moonep_plan_static(moonep_dims d, int32_t planner, const int32_t* topk_idx, int32_t* expert_counts,
                                  double* maxvio, int32_t* cu_seqlens, int32_t* slot_expert, int32_t* dest_idx,
                                  int32_t* src_of_row, int32_t* stats, moonep_stream stream) {
  if (int rc = check_dims(d, "moonep_plan_static")) return rc;
  const size_t need = plan_ws(d, nullptr).bytes;
  MOONEP_REQUIRE(need <= kStaticScratchBytes,
                 "moonep_plan_static: these dims need %zu bytes of planner scratch, more than the %zu bytes the "
                 "library holds per GPU; use moonep_plan_ex with a workspace",
                 need, kStaticScratchBytes);
  // the pointer checks of moonep_plan_ex come first, so a bad call touches no device state
  MOONEP_REQUIRE(expert_counts && maxvio && cu_seqlens && stats, "moonep_plan_static: null output pointer");
  MOONEP_REQUIRE(d.B == 0 || slot_expert, "moonep_plan_static: slot_expert is null with B > 0");
  MOONEP_REQUIRE(n_pairs(d) == 0 || (topk_idx && dest_idx), "moonep_plan_static: null topk_idx or dest_idx");
  void* ws = static_scratch();
  if (ws == nullptr) return MOONEP_EHIP;
  // every planner kernel writes its part of the workspace before reading it: nothing needs clearing
  return moonep_plan_ex(d, planner, topk_idx, expert_counts, maxvio, cu_seqlens, slot_expert, dest_idx, src_of_row,
                        stats, ws, stream);
}
