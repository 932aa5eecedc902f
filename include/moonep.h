/*
 * moonep.h -- C ABI of the balanced expert-parallel MoE layer on one MI355X (gfx950).
 *
 * R virtual expert-parallel ranks live in one GPU's HBM.  The library plans,
 * from top-K router output, how many pairs each rank processes so that every
 * rank handles exactly S*K (token, expert) pairs, then moves rows and runs the
 * expert GEMMs under that plan.
 *
 * Sources (web pages about MoonEP; a section name follows each citation):
 *   [P1] "Valhalla static engineering review #004 -- MoonshotAI MoonEP"
 *        (wsisp.com), section 2 "Project background".
 *   [P2] "Moonshot open-sources MoonEP: an expert-parallel communication
 *        library for MoE training" (umios.umi6.com), sections "Core problem",
 *        "Core technique: dynamic redundant experts", "Memory contract and
 *        weight layout".
 *   [P3] "Moonshot AI Open-Sources MoonEP for Expert Parallelism"
 *        (interestana.com), paragraphs two (maxvio) and three (S*K invariant).
 *
 * Notation ([P2] "Memory contract and weight layout"): E routed experts, E/R
 * home experts per rank (expert e lives on rank e / (E/R)), B prefetch slots
 * per rank, S tokens per rank, K experts per token, H hidden size, Hp = H'
 * FFN width.  P = S*K rows per rank, N = R*P rows in total.  Rank r sees a
 * logical [E+B, H, Hp] weight tensor: row g < E is W_home[g], row E+j is its
 * slot W_slots[r, j].
 *
 * Conventions shared by every call
 *   - All array pointers are DEVICE memory owned by the caller, dense and
 *     row-major with the shapes given.  The library never allocates, frees,
 *     copies to the host or synchronises: each call only enqueues kernels on
 *     `stream` (a hipStream_t; NULL is the null stream), so a call sequence
 *     can be captured in a HIP graph.
 *   - Shapes are static: no output size depends on the routing.
 *   - Return value: MOONEP_OK, or a negative code.  MOONEP_EINVAL (bad
 *     dimension, null pointer, misaligned pointer) and MOONEP_EUNSUPPORTED
 *     are returned before anything is enqueued.  MOONEP_EHIP means a launch
 *     failed; the device state of the outputs is then unspecified.
 *     moonep_last_error() gives a human-readable reason for the calling thread.
 *   - Device-side contract violations are never trapped: top-K ids outside
 *     [0, E) and a repeated expert within one token are counted in
 *     stats[3] by moonep_plan; other results are then unspecified (but every
 *     kernel stays inside its buffers).
 *   - Row pointers whose rows are a multiple of 16 bytes must be 16-byte
 *     aligned (checked).
 */
#ifndef MOONEP_H
#define MOONEP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moonep_dims {
  int32_t R; /* virtual ranks, >= 1 */
  int32_t E; /* routed experts, >= 1, E % R == 0 */
  int32_t B; /* prefetch slots per rank, >= 0 (training uses E/R, inference 3-4) */
  int32_t S; /* tokens per rank, >= 0 */
  int32_t K; /* experts per token, 1 <= K <= E; R*S*K < 2^31 */
} moonep_dims;

typedef enum moonep_dtype {
  MOONEP_F32 = 0, /* float32 activations and weights */
  MOONEP_BF16 = 1 /* bfloat16 activations and weights, float32 accumulation */
} moonep_dtype;

enum {
  MOONEP_OK = 0,
  MOONEP_EINVAL = -1,
  MOONEP_EHIP = -2,
  MOONEP_EUNSUPPORTED = -3
};

typedef void* moonep_stream; /* a hipStream_t */

/* Text of the last error raised on the calling thread ("" when none). */
const char* moonep_last_error(void);

/* Planners of moonep_plan_ex. */
typedef enum moonep_planner {
  MOONEP_PLAN_PREFIX = 0, /* home-first prefix: each rank keeps the first S*K pairs of its home experts */
  MOONEP_PLAN_MINCOPY = 1 /* fewest copies: an overloaded rank's excess leaves through its largest experts */
} moonep_planner;

/* Bytes of device workspace moonep_plan needs for these dims (256-byte aligned pointer). */
size_t moonep_plan_workspace_bytes(moonep_dims d);

/*
 * moonep_plan -- histogram, maxvio and the home-first prefix-sum plan.
 *   maxvio = max_e(T_e / Tbar) - 1, Tbar = N / E ([P2] "Core problem"; [P3]
 *   paragraph two), evaluated as (double)(E * max_e T_e) / (double)N - 1.0
 *   (0.0 when N == 0).  Every rank then receives exactly P = S*K pairs
 *   ([P1] section 2; [P2] "Core technique"; [P3] paragraph three): rank r keeps
 *   the first P pairs of its home experts' pairs taken in (expert, src rank,
 *   token, k) order; the rest, in ascending (expert, order), are cut
 *   contiguously into the deficits P - L_r of the underloaded ranks in rank
 *   order.  On a receiving rank the arriving experts, in ascending order, take
 *   slots j = 0..B-1 (group E+j); beyond B they are read from their home row
 *   (group e) ([P2] "Memory contract and weight layout").
 * In:  topk_idx [R,S,K] int32 expert ids, pair (r,s,k) is flat id (r*S+s)*K+k.
 * Out: expert_counts [E]        int32  T_e.
 *      maxvio        [1]        double.
 *      cu_seqlens    [R,E+B+1]  int32  rank r's group g occupies local rows
 *                                      [cu[r,g], cu[r,g+1]); cu[r,0]=0, cu[r,E+B]=P.
 *      slot_expert   [R,B]      int32  expert held by slot j of rank r, -1 unused
 *                                      (may be NULL when B == 0).
 *      dest_idx      [R,S,K]    int32  global row r'*P + local row of each pair;
 *                                      -1 for an id outside [0,E).
 *      src_of_row    [R*S*K]    int32  inverse of dest_idx (flat pair id per row),
 *                                      or NULL to skip.
 *      stats         [4]        int32  copies (expert, non-home rank) used,
 *                                      of them slotted, of them direct reads,
 *                                      invalid ids + repeated ids within a token.
 * workspace: moonep_plan_workspace_bytes(d) bytes of device memory, contents
 * ignored on entry.
 * Limits (MOONEP_EINVAL beyond them): E <= 4096, R <= 4096, and each planner
 * block keeps per-expert and per-rank tables in LDS, so the largest of
 * E + max(1024, K), 5E + 4R and 8E + 3R int32 values must fit in 158 KiB
 * (E = 4096 allows R <= 2048; E = 2048 any R that divides it).
 */
int moonep_plan(moonep_dims d, const int32_t* topk_idx, int32_t* expert_counts, double* maxvio,
                int32_t* cu_seqlens, int32_t* slot_expert, int32_t* dest_idx, int32_t* src_of_row,
                int32_t* stats, void* workspace, moonep_stream stream);

/*
 * moonep_plan_ex -- moonep_plan with a choice of planner (a moonep_planner value; anything else is
 * MOONEP_EINVAL).  The pages describe their planner as one that keeps the number of redundant experts
 * small ([P1] abstract; [P2] "Core technique: dynamic redundant experts") without printing its program.
 * MOONEP_PLAN_PREFIX is moonep_plan.  MOONEP_PLAN_MINCOPY changes only which pairs stay home: a rank
 * with L_r > P pairs sends its excess L_r - P out of its home experts taken largest first (equal counts:
 * lower id first), each overflowing what is still needed, so the excess leaves through the fewest
 * experts; every expert keeps the first keep_e pairs of its (src rank, token, k)-ordered list.  The
 * overflow list, the contiguous cut into deficits in rank order, slots, direct reads past B, cu_seqlens
 * and destinations then follow exactly as in moonep_plan.  Arguments, layouts, workspace (the same
 * moonep_plan_workspace_bytes) and limits are those of moonep_plan.
 */
int moonep_plan_ex(moonep_dims d, int32_t planner, const int32_t* topk_idx, int32_t* expert_counts,
                   double* maxvio, int32_t* cu_seqlens, int32_t* slot_expert, int32_t* dest_idx,
                   int32_t* src_of_row, int32_t* stats, void* workspace, moonep_stream stream);

/*
 * moonep_plan_static -- moonep_plan_ex for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  It takes no workspace: the
 * planner's scratch is a device array inside the library, moonep_plan_static_scratch_bytes() (8 MiB)
 * large, of which every GPU the library runs on holds its own copy until the process ends.  The call
 * allocates and frees nothing.  Arguments, outputs and limits are those of moonep_plan_ex; dims whose
 * moonep_plan_workspace_bytes exceed the scratch size are refused with MOONEP_EINVAL (use moonep_plan_ex
 * with a workspace then).  Every call on one GPU uses that GPU's one array: calls that overlap on a GPU
 * (concurrent streams, or threads) race and give unspecified plans; calls in stream order do not.  No
 * scratch contents carry over between calls (every planner kernel writes its part before reading it).
 * MOONEP_EHIP when the array's device address cannot be obtained on the current device.
 */
size_t moonep_plan_static_scratch_bytes(void);
int moonep_plan_static(moonep_dims d, int32_t planner, const int32_t* topk_idx, int32_t* expert_counts,
                       double* maxvio, int32_t* cu_seqlens, int32_t* slot_expert, int32_t* dest_idx,
                       int32_t* src_of_row, int32_t* stats, moonep_stream stream);

/*
 * moonep_dispatch -- fused permute ([P2] "Core technique": each token row is
 * written straight into its expert-grouped row of the fixed S*K buffer).
 *   Xp[dest_idx[r,s,k], :] = X[r,s,:] for every k; rows with dest -1 are skipped.
 * In:  X [R,S,H] dtype t;  dest_idx [R,S,K] int32 from moonep_plan.
 * Out: Xp [R*S*K, H] dtype t (bit-exact copies).
 */
int moonep_dispatch(moonep_dims d, int32_t H, moonep_dtype t, const void* X, const int32_t* dest_idx,
                    void* Xp, moonep_stream stream);

/*
 * moonep_prefetch -- copy each used slot's expert weights into the slot
 * ([P2] "Core technique" and "Memory contract": redundant experts are fetched
 * into rows [E, E+B) before expert compute).
 *   W_slots[r,j] = W_home[slot_expert[r,j]] when slot_expert[r,j] >= 0;
 *   unused slots are not written.
 * In:  W_home [E,H,Hp] dtype t;  slot_expert [R,B] int32.
 * Out: W_slots [R,B,H,Hp] dtype t (bit-exact copies).
 */
int moonep_prefetch(moonep_dims d, int32_t H, int32_t Hp, moonep_dtype t, const void* W_home,
                    const int32_t* slot_expert, void* W_slots, moonep_stream stream);

/* Bytes of device workspace moonep_group_gemm needs. */
size_t moonep_group_gemm_workspace_bytes(moonep_dims d);

/*
 * moonep_group_gemm -- the VM group GEMM over each rank's logical [E+B,H,Hp]
 * weight tensor, groups delimited by cu_seqlens ([P2] "Memory contract").
 *   For rank r, group g: Yp[rows] = Xp[rows] @ W_r[g], rows = r*P + [cu[r,g], cu[r,g+1]).
 *   bf16: float32 accumulation, result rounded to nearest-even bf16.
 *   f32:  float32 throughout.
 * In:  Xp [R*S*K,H], W_home [E,H,Hp], W_slots [R,B,H,Hp] (NULL when B == 0), dtype t;
 *      cu_seqlens [R,E+B+1] int32.
 * Out: Yp [R*S*K,Hp] dtype t.
 * workspace: moonep_group_gemm_workspace_bytes(d) bytes.
 */
int moonep_group_gemm(moonep_dims d, int32_t H, int32_t Hp, moonep_dtype t, const void* Xp,
                      const void* W_home, const void* W_slots, const int32_t* cu_seqlens, void* Yp,
                      void* workspace, moonep_stream stream);

/*
 * moonep_combine -- gate-weighted fused unpermute ([P2] "Core technique").
 *   out[r,s,:] = sum_{k=0..K-1} gates[r,s,k] * Yp[dest_idx[r,s,k], :]
 *   float32 accumulation in ascending k (fused multiply-add); dest -1 is skipped.
 * In:  Yp [R*S*K, D] dtype t;  dest_idx [R,S,K] int32;  gates [R,S,K] float32.
 * Out: out [R,S,D] float32.
 */
int moonep_combine(moonep_dims d, int32_t D, moonep_dtype t, const void* Yp, const int32_t* dest_idx,
                   const float* gates, float* out, moonep_stream stream);

/*
 * Backward of the data path.  The pages state that the backward pass runs through the same
 * buffers and that redundant experts' gradients go back to their home experts ([P2] "Core
 * technique"; [P3] third paragraph); read plainly, the data gradients are the chain rule of
 * dispatch -> group GEMM -> combine, each stage the transpose of its forward.
 */

/*
 * moonep_combine_backward -- gradients of moonep_combine given dout = d(loss)/d(out).
 *   For every pair (r,s,k) with q = dest_idx[r,s,k]:
 *     dYp[q] = gates[r,s,k] * dout[r,s]            (float32 product, then rounded to dtype t)
 *     dgates[r,s,k] = sum_n dout[r,s,n] * Yp[q,n]  (float32 accumulation)
 *   Every row of dYp is the destination of exactly one pair, so all of dYp is written.
 * In:  dout [R,S,D] float32;  Yp [R*S*K,D] dtype t;  dest_idx [R,S,K] int32;  gates [R,S,K] float32.
 * Out: dYp [R*S*K,D] dtype t;  dgates [R,S,K] float32.
 */
int moonep_combine_backward(moonep_dims d, int32_t D, moonep_dtype t, const float* dout, const void* Yp,
                            const int32_t* dest_idx, const float* gates, void* dYp, float* dgates,
                            moonep_stream stream);

/*
 * moonep_group_gemm_dgrad -- gradient of the VM group GEMM with respect to its input, through the
 * same groups and the same weight rows (home, slot, or a home row read directly):
 *   For rank r, group g: dXp[rows] = dYp[rows] @ W_r[g]^T, rows = r*P + [cu[r,g], cu[r,g+1]).
 *   bf16: float32 accumulation, result rounded to nearest-even bf16;  f32: float32 throughout.
 * In:  dYp [R*S*K,Hp], W_home [E,H,Hp], W_slots [R,B,H,Hp] (NULL when B == 0), dtype t;
 *      cu_seqlens [R,E+B+1] int32.
 * Out: dXp [R*S*K,H] dtype t.
 * workspace: moonep_group_gemm_workspace_bytes(d) bytes (the same workspace as the forward).
 */
int moonep_group_gemm_dgrad(moonep_dims d, int32_t H, int32_t Hp, moonep_dtype t, const void* dYp,
                            const void* W_home, const void* W_slots, const int32_t* cu_seqlens, void* dXp,
                            void* workspace, moonep_stream stream);

/*
 * moonep_dispatch_backward -- gradient of moonep_dispatch (the fused permute):
 *   dX[r,s] = sum over k ascending of dXp[dest_idx[r,s,k]], float32 additions.
 * In:  dXp [R*S*K,H] dtype t;  dest_idx [R,S,K] int32.
 * Out: dX [R,S,H] float32.
 */
int moonep_dispatch_backward(moonep_dims d, int32_t H, moonep_dtype t, const void* dXp, const int32_t* dest_idx,
                             float* dX, moonep_stream stream);

/*
 * Full gated expert FFN.  The pages ask for one [E+B, H, H'] tensor per expert projection ([P2]
 * "Memory contract and weight layout") without naming the FFN; read plainly it is the gated expert:
 * a gate|up projection [E+B, H, 2H'] (gate in output columns [0, H'), up in [H', 2H')), then
 * act = silu(gate) * up, then a down projection [E+B, H', H].  Both projections run through
 * moonep_group_gemm / moonep_group_gemm_dgrad / moonep_wgrad / moonep_reduce_grad with their own
 * (H, Hp) -- (H, 2H') and (H', H) -- and the same plan; these two calls are the activation.
 */

/*
 * moonep_swiglu -- A[q, c] = silu(Ygu[q, c]) * Ygu[q, Hp + c] for every dispatched row q < R*S*K and
 *   c < Hp, silu(g) = g * sigmoid(g); float32 arithmetic, rounded once to dtype t.
 * In:  Ygu [R*S*K, 2*Hp] dtype t.   Out: A [R*S*K, Hp] dtype t.
 */
int moonep_swiglu(moonep_dims d, int32_t Hp, moonep_dtype t, const void* Ygu, void* A, moonep_stream stream);

/*
 * moonep_swiglu_backward -- gradient of moonep_swiglu: with g = Ygu[q,c], u = Ygu[q,Hp+c],
 *   s = sigmoid(g), da = dA[q,c]:  dYgu[q,c] = da * u * s * (1 + g * (1 - s)),  dYgu[q,Hp+c] = da * g * s;
 *   float32 arithmetic, rounded once to dtype t.
 * In:  Ygu [R*S*K, 2*Hp], dA [R*S*K, Hp] dtype t.   Out: dYgu [R*S*K, 2*Hp] dtype t.
 */
int moonep_swiglu_backward(moonep_dims d, int32_t Hp, moonep_dtype t, const void* Ygu, const void* dA, void* dYgu,
                           moonep_stream stream);

/* Bytes of device workspace moonep_wgrad needs. */
size_t moonep_wgrad_workspace_bytes(moonep_dims d);

/*
 * moonep_wgrad -- weight-gradient group GEMM into the float32 gradient
 * buffers ([P2] "Memory contract": an fp32 [E+B,H,Hp] gradient per projection
 * whose rows [E,E+B) are separate reduce buffers).
 *   For every rank r and group g: dW_r[g] += Xp[rows]^T @ dY[rows].
 *   g < E adds into dW_home[g]; when several ranks hold rows of home row g
 *   (the home rank plus direct reads) their rows are summed in ascending rank
 *   order into one float32 accumulator and added once.  g = E+j adds into
 *   dW_slots[r,j].  Groups with no rows leave their gradient untouched.
 * In:  Xp [R*S*K,H], dY [R*S*K,Hp] dtype t;  cu_seqlens [R,E+B+1].
 * In/Out: dW_home [E,H,Hp] float32;  dW_slots [R,B,H,Hp] float32 (NULL when B == 0).
 * workspace: moonep_wgrad_workspace_bytes(d) bytes of device memory (256-byte aligned), contents
 * ignored on entry (it holds the size-ordered list of gradient jobs that have rows, the work
 * queue counters and a row of zeros, all of which the call itself writes before use).
 */
int moonep_wgrad(moonep_dims d, int32_t H, int32_t Hp, moonep_dtype t, const void* Xp, const void* dY,
                 const int32_t* cu_seqlens, float* dW_home, float* dW_slots, void* workspace,
                 moonep_stream stream);

/*
 * moonep_reduce_grad -- fold redundant-expert gradients back to their home
 * expert and clear them ([P2] "Core technique" and "Memory contract": the
 * R reduce buffers viewed as [R,B,H,Hp]; each slot's gradient is added into
 * the parameter gradient, then the consumed slot is zeroed).
 *   For each expert e and each element, in float32:
 *     acc = dW_home[e]; for r = 0..R-1: for the slot j of rank r holding e:
 *       acc += dW_slots[r,j]; dW_slots[r,j] = 0;   then dW_home[e] = acc.
 *   Unused slots (slot_expert -1) are neither read nor written.
 * In:  slot_expert [R,B] int32.
 * In/Out: dW_home [E,H,Hp] float32;  dW_slots [R,B,H,Hp] float32.
 */
int moonep_reduce_grad(moonep_dims d, int32_t H, int32_t Hp, const int32_t* slot_expert, float* dW_home,
                       float* dW_slots, moonep_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* MOONEP_H */
