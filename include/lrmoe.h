/*
 * lrmoe.h -- C ABI of the MI355X (gfx950) pruned MoE expert backward.
 *
 * The library implements, for the experts local to one GPU, the backward of
 * one expert projection y = W_e phi under LRMoE's pruning:
 *
 *   1. quota     q_e pairs kept per expert, fixed before the backward
 *                ("LRMoE: Trimming Backward Work in Memory-Bound MoE Training",
 *                section "Backward demand is not a constant").
 *   2. score     R_u = alpha_u^2 * ||g_t||^2 * ||phi_u||^2 for each routed pair
 *                u = (t, e) (same article, section "LRM: a decomposable
 *                contribution score").
 *   3. select    per expert, the q_e pairs with the highest R_u
 *                ("LRMoE poda a passagem reversa do MoE ...", bullet on
 *                selection by the LRM metric).
 *   4. compact   kept g rows, phi rows and alpha packed into contiguous,
 *                expert-segmented, unpadded buffers (English article, section
 *                "The part that is easy to get wrong"; Portuguese write-up,
 *                bullet on physical compaction).
 *   5. GEMMs     dW_e = sum_kept (alpha_u g_t) phi_u^T and
 *                dphi_u = alpha_u W_e^T g_t, written back to the original pair
 *                layout (English article, "LRM: ..." for the per-pair outer
 *                product; Portuguese write-up, compaction bullet, for the
 *                return to the original layout).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pairs are expert-sorted: pairs [off_e, off_e + n_e) belong to local
 *    expert e, off_e = n_0 + ... + n_{e-1}.  Pair index u is the row of phi.
 *  - Tensors are dense row-major.  g is [T, d_out], phi is [P, d_in], W is
 *    [E, d_out, d_in] (W_e maps phi in R^d_in to y in R^d_out), dW is
 *    [E, d_out, d_in] float32, dphi is [P, d_in] float32.
 *  - Storage type of g, phi, W and of the compacted g_c, phi_c is given by
 *    lrmoe_problem.dtype (bfloat16 or float32).  Arithmetic is float32
 *    (bf16 matrix cores with float32 accumulation for the GEMMs).
 *  - Counts and quotas are HOST arrays, read during the call only.  Every
 *    other pointer is a DEVICE pointer, used asynchronously in the order of
 *    `stream` (a hipStream_t; NULL means the null stream).  The caller owns
 *    all memory; the library allocates nothing and keeps no state between
 *    calls, so calls on different streams may run concurrently if their
 *    buffers are disjoint.  Outputs must not alias inputs.
 *  - Device pointers must be 16-byte aligned.  d_out and d_in must be
 *    multiples of 8 (bf16) or 4 (float32).
 *  - Row indices are a precondition the host cannot check (they live in
 *    device memory): 0 <= g_row_index[u] < T and 0 <= phi_row_index[u] <
 *    T_phi.  The kernels still bound every index they read, so a violation
 *    does not fault: a g or phi row whose index is out of range reads as a
 *    row of zeros (score 0, zero compacted row), and a perm entry outside
 *    0..P-1 is skipped.  A call that reads g rows for P > 0 pairs needs
 *    T >= 1 (LRMOE_ERR_SHAPE otherwise), and one that reads phi through a
 *    row index for M > 0 kept pairs needs 1 <= T_phi < 2^31.
 *  - Errors: every host-detectable problem is reported before anything is
 *    launched, and no entry point aborts or prints.  A failed kernel launch
 *    returns LRMOE_ERR_HIP; faults inside kernels surface at the caller's
 *    next synchronisation.
 */
#ifndef LRMOE_H
#define LRMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LRMOE_ABI_VERSION 4
#define LRMOE_MAX_EXPERTS 256

typedef enum {
  LRMOE_OK = 0,
  LRMOE_ERR_NULL = 1,      /* a required pointer is NULL                     */
  LRMOE_ERR_INVALID = 2,   /* bad expert count, quota or policy              */
  LRMOE_ERR_SHAPE = 3,     /* sizes inconsistent or out of range             */
  LRMOE_ERR_ALIGN = 4,     /* pointer or row length misaligned               */
  LRMOE_ERR_DTYPE = 5,     /* unknown storage type                           */
  LRMOE_ERR_WORKSPACE = 6, /* workspace smaller than lrmoe_workspace_size    */
  LRMOE_ERR_HIP = 7,       /* a HIP runtime call or launch failed            */
  LRMOE_ERR_SCRATCH = 8    /* more scratch than the static buffer holds
                              (lrmoe_score_select_compact_noalloc)           */
} lrmoe_status;

typedef enum { LRMOE_F32 = 0, LRMOE_BF16 = 1 } lrmoe_dtype;

typedef enum {
  /* keep floor(n_e * num / den) pairs of every expert (C-level Cx is
   * num/den = (100 - x)/100; C0 keeps everything)                          */
  LRMOE_QUOTA_RATIO = 0,
  /* a fixed number of pairs for the layer call, shared in proportion to
   * demand: q_e = min(n_e, floor(n_e * budget_pairs / P))                  */
  LRMOE_QUOTA_BUDGET = 1
} lrmoe_quota_mode;

typedef struct {
  int32_t mode;          /* lrmoe_quota_mode                                */
  int64_t num, den;      /* RATIO: 0 <= num <= den, den > 0                 */
  int64_t budget_pairs;  /* BUDGET: >= 0                                    */
} lrmoe_quota_policy;

/* How the GEMMs fold alpha into the weight gradient.  alpha multiplies the
 * reduction index of dW_e = sum_j (alpha_j g_j) phi_j^T, so it enters an
 * operand before the matrix cores (the narrower of g and phi carries it).
 * EXACT (0): alpha*x is split into a bf16 high part and a bf16 residual and
 *   both are multiplied (two matrix-core passes for dW), so dW carries
 *   float32-level error (about 2^-16 relative per term).
 * BF16 (1): alpha*x is rounded once to bf16 (the rounding a bf16 training
 *   step applies); one pass, up to 2^-8 relative per term.
 * F16 (2): one pass on float16 matrix cores (the same rate as bf16): the
 *   other operand converts from bf16 exactly, alpha*x is rounded once to
 *   float16 (2^-11 relative per term, eight times finer than bf16).  Both
 *   are scaled per expert by powers of two taken from the largest row norm
 *   over the expert's kept rows (a bound of the largest magnitude), so any
 *   bf16 range maps into float16's; the product is unscaled exactly.  bf16
 *   storage only (float32 storage uses EXACT).
 * dphi always applies alpha in float32 after the product.  float32 storage
 * always splits both operands (three bf16 passes). */
typedef enum { LRMOE_DW_EXACT = 0, LRMOE_DW_BF16 = 1, LRMOE_DW_F16 = 2 } lrmoe_dw_mode;

/* Scoring rule of lrmoe_score_select_compact.  LRM is the method's metric
 * R_u = alpha_u^2 * ||g_t||^2 * ||phi_u||^2.  The others are the ablation
 * baselines the pages compare it with ("LRMoE: Trimming Backward Work in
 * Memory-Bound MoE Training", section "What the measurements show"): the
 * squared norm of the upstream gradient alone, ||g_t||^2, and its absolute
 * magnitude, read here as the L1 norm sum_i |g_t,i| (the Euclidean norm
 * would rank pairs exactly like the squared norm).  Random dropping, the
 * third baseline, takes caller-drawn scores through lrmoe_select_compact.
 * The gradient-only rules read no phi row.  Sums are float32. */
typedef enum {
  LRMOE_SCORE_LRM = 0,
  LRMOE_SCORE_GRAD_SQNORM = 1,
  LRMOE_SCORE_GRAD_L1 = 2
} lrmoe_score_mode;

typedef struct {
  int32_t E;               /* local experts, 1 .. LRMOE_MAX_EXPERTS          */
  int32_t dtype;           /* lrmoe_dtype                                    */
  int64_t P;               /* routed pairs, 0 <= P < 2^31                     */
  int64_t T;               /* rows of g (T == P when every pair has its row) */
  int32_t d_out;           /* length of g rows = rows of W_e                 */
  int32_t d_in;            /* length of phi rows = columns of W_e            */
  const int64_t* counts;   /* host [E]: n_e, sum = P                          */
  const int64_t* quotas;   /* host [E]: q_e, 0 <= q_e <= n_e                  */
  int32_t dw_mode;         /* lrmoe_dw_mode                                  */
  int32_t score_mode;      /* lrmoe_score_mode (0 = LRM)                     */
  int64_t T_phi;           /* rows of phi when a phi_row_index is passed
                              (lrmoe_gather_compact, lrmoe_gather_backward);
                              ignored otherwise, where phi has P rows        */
} lrmoe_problem;

/* ABI version of the loaded library (LRMOE_ABI_VERSION at build time). */
int32_t lrmoe_abi_version(void);

/* Static English text for a status code (never NULL). */
const char* lrmoe_status_string(lrmoe_status s);

/* Step 1 (host only, no GPU): quotas_out[e] from counts[e] under `policy`.
 * Integer arithmetic, floor rounding, no minimum of one (an expert with one
 * pair at C20 keeps none).  The quota is fixed for the whole layer call.
 * Errors: NULL pointers; E outside 1..LRMOE_MAX_EXPERTS, a negative count or
 * a bad policy -> LRMOE_ERR_INVALID. */
lrmoe_status lrmoe_plan_quota(int32_t E, const int64_t* counts,
                              const lrmoe_quota_policy* policy,
                              int64_t* quotas_out);

/* Step 1 on the device, from the forward's routing instead of host counts
 * (the quota is fixed before the backward from how many pairs reached each
 * expert -- "LRMoE poda a passagem reversa do MoE e acelera o treinamento
 * em 21-45%", bullet "Cotas antes do calculo").
 *   expert_ids   int32 [n_ids] device: local expert index of every routed
 *                pair, any order; an index outside 0..E-1 is not routed and
 *                is counted in *invalid_out instead
 *   counts_out   int64 [E] device: n_e
 *   quotas_out   int64 [E] device: q_e, the same integer rules and results
 *                as lrmoe_plan_quota on counts_out (budget P = sum n_e)
 *   seg_offsets_out int64 [E+1] device: exclusive prefix sum of q_e (the
 *                last entry is M)
 *   invalid_out  int64 [1] device or NULL
 * Asynchronous on `stream`; device pointers 16-byte aligned.  Errors (before
 * any launch): NULL policy or required pointer, misalignment, E outside
 * 1..LRMOE_MAX_EXPERTS or a bad policy (LRMOE_ERR_INVALID), n_ids outside
 * 0..2^31-1 (LRMOE_ERR_SHAPE). */
lrmoe_status lrmoe_plan_quota_device(int32_t E, const int32_t* expert_ids, int64_t n_ids,
                                     const lrmoe_quota_policy* policy, int64_t* counts_out,
                                     int64_t* quotas_out, int64_t* seg_offsets_out,
                                     int64_t* invalid_out, void* stream);

/* Workspace bytes needed by every call of this problem that takes a
 * workspace (one buffer may serve all of them when they run in order on one
 * stream).  Validates the problem like the calls that use it.  The size is
 * returned through bytes_out, so that a bad problem is reported as a status
 * like everywhere else. */
lrmoe_status lrmoe_workspace_size(const lrmoe_problem* pb, size_t* bytes_out);

/* Steps 2-4.  Inputs: alpha f32 [P]; g [T, d_out]; phi [P, d_in];
 * g_row_index int32 [P] gives the g row of each pair (NULL when T == P and
 * pair u uses row u).
 * Outputs (M = sum of quotas, known to the caller from the host quotas):
 *   scores      f32 [P]   R_u (float32 arithmetic, norms summed in float32)
 *   keep        u8  [P]   1 if the pair is kept
 *   seg_offsets i32 [E+1] exclusive prefix sum of the quotas
 *   perm        i32 [M]   original pair index of each compacted row; segments
 *                         in ascending expert order, ascending pair index
 *                         inside a segment
 *   g_c [M, d_out], phi_c [M, d_in], alpha_c f32 [M]: bit-exact copies of the
 *                         kept rows
 *   dphi_zero   f32 [P, d_in] or NULL: rows of dropped pairs are set to 0 (the
 *                         kept rows are left for lrmoe_grouped_backward)
 * Selection: the q_e-th largest score of expert e is the threshold tau_e;
 * every pair above it is kept and pairs equal to it are kept in ascending
 * pair index until q_e pairs are kept.  Scores must be finite. */
lrmoe_status lrmoe_score_select_compact(
    const lrmoe_problem* pb, const int32_t* g_row_index, const float* alpha,
    const void* g, const void* phi, float* scores, uint8_t* keep,
    int32_t* seg_offsets, int32_t* perm, void* g_c, void* phi_c, float* alpha_c,
    float* dphi_zero, void* workspace, size_t ws_bytes, void* stream);

/* lrmoe_score_select_compact for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): no workspace argument.  The selection's scratch -- used when
 * an expert has more than 24576 pairs: three radix-digit histograms and the
 * select state per expert (33 KiB) and two counts per 4096-pair chunk --
 * lives in a static device array of the library, 8 MiB, which every GPU the
 * library runs on holds until the process ends.  Problems that need more
 * (about 240 experts or more, with one of them above 24576 pairs) are
 * rejected with LRMOE_ERR_SCRATCH before anything is launched.  The call allocates nothing; on its first call on a
 * device it looks up that device's copy of the array (the current device,
 * which `stream` must belong to).  Nothing in the scratch needs to start at
 * zero: every call writes what it later reads.  All calls on one GPU share
 * that GPU's array, so calls that overlap in time on one GPU (different
 * streams, or different host threads) race and must not be issued.
 * Arguments, results and other errors as for lrmoe_score_select_compact. */
lrmoe_status lrmoe_score_select_compact_noalloc(
    const lrmoe_problem* pb, const int32_t* g_row_index, const float* alpha,
    const void* g, const void* phi, float* scores, uint8_t* keep,
    int32_t* seg_offsets, int32_t* perm, void* g_c, void* phi_c, float* alpha_c,
    float* dphi_zero, void* stream);

/* Steps 3-4 on caller-provided scores (float32 [P], finite; -0.0 counts as
 * 0.0), for scoring rules other than LRM.  Arguments as above. */
lrmoe_status lrmoe_select_compact(
    const lrmoe_problem* pb, const float* scores, const int32_t* g_row_index,
    const float* alpha, const void* g, const void* phi, uint8_t* keep,
    int32_t* seg_offsets, int32_t* perm, void* g_c, void* phi_c, float* alpha_c,
    float* dphi_zero, void* workspace, size_t ws_bytes, void* stream);

/* Steps 2-3 without compaction: scores, keep flags, seg_offsets and perm as
 * in lrmoe_score_select_compact, no row is moved.  For the zero-masked dense
 * alternative below. */
lrmoe_status lrmoe_score_select(
    const lrmoe_problem* pb, const int32_t* g_row_index, const float* alpha,
    const void* g, const void* phi, float* scores, uint8_t* keep,
    int32_t* seg_offsets, int32_t* perm, void* workspace, size_t ws_bytes,
    void* stream);

/* Zero-masked dense alternative to compaction (what the pages argue against:
 * masking the surplus rows of full-size tensors saves neither time nor
 * memory -- "LRMoE poda a passagem reversa do MoE e acelera o treinamento em
 * 21-45%", the paragraph after the bullets).  alpha_masked f32 [P] = alpha
 * where keep, 0 where dropped; perm_identity int32 [P] (or NULL) = 0..P-1.
 * Running lrmoe_grouped_backward with quotas = counts, perm_identity,
 * alpha_masked and the uncompacted g (one row per pair) and phi yields the
 * same dW and dphi as the compacted path, dropped dphi rows included (0).
 * Errors: NULL / misaligned pointers, P outside 0..2^31-1. */
lrmoe_status lrmoe_mask_alpha(int64_t P, const uint8_t* keep, const float* alpha,
                              float* alpha_masked, int32_t* perm_identity, void* stream);

/* Step 4 alone, for a second projection of the same pairs that inherits an
 * existing keep set (the gate/up projection of the expert MLP: a pair whose
 * down-projection input gradient is zero has zero gate/up gradient, so it is
 * not rescored).  pb describes the second projection (its d_out, d_in, T and
 * dtype; the same counts and quotas); perm and keep come from an earlier
 * lrmoe_score_select_compact.  g_row_index / phi_row_index (int32 [P], or
 * NULL for row u of pair u) pick the source rows of g and phi; the kept
 * rows are copied bit for bit into g_c [M, d_out] and phi_c [M, d_in], alpha
 * into alpha_c [M], and dphi_zero (or NULL) gets zero rows for dropped
 * pairs.  g and g_c may both be NULL: only phi rows and alpha are gathered
 * (the gate/up output gradient of lrmoe_grouped_backward_glu is already
 * compacted). */
lrmoe_status lrmoe_gather_compact(
    const lrmoe_problem* pb, const int32_t* perm, const uint8_t* keep,
    const int32_t* g_row_index, const int32_t* phi_row_index,
    const float* alpha, const void* g, const void* phi, void* g_c,
    void* phi_c, float* alpha_c, float* dphi_zero, void* stream);

/* lrmoe_gather_compact followed by lrmoe_grouped_backward on the same
 * buffers, for a projection on an inherited keep set (the gate/up projection
 * above), in one call.  With bf16 storage the gather also writes the GEMM's
 * operand planes from the rows it moves (as in lrmoe_pruned_backward), bit
 * for bit the separate calls' results.  g and g_c are required here; dphi is
 * both the zero target of dropped rows and the output of kept rows (or
 * NULL); dropped rows of at least 512 MiB in all are cleared inside the
 * grouped GEMM launch, as in lrmoe_pruned_backward.  workspace:
 * lrmoe_workspace_size bytes.  Errors as for the two calls. */
lrmoe_status lrmoe_gather_backward(
    const lrmoe_problem* pb, const int32_t* perm, const uint8_t* keep,
    const int32_t* g_row_index, const int32_t* phi_row_index,
    const float* alpha, const void* g, const void* phi, const void* W,
    void* g_c, void* phi_c, float* alpha_c, float* dW, float* dphi,
    void* workspace, size_t ws_bytes, void* stream);

/* Step 5: variable-length grouped GEMMs over the compacted buffers.
 *   dW   f32 [E, d_out, d_in]: fully overwritten (zero for q_e = 0)
 *   dphi f32 [P, d_in] or NULL: rows perm[j] receive alpha_c[j] W_e^T g_c[j];
 *        other rows are not touched (see dphi_zero above).
 * W is [E, d_out, d_in] in the storage type; segments are given by the host
 * quotas of pb. */
lrmoe_status lrmoe_grouped_backward(
    const lrmoe_problem* pb, const int32_t* perm, const float* alpha_c,
    const void* g_c, const void* phi_c, const void* W, float* dW, float* dphi,
    void* workspace, size_t ws_bytes, void* stream);

/* The expert MLP's activation backward, chained on the compacted layout.
 * The models trained in "What the measurements show" ("LRMoE: Trimming
 * Backward Work in Memory-Bound MoE Training": Qwen3-30B-A3B,
 * GLM4.5-106B-A12B) have gated-MLP experts whose down projection reads
 * phi = SiLU(a) * b, a and b being the saved gate and up pre-activations.
 * The pages do not spell this step out (a reading); they only say that the
 * original layout is restored after the compacted GEMMs ("LRMoE poda a
 * passagem reversa do MoE e acelera o treinamento em 21-45%", compaction
 * bullet), which this entry point postpones past the activation backward.  Same as lrmoe_grouped_backward for dW (the down projection's),
 * but instead of dphi it writes, for every compacted row j (pair
 * u = perm[j] of expert e), with d = W_e^T g_c[j] before the routing weight:
 *   dgu_c[j] = [ d * b_u * SiLU'(a_u)  |  d * SiLU(a_u) ]
 * SiLU'(a) = s (1 + a (1 - s)), s = sigmoid(a), computed in float32.  dgu_c
 * is [M, 2 d_in], gate half first: the gate/up projection's output gradient,
 * already compacted.  Its storage follows pb->dw_mode: float32 (unrounded)
 * unless dw_mode is LRMOE_DW_BF16, where each entry is rounded once to bf16
 * (the single-rounding mode, with that mode's error bound).  The chain ends
 * with lrmoe_gather_compact (g = g_c = NULL) of the gate/up projection's
 * inputs x, then, with the same perm and alpha_c (alpha applied once,
 * there), lrmoe_grouped_backward_gate_up on the float32 dgu_c, or
 * lrmoe_grouped_backward with g_c = dgu_c on the bf16 one.  No
 * original-layout dphi is written and none needs zeroing.
 *   act_a, act_b  bf16 [P, d_in], pair-indexed like phi.
 * act_a, act_b and dgu_c may be NULL when no pair is kept (M = 0).  bf16
 * storage only (LRMOE_ERR_DTYPE otherwise); other errors as for
 * lrmoe_grouped_backward. */
lrmoe_status lrmoe_grouped_backward_glu(
    const lrmoe_problem* pb, const int32_t* perm, const float* alpha_c,
    const void* g_c, const void* phi_c, const void* W, float* dW,
    const void* act_a, const void* act_b, void* dgu_c, void* workspace,
    size_t ws_bytes, void* stream);

/* The gate/up projection's backward at the end of the MLP chain above: the
 * same products as lrmoe_grouped_backward (dW [E, d_out, d_in] of the gate/up
 * weight, dx rows perm[j] of [P, d_in], alpha applied once) with the float32
 * output gradient dgu_c [M, d_out] of lrmoe_grouped_backward_glu (d_out = 2
 * d_in of the down projection) as g_c, and bf16 x_c [M, d_in] and W
 * [E, d_out, d_in].  alpha * dgu_c is split into a bf16 high part and
 * residual (hi only when dw_mode is LRMOE_DW_BF16) that feed both products,
 * so the gradient handed over keeps float32-level precision.  dx may be NULL
 * (dW only).  pb->dtype must be LRMOE_BF16 (LRMOE_ERR_DTYPE otherwise);
 * workspace: lrmoe_workspace_size of pb; other errors as for
 * lrmoe_grouped_backward. */
lrmoe_status lrmoe_grouped_backward_gate_up(
    const lrmoe_problem* pb, const int32_t* perm, const float* alpha_c, const float* dgu_c,
    const void* x_c, const void* W, float* dW, float* dx, void* workspace, size_t ws_bytes,
    void* stream);

/* Steps 2-5 in one call: lrmoe_score_select_compact followed by
 * lrmoe_grouped_backward on the same buffers, with the same arguments and
 * results (dphi is both the zero target of dropped rows and the output of
 * kept rows; NULL for dW only).  With bf16 storage the gather also writes the
 * GEMM's operand planes (alpha times the narrower compacted operand, as bf16
 * hi and, in exact mode, lo) from the rows it moves, so no separate pass
 * reads the compacted operand again; the planes and every result are bit for
 * bit those of the two separate calls.  When the dropped pairs' dphi rows
 * hold at least 512 MiB ((P - M) * d_in * 4 bytes), the grouped GEMM launch
 * clears them beside its tiles instead of the gather (same results).
 * workspace: lrmoe_workspace_size bytes.  Errors as for the two calls. */
lrmoe_status lrmoe_pruned_backward(
    const lrmoe_problem* pb, const int32_t* g_row_index, const float* alpha,
    const void* g, const void* phi, const void* W, float* scores, uint8_t* keep,
    int32_t* seg_offsets, int32_t* perm, void* g_c, void* phi_c, float* alpha_c,
    float* dW, float* dphi, void* workspace, size_t ws_bytes, void* stream);

/* Per-kernel timing.  Each entry point below launches a fixed sequence of
 * kernels; for every non-NULL pair, `before` and `after` (hipEvent_t created
 * by the caller with timing enabled) are recorded on `stream` right before
 * and right after that kernel's launch.  Kernels not launched for a problem
 * (an empty range) leave their events unrecorded.
 *   lrmoe_score_select_compact_timed: [0] score  [1] select+scan  [2] gather
 *   lrmoe_select_compact_timed:       [1] select+scan  [2] gather
 *   lrmoe_grouped_backward_timed,
 *   lrmoe_grouped_backward_glu_timed,
 *   lrmoe_grouped_backward_gate_up_timed:
 *                                     [0] operand prologue  [1] grouped GEMM
 *                                     [2] split-K reduction
 *   lrmoe_pruned_backward_timed:      [0] score  [1] select+scan  [2] gather
 *                                     [3] grouped GEMM  [4] split-K reduction
 *                                     [5] operand prologue (float32 storage)
 *   lrmoe_gather_backward_timed:      [2] gather  [3] grouped GEMM
 *                                     [4] split-K reduction
 *                                     [5] operand prologue (float32 storage) */
#define LRMOE_TIMING_SLOTS 8
typedef struct {
  void* before[LRMOE_TIMING_SLOTS];
  void* after[LRMOE_TIMING_SLOTS];
} lrmoe_timing;

/* lrmoe_score_select_compact with per-kernel events (timing may be NULL). */
lrmoe_status lrmoe_score_select_compact_timed(
    const lrmoe_problem* pb, const int32_t* g_row_index, const float* alpha,
    const void* g, const void* phi, float* scores, uint8_t* keep,
    int32_t* seg_offsets, int32_t* perm, void* g_c, void* phi_c, float* alpha_c,
    float* dphi_zero, void* workspace, size_t ws_bytes, void* stream,
    const lrmoe_timing* timing);

/* lrmoe_select_compact with per-kernel events (timing may be NULL). */
lrmoe_status lrmoe_select_compact_timed(
    const lrmoe_problem* pb, const float* scores, const int32_t* g_row_index,
    const float* alpha, const void* g, const void* phi, uint8_t* keep,
    int32_t* seg_offsets, int32_t* perm, void* g_c, void* phi_c, float* alpha_c,
    float* dphi_zero, void* workspace, size_t ws_bytes, void* stream,
    const lrmoe_timing* timing);

/* lrmoe_grouped_backward with per-kernel events (timing may be NULL). */
lrmoe_status lrmoe_grouped_backward_timed(
    const lrmoe_problem* pb, const int32_t* perm, const float* alpha_c,
    const void* g_c, const void* phi_c, const void* W, float* dW, float* dphi,
    void* workspace, size_t ws_bytes, void* stream, const lrmoe_timing* timing);

/* lrmoe_pruned_backward with per-kernel events (timing may be NULL). */
lrmoe_status lrmoe_pruned_backward_timed(
    const lrmoe_problem* pb, const int32_t* g_row_index, const float* alpha,
    const void* g, const void* phi, const void* W, float* scores, uint8_t* keep,
    int32_t* seg_offsets, int32_t* perm, void* g_c, void* phi_c, float* alpha_c,
    float* dW, float* dphi, void* workspace, size_t ws_bytes, void* stream,
    const lrmoe_timing* timing);

/* lrmoe_gather_backward with per-kernel events (timing may be NULL). */
lrmoe_status lrmoe_gather_backward_timed(
    const lrmoe_problem* pb, const int32_t* perm, const uint8_t* keep,
    const int32_t* g_row_index, const int32_t* phi_row_index,
    const float* alpha, const void* g, const void* phi, const void* W,
    void* g_c, void* phi_c, float* alpha_c, float* dW, float* dphi,
    void* workspace, size_t ws_bytes, void* stream, const lrmoe_timing* timing);

/* lrmoe_grouped_backward_glu with per-kernel events (timing may be NULL). */
lrmoe_status lrmoe_grouped_backward_glu_timed(
    const lrmoe_problem* pb, const int32_t* perm, const float* alpha_c,
    const void* g_c, const void* phi_c, const void* W, float* dW,
    const void* act_a, const void* act_b, void* dgu_c, void* workspace,
    size_t ws_bytes, void* stream, const lrmoe_timing* timing);

/* lrmoe_grouped_backward_gate_up with per-kernel events (timing may be NULL). */
lrmoe_status lrmoe_grouped_backward_gate_up_timed(
    const lrmoe_problem* pb, const int32_t* perm, const float* alpha_c, const float* dgu_c,
    const void* x_c, const void* W, float* dW, float* dx, void* workspace, size_t ws_bytes,
    void* stream, const lrmoe_timing* timing);

#ifdef __cplusplus
}
#endif
#endif /* LRMOE_H */
