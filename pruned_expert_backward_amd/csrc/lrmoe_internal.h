// Internal declarations shared by the HIP translation units of liblrmoe.
// Nothing here is part of the C ABI (include/lrmoe.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lrmoe.h"

namespace lrmoe {

constexpr int kMaxE = LRMOE_MAX_EXPERTS;

// Per-expert offsets, known on the host before the backward starts (the
// quotas are fixed ahead of it), passed to kernels by value so that no
// host-to-device copy or device-side prefix sum is needed.
// Selection.  Problems whose experts all have at most kSelLdsKeys pairs are
// selected by one workgroup per expert with the keys in LDS.  Otherwise every
// expert's pairs are cut into chunks of kSelChunk, and each pass of the radix
// select and the scan runs one workgroup per chunk.
constexpr int kSelLdsKeys = 24576;
constexpr int kSelChunk = 4096;

struct ExpertTable {
  int32_t E;
  int32_t M;                      // total kept pairs
  int32_t pair_off[kMaxE + 1];    // first pair of expert e (expert-sorted)
  int32_t seg_off[kMaxE + 1];     // first compacted row of expert e
  int32_t chunk_off[kMaxE + 1];   // first selection chunk of expert e
};

// Selection chunks of an expert with n pairs.
inline int sel_chunks(int64_t n) { return (int)((n + kSelChunk - 1) / kSelChunk); }

// Tile schedule of the grouped GEMMs (host-built, by value).  Output tiles
// are kTile x kTile.  Tiles are handed out in groups of kGroupSlots slots
// (a gm x gn block of tiles of one expert and K chunk, sharing operand
// panels).  Each XCD owns a queue of groups that its resident workgroups
// drain through an atomic counter, so a group's panels meet in one L2.  The
// weight gradient of an expert with many kept rows is split along K into
// chunks of kc rows whose fp32 partial tiles are summed afterwards in chunk
// order.
constexpr int kTile = 256;
constexpr int kGroupSlots = 12;
constexpr int kXcds = 8;
// Work counters of the grouped GEMM launch: one tile queue per XCD, then the
// zero-fill of dropped input-gradient rows.
constexpr int kZeroCounter = kXcds;
constexpr int kHeadCounters = kXcds + 1;
constexpr int kMaxGroups = 600;

// Group descriptor: bit 31 = weight gradient, bits 23..30 expert,
// bits 15..22 K chunk, bits 0..14 sub-group inside the expert (and chunk).
__host__ __device__ inline uint32_t group_desc(bool dw, int e, int chunk, int sub) {
  return (dw ? 0x80000000u : 0u) | ((uint32_t)e << 23) | ((uint32_t)chunk << 15) | (uint32_t)sub;
}

struct GemmTable {
  int32_t E;
  int32_t tiles_n;                // output column tiles (over d_in)
  int32_t dw_tiles_m;             // dW row tiles (over d_out)
  int32_t dw_gm, dw_gn;           // dW group shape, dw_gm * dw_gn <= kGroupSlots
  int32_t dp_gm, dp_gn;           // dphi group shape
  int32_t kc;                     // dW K-chunk length (multiple of the K step)
  int32_t use_table;              // 1: groups[] below; 0: formula order (fallback)
  int32_t tall;                   // 1: the last column holds <= kTile/2 columns; its
                                  //    input-gradient tiles are 512 x 128, each over two
                                  //    row tiles
  int32_t dw_groups;              // formula order: dW groups first ...
  int32_t total_groups;           // ... then dphi groups
  int32_t qoff[kXcds + 1];        // table: XCD x drains groups [qoff[x], qoff[x+1])
  int32_t seg_off[kMaxE + 1];     // compacted segment offsets
  union {
    uint32_t groups[kMaxGroups];  // table: group descriptors, XCD-major
    struct {
      int32_t dw_goff[kMaxE + 1]; // formula: first dW group of the expert of LPT rank r
      int32_t dp_goff[kMaxE + 1]; // formula: first dphi group of expert e
      uint8_t order[kMaxE];       // formula: expert of LPT rank r
    } f;
  };
};

// Device operand planes of the two products.  Every plane is bf16; a second
// plane holds the residual of a float32 value split as hi + lo.
struct GemmOperands {
  const uint16_t* dw_a[2];        // [M, d_out]: g_c, or alpha*g_c split
  const uint16_t* dw_b[2];        // [M, d_in]: phi_c, or alpha*phi_c split
  const uint16_t* dp_a[2];        // [M, d_out]: g_c
  const uint16_t* dp_b[2];        // [E, d_out, d_in]: W
  int32_t dw_pa, dw_pb, dp_pa, dp_pb;   // planes in use (1 or 2)
  float* partials;                // fp32 partial dW tiles of split experts
  int32_t* queue_heads;           // kHeadCounters counters, zeroed by the prologue
  // Zero-fill carried by the launch (zero_rows != nullptr): the rows u of
  // zero_rows ([P, d_in] float32) with zero_keep[u] == 0 are cleared.  The
  // first zero_first workgroups start with it, every workgroup helps once
  // its tile queues are empty.
  const uint8_t* zero_keep;
  float* zero_rows;
  int32_t zero_first;
  // SiLU-GLU chain (glu_out != nullptr): the input-gradient tiles, instead of
  // writing alpha * dphi, write the gate/up output gradient of each kept
  // pair from its saved pre-activations a = glu_a[u], b = glu_b[u] ([P,
  // d_in] bf16, u = perm[j]): glu_out[j] = [dphi*b*silu'(a), dphi*silu(a)]
  // ([M, 2 d_in], float32 if glu_f32 else bf16), dphi before alpha.
  const uint16_t* glu_a;
  const uint16_t* glu_b;
  void* glu_out;
  int32_t glu_f32;
  // float16 weight gradient (see f16_scale_exp), with powers of two from
  // dw_ebound.  1: dw_a is the compacted bf16 g_c and dw_b the scaled
  // float16 plane of alpha * phi_c; 2: dw_a the plane of alpha * g_c and dw_b
  // the bf16 phi_c (the bf16 side is converted to scaled float16 in the
  // GEMM's registers); 3: both are scaled float16 planes.
  int32_t dw_f16;
  const float* dw_ebound;
  // 1: the input-gradient A planes already carry alpha (alpha * g_c split),
  // so the epilogue does not scale the rows again.
  int32_t dp_alpha_folded;
};

// Number of K chunks of an expert with q kept rows.
__host__ __device__ inline int dw_chunks(int q, int kc) { return q <= kc ? 1 : (q + kc - 1) / kc; }

// First partial tile of expert e (tiles of split experts, chunk-minor).
__host__ __device__ inline int64_t partial_base(const GemmTable& t, int e) {
  int64_t base = 0;
  const int tiles = t.dw_tiles_m * t.tiles_n;
  for (int x = 0; x < e; ++x) {
    const int S = dw_chunks(t.seg_off[x + 1] - t.seg_off[x], t.kc);
    if (S > 1) base += (int64_t)tiles * S;
  }
  return base;
}

// alpha * x split into bf16 hi = RNE(alpha x) and lo = RNE(alpha x - hi),
// the residual from one explicit FMA (exact product, one rounding), so that
// the operand planes are bit for bit the same wherever they are written --
// no compiler choice of contraction is involved.
struct HiLo {
  __bf16 h, l;
};
__device__ __forceinline__ HiLo alpha_split(float a, float x) {
  const __bf16 h = (__bf16)(a * x);
  return {h, (__bf16)__builtin_fmaf(a, x, -(float)h)};
}

// ---- float16 weight-gradient mode (LRMOE_DW_F16)
// dW_e = sum_j A_j B_j^T runs on float16 matrix cores: A = 2^sA (the g row),
// B = 2^sB (the phi row), alpha folded into one side and rounded once to 11
// significant bits (the other side converts from bf16 exactly, in its own
// plane or inside the GEMM).  sA, sB are
// per-expert powers of two from the largest row norm over the expert's kept
// rows (ebound[e] = {max |A row|, max |B row|}, each at least the largest
// magnitude): 2^s ebound lands in [2^14, 2^15), so every scaled value stays
// below 65504, and values down to 2^-28 of it (2^-34 for rows of 4096)
// stay normal.  The epilogue multiplies by 2^-(sA + sB), exactly.
__device__ __forceinline__ int f16_scale_exp(float m) {
  if (!(m > 0.f) || !(m <= 3.4028235e38f)) return 0;   // 0 (no kept row) or not finite
  return 15 - __builtin_amdgcn_frexp_expf(m);             // m = f 2^e, f in [0.5, 1)
}

// Compacted segment offsets by value (row j of expert e: seg_off[e] <= j <
// seg_off[e + 1]).
struct SegTable {
  int32_t E;
  int32_t off[kMaxE + 1];
};

__device__ __forceinline__ int expert_of_row(const SegTable& t, int j) {
  int lo = 0, hi = t.E - 1;   // last e with off[e] <= j
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (t.off[mid] <= j) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Launchers (return hipSuccess or the launch error).
// g has T rows; a row index outside [0, T) reads as a zero row.  rnorm (bf16
// storage, float16 weight-gradient mode; else null): per pair the Euclidean
// norms of the weight-gradient operand rows (A the g row, B the phi row,
// alpha on the phi side if alpha_on_phi, else on the g side).
hipError_t launch_score(int dtype, int mode, const void* g, const void* phi, const float* alpha,
                        const int32_t* row_index, int32_t P, int32_t T, int32_t d_out,
                        int32_t d_in, float* scores, hipStream_t s, float2* rnorm = nullptr,
                        int alpha_on_phi = 1);

// Bytes of the selection's workspace (digit histograms, select state and
// chunk counts of the chunked passes; 0 for the LDS path).
size_t select_workspace_bytes(const ExpertTable& tab);

// Per-expert top-quota selection and the compaction scan: keep flags, perm
// and seg_offsets.  ws: select_workspace_bytes(tab) bytes, 16-byte aligned;
// nothing in it needs to start at zero.  ebound (or null): float32 [E][2],
// the largest rnorm over each expert's kept pairs (0 for an expert that
// keeps nothing).
hipError_t launch_select(const ExpertTable& tab, const float* scores, uint8_t* keep,
                         int32_t* perm, int32_t* seg_offsets_out, uint32_t* ws, hipStream_t s,
                         const float2* rnorm = nullptr, float* ebound = nullptr);

hipError_t launch_plan_quota_device(const int32_t* ids, int32_t n_ids, int32_t E, int32_t mode,
                                    int64_t num, int64_t den, int64_t Q, int64_t* counts,
                                    int64_t* quotas, int64_t* seg_offsets, int64_t* invalid,
                                    hipStream_t s);

hipError_t launch_mask_alpha(int32_t P, const uint8_t* keep, const float* alpha,
                             float* alpha_masked, int32_t* perm_identity, hipStream_t s);

// Operand planes the gather may write in passing (bf16 storage): alpha[u] *
// (the kept row of phi if from_phi, else of g) as bf16 hi (+ lo) planes,
// [M, width], row j for compacted row j -- what launch_split would write
// from the compacted buffer -- and the GEMM's queue counters cleared.
struct GatherPlanes {
  uint16_t* hi = nullptr;   // nullptr: no planes
  uint16_t* lo = nullptr;
  bool from_phi = true;
  int32_t* zero = nullptr;
  int nzero = 0;
  // float16 weight-gradient mode instead: the planes of the g rows ([M,
  // d_out]) and of the phi rows ([M, d_in]), each scaled by its side's power
  // of two of the expert from ebound, alpha on the phi side if from_phi.  The
  // plane of the side without alpha may be null (the GEMM converts that
  // side's compacted bf16 rows itself).
  uint16_t* f16_g = nullptr;
  uint16_t* f16_phi = nullptr;
  float* ebound = nullptr;
  SegTable seg;
  // float16 mode: write the compacted rows and the planes with non-temporal
  // stores (when the grouped GEMM launch also clears the dropped dphi rows)
  bool stream_out = false;
};

// g has g_rows rows and phi phi_rows rows; a source row index outside them
// reads as a zero row.
hipError_t launch_gather(int dtype, const int32_t* perm, const uint8_t* keep,
                         const int32_t* g_row_index, const int32_t* phi_row_index,
                         const float* alpha, const void* g, const void* phi, void* g_c,
                         void* phi_c, float* alpha_c, float* dphi_zero, int32_t M,
                         int32_t P, int32_t g_rows, int32_t phi_rows, int32_t d_out,
                         int32_t d_in, hipStream_t s,
                         const GatherPlanes& planes = GatherPlanes());

// float16 weight-gradient mode without a score pass to take the bounds
// from: ebound[e] = the largest operand row norm over expert e's M rows
// (rn: M float2 of scratch), from the compacted rows (perm null: g = g_c,
// phi = phi_c, alpha = alpha_c, row j) or through perm from the source rows
// (bit for bit the score pass's per-pair norms either way).  Then
// launch_split_f16 writes the scaled float16 planes (either may be null)
// from the compacted bf16 rows, bit for bit what the gather writes in the
// one-call path.
hipError_t launch_expert_bounds(const SegTable& seg, const uint16_t* g, const uint16_t* phi,
                                const float* alpha, const int32_t* perm,
                                const int32_t* g_row_index, const int32_t* phi_row_index,
                                int32_t M, int32_t P, int32_t g_rows, int32_t phi_rows,
                                int32_t d_out, int32_t d_in, bool alpha_on_phi, float2* rn,
                                float* ebound, hipStream_t s);
hipError_t launch_split_f16(const SegTable& seg, const uint16_t* g_c, const uint16_t* phi_c,
                            const float* alpha_c, int32_t M, int32_t d_out, int32_t d_in,
                            bool alpha_on_phi, const float* ebound, uint16_t* f16_g,
                            uint16_t* f16_phi, hipStream_t s);

// hi (and lo, if non-null) bf16 planes of alpha[row] * src[row][col] (alpha
// may be null); src is bf16 or float32 storage.
hipError_t launch_split(int src_dtype, const void* src, int64_t rows, int32_t cols,
                        const float* alpha, uint16_t* hi, uint16_t* lo, hipStream_t s,
                        int32_t* zero = nullptr, int nzero = 0);

// Zeroes n int32 counters (a fill kernel, safe inside captured graphs).
hipError_t launch_zero(int32_t* p, int n, hipStream_t s);

hipError_t launch_grouped_backward(const GemmTable& tab, const GemmOperands& ops,
                                   const int32_t* perm, const float* alpha_c, float* dW,
                                   float* dphi, int32_t d_out, int32_t d_in, int32_t P,
                                   hipStream_t s);

// dW tiles of split experts: sum of the chunk partials, in chunk order.
hipError_t launch_reduce_partials(const GemmTable& tab, const float* partials, float* dW,
                                  int32_t d_out, int32_t d_in, hipStream_t s);

}  // namespace lrmoe
