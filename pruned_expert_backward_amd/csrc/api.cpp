// C-ABI entry points of liblrmoe: argument validation (all of it on the host,
// before any launch), host-side quota planning, the per-expert tables handed
// to kernels by value, and the stream-ordered launch sequence.
#include <string.h>

#include <algorithm>
#include <mutex>
#include <numeric>
#include <vector>

#include "lrmoe_internal.h"

using namespace lrmoe;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Pointer rules: a NULL pointer is accepted only for an empty array.
lrmoe_status need(const void* p, int64_t elems) {
  if (elems == 0) return LRMOE_OK;
  if (p == nullptr) return LRMOE_ERR_NULL;
  if (!aligned16(p)) return LRMOE_ERR_ALIGN;
  return LRMOE_OK;
}

lrmoe_status optional(const void* p) {
  if (p != nullptr && !aligned16(p)) return LRMOE_ERR_ALIGN;
  return LRMOE_OK;
}

#define LRMOE_TRY(x)                      \
  do {                                    \
    lrmoe_status _s = (x);                \
    if (_s != LRMOE_OK) return _s;        \
  } while (0)

struct Checked {
  int64_t M = 0;
  ExpertTable tab;
};

// Validates the problem description; fills the expert table.
lrmoe_status check_problem(const lrmoe_problem* pb, Checked& c) {
  if (pb == nullptr || pb->counts == nullptr || pb->quotas == nullptr) return LRMOE_ERR_NULL;
  if (pb->E < 1 || pb->E > kMaxE) return LRMOE_ERR_INVALID;
  if (pb->dtype != LRMOE_F32 && pb->dtype != LRMOE_BF16) return LRMOE_ERR_DTYPE;
  if (pb->dw_mode != LRMOE_DW_EXACT && pb->dw_mode != LRMOE_DW_BF16 &&
      pb->dw_mode != LRMOE_DW_F16)
    return LRMOE_ERR_INVALID;
  if (pb->score_mode < LRMOE_SCORE_LRM || pb->score_mode > LRMOE_SCORE_GRAD_L1)
    return LRMOE_ERR_INVALID;
  if (pb->P < 0 || pb->P >= (int64_t(1) << 31)) return LRMOE_ERR_SHAPE;
  if (pb->T < 0 || pb->T >= (int64_t(1) << 31)) return LRMOE_ERR_SHAPE;
  if (pb->d_out < 1 || pb->d_in < 1 || pb->d_out > (1 << 20) || pb->d_in > (1 << 20))
    return LRMOE_ERR_SHAPE;
  const int per = pb->dtype == LRMOE_BF16 ? 8 : 4;
  if (pb->d_out % per != 0 || pb->d_in % per != 0) return LRMOE_ERR_ALIGN;
  memset(&c.tab, 0, sizeof(c.tab));
  c.tab.E = pb->E;
  int64_t P = 0, M = 0;
  for (int e = 0; e < pb->E; ++e) {
    const int64_t n = pb->counts[e], q = pb->quotas[e];
    if (n < 0 || q < 0 || q > n) return LRMOE_ERR_INVALID;
    c.tab.pair_off[e] = (int32_t)P;
    c.tab.seg_off[e] = (int32_t)M;
    P += n;
    M += q;
    if (P >= (int64_t(1) << 31)) return LRMOE_ERR_SHAPE;
  }
  if (P != pb->P) return LRMOE_ERR_SHAPE;
  c.tab.pair_off[pb->E] = (int32_t)P;
  c.tab.seg_off[pb->E] = (int32_t)M;
  int32_t hc = 0;
  for (int e = 0; e < pb->E; ++e) {
    c.tab.chunk_off[e] = hc;
    hc += sel_chunks(pb->counts[e]);
  }
  c.tab.chunk_off[pb->E] = hc;
  c.tab.M = (int32_t)M;
  c.M = M;
  return LRMOE_OK;
}

size_t round256(size_t n) { return (n + 255) & ~size_t(255); }

// Workspace of lrmoe_grouped_backward: bf16 operand planes prepared by the
// prologue, then the fp32 partial dW tiles of experts split along K.
// bf16 storage: alpha times the narrower of g_c / phi_c, as hi + lo planes
// (exact) or hi only.  float32 storage: hi + lo planes of g_c, alpha*phi_c
// and W.  g_f32 (lrmoe_grouped_backward_gate_up: float32 g_c, bf16 phi_c and
// W): hi (+ lo) planes of alpha*g_c, read by both products.
struct GemmWorkspace {
  bool alpha_on_phi = true;
  size_t a_hi = 0, a_lo = 0, b_hi = 0, b_lo = 0, w_hi = 0, w_lo = 0, partials = 0, total = 0;
  int dw_pa = 1, dw_pb = 1, dp_pa = 1, dp_pb = 1;
  int32_t kc = 0;          // dW K-chunk length
  int64_t part_tiles = 0;  // partial tiles of split experts
  size_t heads = 0;        // work counters (kHeadCounters int32), then at +kEmaxOff ...
  bool f16 = false;        // float16 weight gradient: planes of g at a_hi, of phi at b_hi
  bool f16_g = false, f16_phi = false;   // ... which of the two exist
  size_t rnorm = 0;        // ... the per-expert bounds ebound; here per-pair row norms
};

// Float16 mode: the expert bounds (largest kept row norms) sit right behind
// the queue counters, so that one fill kernel clears both.
constexpr size_t kEmaxOff = 256;
constexpr size_t kHeadsBytes = kEmaxOff + 2 * kMaxE * sizeof(float);

constexpr int kStepK = 32;   // K rows per pipeline step of the GEMM kernel
// Workgroups of the grouped GEMM launch that start with the zero-fill of the
// dropped pairs' dphi rows (3 per XCD) instead of tiles.
constexpr int kZeroStarters = 24;
// The one-call paths clear the dropped pairs' dphi rows inside the grouped
// GEMM launch when those rows hold at least this many bytes (there the stores
// overlap the matrix-core work: 3.3 GB cost the launch 0.4 ms against 0.58 ms
// in the gather); smaller fills stay in the gather, where they cost less than
// the starters delay a short launch.
constexpr int64_t kZeroInGemmBytes = int64_t(512) << 20;
bool zero_in_gemm(const lrmoe_problem* pb, int64_t M) {
  return (pb->P - M) * (int64_t)pb->d_in * 4 >= kZeroInGemmBytes;
}

// Float16 mode: the weight-gradient tiles convert the operand without alpha
// from its compacted bf16 rows in registers (5 VALU instructions beside each
// MFMA) instead of reading a float16 plane of it, when the operand with
// alpha is at most this wide.  The conversion costs GEMM time in proportion
// to that width per kept row, while the plane it saves costs the gather a
// fixed amount per kept row: on the qwen3 down projection (768) the step got
// 6 % faster, on the GLM one (1408) 2 % slower.
constexpr int kF16ConvertMaxWidth = 1024;
bool f16_in_gemm(const lrmoe_problem* pb) {
  return std::min(pb->d_in, pb->d_out) <= kF16ConvertMaxWidth;
}

GemmWorkspace gemm_workspace(const lrmoe_problem* pb, int64_t M, bool g_f32 = false) {
  GemmWorkspace w;
  const size_t Mz = (size_t)M;
  if (!g_f32 && pb->dtype == LRMOE_BF16 && pb->dw_mode == LRMOE_DW_F16) {
    // queue counters and expert bounds, the score pass's per-pair row norms,
    // then the float16 planes of the weight-gradient operands: always the one
    // that carries alpha (the narrower), the other only where the GEMM does
    // not convert it from its bf16 rows (f16_in_gemm); the selection's
    // scratch of the one-call path goes where the planes will be, so that it
    // never meets the norms it runs beside
    w.f16 = true;
    w.alpha_on_phi = pb->d_in <= pb->d_out;
    const bool cvt = f16_in_gemm(pb);
    w.f16_g = !cvt || !w.alpha_on_phi;
    w.f16_phi = !cvt || w.alpha_on_phi;
    w.heads = 0;
    w.rnorm = kHeadsBytes;
    w.a_hi = round256(w.rnorm + (size_t)pb->P * 8);
    w.b_hi = w.a_hi + (w.f16_g ? round256(Mz * (size_t)pb->d_out * 2) : 0);
    w.total = w.b_hi + (w.f16_phi ? round256(Mz * (size_t)pb->d_in * 2) : 0);
  } else if (g_f32) {
    w.alpha_on_phi = false;
    const size_t plane = round256(Mz * (size_t)pb->d_out * 2);
    const bool exact = pb->dw_mode != LRMOE_DW_BF16;
    w.b_hi = 0;
    w.b_lo = plane;
    w.total = exact ? 2 * plane : plane;
    w.dw_pa = w.dp_pa = exact ? 2 : 1;
  } else if (pb->dtype == LRMOE_BF16) {
    w.alpha_on_phi = pb->d_in <= pb->d_out;
    const size_t plane = round256(Mz * (size_t)(w.alpha_on_phi ? pb->d_in : pb->d_out) * 2);
    const bool exact = pb->dw_mode == LRMOE_DW_EXACT;
    w.b_hi = 0;                 // offsets of the scaled operand's planes
    w.b_lo = plane;
    w.total = exact ? 2 * plane : plane;
    const int np = exact ? 2 : 1;
    w.dw_pa = w.alpha_on_phi ? 1 : np;
    w.dw_pb = w.alpha_on_phi ? np : 1;
  } else {
    w.alpha_on_phi = true;
    const size_t gpl = round256(Mz * (size_t)pb->d_out * 2);
    const size_t ppl = round256(Mz * (size_t)pb->d_in * 2);
    const size_t wpl = round256((size_t)pb->E * (size_t)pb->d_out * (size_t)pb->d_in * 2);
    w.a_hi = 0;
    w.a_lo = gpl;
    w.b_hi = 2 * gpl;
    w.b_lo = 2 * gpl + ppl;
    w.w_hi = 2 * gpl + 2 * ppl;
    w.w_lo = w.w_hi + wpl;
    w.total = w.w_lo + wpl;
    w.dw_pa = w.dw_pb = w.dp_pa = w.dp_pb = 2;
  }
  // K chunk: about one CU's share of the MFMA work (both products) per dW
  // tile chunk, and never under 1024 rows (fewer partial tiles); the many
  // shorter tiles fill in around the long ones.
  const int terms_dw = 1 + (w.dw_pa == 2) + (w.dw_pb == 2);
  const int terms_dp = 1 + (w.dp_pa == 2) + (w.dp_pb == 2);
  const int64_t tiles_n = (pb->d_in + kTile - 1) / kTile;
  const int64_t tiles_m = (pb->d_out + kTile - 1) / kTile;
  int64_t rows_steps = 0, mtiles = 0;
  for (int e = 0; e < pb->E; ++e) {
    rows_steps += (pb->quotas[e] + kStepK - 1) / kStepK;
    mtiles += (pb->quotas[e] + kTile - 1) / kTile;
  }
  const int64_t units = tiles_m * tiles_n * rows_steps * terms_dw +
                        tiles_n * mtiles * ((pb->d_out + kStepK - 1) / kStepK) * terms_dp;
  int64_t kc = units / 256 * kStepK / terms_dw;
  if (kc < 1024) kc = 1024;
  kc = (kc + kStepK - 1) / kStepK * kStepK;
  if (kc > (int64_t(1) << 30)) kc = int64_t(1) << 30;
  w.kc = (int32_t)kc;
  for (int e = 0; e < pb->E; ++e) {
    const int S = dw_chunks((int)pb->quotas[e], w.kc);
    if (S > 1) w.part_tiles += tiles_m * tiles_n * S;
  }
  w.partials = round256(w.total);
  if (w.f16) {   // counters and bounds were placed first
    w.total = w.partials + (size_t)w.part_tiles * kTile * kTile * 4;
    return w;
  }
  w.heads = w.partials + (size_t)w.part_tiles * kTile * kTile * 4;
  w.total = w.heads + kHeadsBytes;   // per-XCD queue counters of the grouped GEMM
  return w;
}

// Selection: three digit histograms and the select state per expert, two
// counts per chunk.
size_t select_workspace(const Checked& c) { return select_workspace_bytes(c.tab); }

// One size for every call of the problem: the selection, the grouped GEMMs,
// and (bf16 storage) the gate/up variant with a float32 output gradient.
size_t workspace_bytes(const lrmoe_problem* pb, const Checked& c) {
  const GemmWorkspace w = gemm_workspace(pb, c.M);
  // the one-call float16 path runs the selection in the plane region
  size_t n = std::max(w.total, (w.f16 ? w.a_hi : 0) + select_workspace(c));
  if (pb->dtype == LRMOE_BF16) n = std::max(n, gemm_workspace(pb, c.M, true).total);
  return n;
}

// Group shape gm x gn (gm * gn = kGroupSlots) over an expert's tile grid with
// nt column tiles.  A group reads gm row panels and gn column panels of equal
// size (256 operand rows or columns by the K extent), so the shape takes the
// least idle slots at the grid edge, then the least gm + gn, then gn nearest
// `pref`.
void group_shape(int nt, int pref, int32_t& gm, int32_t& gn) {
  const int cands[6] = {1, 2, 3, 4, 6, 12};
  int best = -1, best_waste = 1 << 30, best_sum = 1 << 30, best_dist = 1 << 30;
  for (int c : cands) {
    const int waste = ((nt + c - 1) / c) * c - nt;
    const int sum = c + kGroupSlots / c;
    const int dist = c > pref ? c - pref : pref - c;
    if (waste < best_waste || (waste == best_waste && sum < best_sum) ||
        (waste == best_waste && sum == best_sum && dist < best_dist)) {
      best = c;
      best_waste = waste;
      best_sum = sum;
      best_dist = dist;
    }
  }
  gn = best;
  gm = kGroupSlots / best;
}

lrmoe_status hip_status(hipError_t e) { return e == hipSuccess ? LRMOE_OK : LRMOE_ERR_HIP; }

// ---- Selection scratch for callers that cannot allocate
// (lrmoe_score_select_compact_noalloc).  A file-scope device array: every GPU
// the library runs on holds its own copy of kScratchBytes until the process
// ends.  In host code `scratch` names a host-side stand-in, not device
// memory, so kernels get the address hipGetSymbolAddress returns for the
// current device, looked up once per device and kept.
constexpr size_t kScratchBytes = size_t(8) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

lrmoe_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LRMOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return LRMOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LRMOE_OK;
}

// Records the caller's event of one timing slot (if any) on the stream.
lrmoe_status mark(const lrmoe_timing* t, bool after, int slot, hipStream_t s) {
  if (t == nullptr) return LRMOE_OK;
  void* ev = after ? t->after[slot] : t->before[slot];
  if (ev == nullptr) return LRMOE_OK;
  return hip_status(hipEventRecord(reinterpret_cast<hipEvent_t>(ev), s));
}

// Shared body of the two select entry points.
lrmoe_status select_compact(const lrmoe_problem* pb, bool compute_scores, const float* scores_in,
                            const int32_t* g_row_index, const float* alpha, const void* g,
                            const void* phi, float* scores_out, uint8_t* keep,
                            int32_t* seg_offsets, int32_t* perm, void* g_c, void* phi_c,
                            float* alpha_c, float* dphi_zero, void* workspace, size_t ws_bytes,
                            void* stream, const lrmoe_timing* timing, bool gather = true,
                            const GatherPlanes& planes = GatherPlanes(),
                            bool use_scratch = false, float2* rnorm = nullptr,
                            float* ebound = nullptr) {
  Checked c;
  LRMOE_TRY(check_problem(pb, c));
  const int64_t P = pb->P, M = c.M;
  if (g_row_index == nullptr && pb->T != P) return LRMOE_ERR_SHAPE;
  // g rows are read by the score pass (every pair) and by the gather (kept pairs)
  const bool reads_g = P > 0 && (compute_scores || (gather && M > 0));
  if (reads_g && pb->T < 1) return LRMOE_ERR_SHAPE;
  LRMOE_TRY(need(alpha, P));
  LRMOE_TRY(need(g, reads_g ? pb->T : 0));
  LRMOE_TRY(need(phi, P));
  LRMOE_TRY(optional(g_row_index));
  if (compute_scores) {
    LRMOE_TRY(need(scores_out, P));
  } else {
    LRMOE_TRY(need(scores_in, P));
  }
  LRMOE_TRY(need(keep, P));
  LRMOE_TRY(need(seg_offsets, pb->E + 1));
  LRMOE_TRY(need(perm, M));
  if (gather) {
    LRMOE_TRY(need(g_c, M));
    LRMOE_TRY(need(phi_c, M));
    LRMOE_TRY(need(alpha_c, M));
    LRMOE_TRY(optional(dphi_zero));
  }
  const size_t ws_need = select_workspace(c);   // 0 unless an expert is above kSelLdsKeys
  if (use_scratch) {   // the library's static scratch instead of a workspace
    if (ws_need > kScratchBytes) return LRMOE_ERR_SCRATCH;
    LRMOE_TRY(scratch_address(&workspace));
    ws_bytes = kScratchBytes;
  } else if (ws_need > 0) {
    LRMOE_TRY(need(workspace, 1));
    if (ws_bytes < ws_need) return LRMOE_ERR_WORKSPACE;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const float* scores = scores_in;
  if (compute_scores) {
    LRMOE_TRY(mark(timing, false, 0, s));
    LRMOE_TRY(hip_status(launch_score(pb->dtype, pb->score_mode, g, phi, alpha, g_row_index,
                                      (int32_t)P, (int32_t)pb->T, pb->d_out, pb->d_in,
                                      scores_out, s, rnorm, planes.from_phi ? 1 : 0)));
    LRMOE_TRY(mark(timing, true, 0, s));
    scores = scores_out;
  }
  LRMOE_TRY(mark(timing, false, 1, s));
  LRMOE_TRY(hip_status(launch_select(c.tab, scores, keep, perm, seg_offsets,
                                     reinterpret_cast<uint32_t*>(workspace), s, rnorm, ebound)));
  LRMOE_TRY(mark(timing, true, 1, s));
  if (!gather) return LRMOE_OK;
  LRMOE_TRY(mark(timing, false, 2, s));
  LRMOE_TRY(hip_status(launch_gather(pb->dtype, perm, keep, g_row_index, nullptr, alpha, g, phi,
                                     g_c, phi_c, alpha_c, dphi_zero, (int32_t)M, (int32_t)P,
                                     (int32_t)pb->T, (int32_t)P, pb->d_out, pb->d_in, s,
                                     planes)));
  LRMOE_TRY(mark(timing, true, 2, s));
  return LRMOE_OK;
}

// Shared body of the grouped-backward entry points.  glu: the SiLU-GLU chain
// (dphi is then nullptr and the input-gradient tiles write the compacted
// gate/up output gradient glu_out instead; with no kept pair at all there is
// nothing to write and the pointers may be NULL).
// planes_ready: the gather already wrote the bf16 operand planes (and
// cleared the queue counters), so no prologue runs.  Timing slots: sp
// (prologue), sp + 1 (GEMM), sp + 2 (reduction), or for the whole-path call
// the slots of TimingSlots.
struct TimingSlots {
  int prologue = 0, gemm = 1, reduce = 2;
};

// g_f32: g_c is float32 while phi_c and W are bf16 (the gate/up projection of
// the MLP chain on the float32 output gradient of the SiLU-GLU epilogue).
lrmoe_status grouped_backward(const lrmoe_problem* pb, const int32_t* perm, const float* alpha_c,
                              const void* g_c, const void* phi_c, const void* W, float* dW,
                              float* dphi, bool glu, const uint16_t* glu_a,
                              const uint16_t* glu_b, void* glu_out, void* workspace,
                              size_t ws_bytes, void* stream, const lrmoe_timing* timing,
                              bool planes_ready = false, TimingSlots ts = TimingSlots(),
                              bool g_f32 = false, const uint8_t* zero_keep = nullptr) {
  Checked c;
  LRMOE_TRY(check_problem(pb, c));
  if (g_f32 && pb->dtype != LRMOE_BF16) return LRMOE_ERR_DTYPE;
  const int64_t M = c.M;
  LRMOE_TRY(need(alpha_c, M));
  LRMOE_TRY(need(g_c, M));
  LRMOE_TRY(need(phi_c, M));
  LRMOE_TRY(need(W, 1));
  LRMOE_TRY(need(dW, 1));
  LRMOE_TRY(optional(dphi));
  if (glu) {
    LRMOE_TRY(need(glu_a, M > 0 ? pb->P : 0));
    LRMOE_TRY(need(glu_b, M > 0 ? pb->P : 0));
    LRMOE_TRY(need(glu_out, M));
    if (M == 0) glu_out = nullptr;   // no input-gradient tile: the plain kernel runs
  }
  if (dphi != nullptr || glu) LRMOE_TRY(need(perm, M));
  const GemmWorkspace wl = gemm_workspace(pb, M, g_f32);
  if (ws_bytes < workspace_bytes(pb, c)) return LRMOE_ERR_WORKSPACE;
  LRMOE_TRY(need(workspace, (int64_t)wl.total));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  const int E = pb->E;
  const int d_out = pb->d_out, d_in = pb->d_in;
  GemmTable t;
  memset(&t, 0, sizeof(t));
  t.E = E;
  t.tiles_n = (d_in + kTile - 1) / kTile;
  t.dw_tiles_m = (d_out + kTile - 1) / kTile;
  t.kc = wl.kc;
  group_shape(t.tiles_n, 3, t.dw_gm, t.dw_gn);
  group_shape(t.tiles_n, 3, t.dp_gm, t.dp_gn);
  // a last column of at most 128 columns: 512 x 128 input-gradient tiles
  // there, none of them half empty (the SiLU-GLU epilogue keeps square tiles)
  t.tall = !glu && d_in % kTile != 0 && d_in % kTile <= kTile / 2;
  for (int e = 0; e <= E; ++e) t.seg_off[e] = c.tab.seg_off[e];

  // Groups.  Weight gradient: every expert (zeros for q_e = 0) and K chunk;
  // input gradient: the experts' row tiles.  Work of a group ~ tiles x K steps
  // x MFMA passes.
  std::vector<int> order(E);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int a, int b) { return pb->quotas[a] > pb->quotas[b]; });
  const int ngn_dw = (t.tiles_n + t.dw_gn - 1) / t.dw_gn;
  const int per_chunk = ((t.dw_tiles_m + t.dw_gm - 1) / t.dw_gm) * ngn_dw;
  const int ngn_dp = (t.tiles_n + t.dp_gn - 1) / t.dp_gn;
  const int terms_dw = 1 + (wl.dw_pa == 2) + (wl.dw_pb == 2);
  const int terms_dp = 1 + (wl.dp_pa == 2) + (wl.dp_pb == 2);
  struct G { int64_t work; uint32_t desc; };
  std::vector<G> groups;
  int32_t g = 0;
  for (int r = 0; r < E; ++r) {
    const int e = order[r];
    const int q = (int)pb->quotas[e];
    const int S = dw_chunks(q, t.kc);
    t.f.dw_goff[r] = g;
    t.f.order[r] = (uint8_t)e;
    g += per_chunk * S;
    for (int ch = 0; ch < S; ++ch) {
      const int klen = S > 1 ? std::min(t.kc, q - ch * t.kc) : q;
      for (int sg = 0; sg < per_chunk; ++sg)
        groups.push_back({(int64_t)((klen + kStepK - 1) / kStepK + 1) * terms_dw * kGroupSlots,
                          group_desc(true, e, ch, sg)});
    }
  }
  t.f.dw_goff[E] = g;
  t.dw_groups = g;
  for (int e = 0; e < E; ++e) {
    t.f.dp_goff[e] = g;
    if (dphi == nullptr && !glu) continue;
    const int64_t mt = (pb->quotas[e] + kTile - 1) / kTile;
    const int n = (int)(((mt + t.dp_gm - 1) / t.dp_gm) * ngn_dp);
    g += n;
    for (int sg = 0; sg < n; ++sg)
      groups.push_back({(int64_t)((d_out + kStepK - 1) / kStepK + 1) * terms_dp * kGroupSlots,
                        group_desc(false, e, 0, sg)});
  }
  t.f.dp_goff[E] = g;
  t.total_groups = g;
  bool table_ok = (int)groups.size() <= kMaxGroups && E <= 256;
  for (int e = 0; e < E && table_ok; ++e) table_ok = dw_chunks((int)pb->quotas[e], t.kc) <= 256;
  if (table_ok) {
    // Longest first, each to the XCD with the least work so far; queues keep
    // that order.  (The formula-order tables above are overwritten: union.)
    std::vector<int> idx(groups.size());
    std::iota(idx.begin(), idx.end(), 0);
    std::stable_sort(idx.begin(), idx.end(),
                     [&](int a, int b) { return groups[a].work > groups[b].work; });
    std::vector<std::vector<uint32_t>> qs(kXcds);
    int64_t load[kXcds] = {0};
    for (int i : idx) {
      int best = 0;
      for (int x = 1; x < kXcds; ++x)
        if (load[x] < load[best]) best = x;
      load[best] += groups[i].work;
      qs[best].push_back(groups[i].desc);
    }
    t.use_table = 1;
    int32_t o = 0;
    for (int x = 0; x < kXcds; ++x) {
      t.qoff[x] = o;
      for (uint32_t d : qs[x]) t.groups[o++] = d;
    }
    t.qoff[kXcds] = o;
  }

  // Prologue: bf16 operand planes (unless the gather wrote them).
  if (!planes_ready) LRMOE_TRY(mark(timing, false, ts.prologue, s));
  char* ws = reinterpret_cast<char*>(workspace);
  auto plane = [&](size_t off) { return reinterpret_cast<uint16_t*>(ws + off); };
  int32_t* heads = reinterpret_cast<int32_t*>(ws + wl.heads);
  GemmOperands ops;
  memset(&ops, 0, sizeof(ops));
  const uint16_t* g16 = reinterpret_cast<const uint16_t*>(g_c);
  const uint16_t* p16 = reinterpret_cast<const uint16_t*>(phi_c);
  const uint16_t* w16 = reinterpret_cast<const uint16_t*>(W);
  float* ebound = reinterpret_cast<float*>(ws + wl.heads + kEmaxOff);
  if (wl.f16) {
    // float16 planes, scaled per expert by the powers of two of the kept
    // rows' largest norms (the gather wrote them in the one-call path; here:
    // clear the counters, then the bounds from the compacted rows, then the
    // planes); a missing plane is converted from the bf16 rows by the kernel
    uint16_t* fg = wl.f16_g ? plane(wl.a_hi) : nullptr;
    uint16_t* fp = wl.f16_phi ? plane(wl.b_hi) : nullptr;
    if (!planes_ready) {
      SegTable seg;
      seg.E = E;
      for (int e = 0; e <= E; ++e) seg.off[e] = c.tab.seg_off[e];
      const uint16_t* gc16 = reinterpret_cast<const uint16_t*>(g_c);
      const uint16_t* pc16 = reinterpret_cast<const uint16_t*>(phi_c);
      LRMOE_TRY(hip_status(launch_zero(heads, kHeadCounters, s)));
      LRMOE_TRY(hip_status(launch_expert_bounds(
          seg, gc16, pc16, alpha_c, nullptr, nullptr, nullptr, (int32_t)M, (int32_t)M,
          (int32_t)M, (int32_t)M, d_out, d_in, wl.alpha_on_phi,
          reinterpret_cast<float2*>(ws + wl.rnorm), ebound, s)));
      LRMOE_TRY(hip_status(launch_split_f16(seg, gc16, pc16, alpha_c, (int32_t)M, d_out, d_in,
                                            wl.alpha_on_phi, ebound, fg, fp, s)));
    }
    ops.dw_a[0] = fg != nullptr ? fg : g16;
    ops.dw_b[0] = fp != nullptr ? fp : p16;
    ops.dw_pa = ops.dw_pb = 1;
    ops.dp_a[0] = g16;
    ops.dp_b[0] = w16;
    ops.dp_pa = ops.dp_pb = 1;
    ops.dw_f16 = fg == nullptr ? 1 : fp == nullptr ? 2 : 3;
    ops.dw_ebound = ebound;
  } else if (g_f32) {
    // alpha * g_c (float32) as bf16 hi (+ lo) planes, the A operand of both
    // products; the input-gradient epilogue then applies no alpha
    uint16_t* hi = plane(wl.b_hi);
    uint16_t* lo = wl.dw_pa == 2 ? plane(wl.b_lo) : nullptr;
    LRMOE_TRY(hip_status(launch_split(LRMOE_F32, g_c, M, d_out, alpha_c, hi, lo, s, heads, kHeadCounters)));
    ops.dw_a[0] = ops.dp_a[0] = hi;
    ops.dw_a[1] = ops.dp_a[1] = lo;
    ops.dw_b[0] = p16;
    ops.dp_b[0] = w16;
    ops.dw_pa = ops.dp_pa = wl.dw_pa;
    ops.dw_pb = ops.dp_pb = 1;
    ops.dp_alpha_folded = 1;
  } else if (pb->dtype == LRMOE_BF16) {
    const bool exact = pb->dw_mode == LRMOE_DW_EXACT;
    uint16_t* hi = plane(wl.b_hi);
    uint16_t* lo = exact ? plane(wl.b_lo) : nullptr;
    const void* src = wl.alpha_on_phi ? phi_c : g_c;
    const int cols = wl.alpha_on_phi ? d_in : d_out;
    if (!planes_ready)
      LRMOE_TRY(hip_status(launch_split(LRMOE_BF16, src, M, cols, alpha_c, hi, lo, s, heads, kHeadCounters)));
    if (wl.alpha_on_phi) {
      ops.dw_a[0] = g16;
      ops.dw_b[0] = hi;
      ops.dw_b[1] = lo;
    } else {
      ops.dw_a[0] = hi;
      ops.dw_a[1] = lo;
      ops.dw_b[0] = p16;
    }
    ops.dw_pa = wl.dw_pa;
    ops.dw_pb = wl.dw_pb;
    ops.dp_a[0] = g16;
    ops.dp_b[0] = w16;
    ops.dp_pa = ops.dp_pb = 1;
  } else {
    LRMOE_TRY(hip_status(launch_split(LRMOE_F32, g_c, M, d_out, nullptr, plane(wl.a_hi),
                                      plane(wl.a_lo), s, heads, kHeadCounters)));
    LRMOE_TRY(hip_status(launch_split(LRMOE_F32, phi_c, M, d_in, alpha_c, plane(wl.b_hi),
                                      plane(wl.b_lo), s)));
    if (dphi != nullptr)
      LRMOE_TRY(hip_status(launch_split(LRMOE_F32, W, (int64_t)E * d_out, d_in, nullptr,
                                        plane(wl.w_hi), plane(wl.w_lo), s)));
    ops.dw_a[0] = ops.dp_a[0] = plane(wl.a_hi);
    ops.dw_a[1] = ops.dp_a[1] = plane(wl.a_lo);
    ops.dw_b[0] = plane(wl.b_hi);
    ops.dw_b[1] = plane(wl.b_lo);
    ops.dp_b[0] = plane(wl.w_hi);
    ops.dp_b[1] = plane(wl.w_lo);
    ops.dw_pa = ops.dw_pb = ops.dp_pa = ops.dp_pb = 2;
  }
  (void)w16;
  if (!planes_ready) LRMOE_TRY(mark(timing, true, ts.prologue, s));
  ops.partials = reinterpret_cast<float*>(ws + wl.partials);
  ops.queue_heads = heads;   // cleared by the first prologue launch
  ops.glu_a = glu_a;
  ops.glu_b = glu_b;
  ops.glu_out = glu_out;
  ops.glu_f32 = pb->dw_mode != LRMOE_DW_BF16;   // exact modes hand dgu on unrounded
  if (zero_keep != nullptr && dphi != nullptr && !glu) {
    // the dropped pairs' dphi rows are cleared inside the launch, beside the
    // tiles: kZeroStarters workgroups start with them, the rest join later
    ops.zero_keep = zero_keep;
    ops.zero_rows = dphi;
    ops.zero_first = kZeroStarters;
  }
  LRMOE_TRY(mark(timing, false, ts.gemm, s));
  LRMOE_TRY(hip_status(launch_grouped_backward(t, ops, perm, alpha_c, dW, dphi, d_out, d_in,
                                               (int32_t)pb->P, s)));
  LRMOE_TRY(mark(timing, true, ts.gemm, s));
  // the reduction runs only when an expert's weight gradient was split along
  // K; otherwise its timing events stay unrecorded, like those of any kernel
  // a call does not launch
  bool split = false;
  for (int e = 0; e < E && !split; ++e) split = dw_chunks((int)pb->quotas[e], t.kc) > 1;
  if (split) LRMOE_TRY(mark(timing, false, ts.reduce, s));
  LRMOE_TRY(hip_status(launch_reduce_partials(t, ops.partials, dW, d_out, d_in, s)));
  if (split) LRMOE_TRY(mark(timing, true, ts.reduce, s));
  return LRMOE_OK;
}

// The whole path in one call.  bf16 storage: the gather writes the GEMM's
// operand planes from the rows it moves (no prologue kernel reads the
// compacted operand again); float32 storage: the separate steps.
lrmoe_status pruned_backward(const lrmoe_problem* pb, const int32_t* g_row_index,
                             const float* alpha, const void* g, const void* phi, const void* W,
                             float* scores, uint8_t* keep, int32_t* seg_offsets, int32_t* perm,
                             void* g_c, void* phi_c, float* alpha_c, float* dW, float* dphi,
                             void* workspace, size_t ws_bytes, void* stream,
                             const lrmoe_timing* timing) {
  Checked c;
  LRMOE_TRY(check_problem(pb, c));
  const int64_t M = c.M;
  LRMOE_TRY(need(W, 1));
  LRMOE_TRY(need(dW, 1));
  const GemmWorkspace wl = gemm_workspace(pb, M);
  if (ws_bytes < workspace_bytes(pb, c)) return LRMOE_ERR_WORKSPACE;
  LRMOE_TRY(need(workspace, (int64_t)wl.total));
  GatherPlanes planes;
  const bool fused = pb->dtype == LRMOE_BF16;
  float2* rnorm = nullptr;
  float* ebound = nullptr;
  if (fused) {
    char* ws = reinterpret_cast<char*>(workspace);
    planes.from_phi = wl.alpha_on_phi;
    planes.zero = reinterpret_cast<int32_t*>(ws + wl.heads);
    planes.nzero = kHeadCounters;
    if (wl.f16) {
      // the score pass writes per-pair row norms, the select reduces them
      // over each expert's kept pairs, the gather writes the float16 planes
      rnorm = reinterpret_cast<float2*>(ws + wl.rnorm);
      ebound = reinterpret_cast<float*>(ws + wl.heads + kEmaxOff);
      if (wl.f16_g) planes.f16_g = reinterpret_cast<uint16_t*>(ws + wl.a_hi);
      if (wl.f16_phi) planes.f16_phi = reinterpret_cast<uint16_t*>(ws + wl.b_hi);
      planes.ebound = ebound;
      planes.seg.E = pb->E;
      for (int e = 0; e <= pb->E; ++e) planes.seg.off[e] = c.tab.seg_off[e];
    } else {
      planes.hi = reinterpret_cast<uint16_t*>(ws + wl.b_hi);
      planes.lo = pb->dw_mode == LRMOE_DW_EXACT ? reinterpret_cast<uint16_t*>(ws + wl.b_lo)
                                                : nullptr;
    }
  }
  // float16: the selection's scratch sits where the planes will be (the
  // counters and bounds come first).  The dropped pairs' dphi rows are
  // cleared by the gather, or (large fills) by the grouped GEMM launch, where
  // the stores overlap the matrix-core work.
  const size_t sel_off = wl.f16 ? wl.a_hi : 0;
  LRMOE_TRY(optional(dphi));
  const bool zfill = dphi != nullptr && zero_in_gemm(pb, M);
  planes.stream_out = zfill;
  LRMOE_TRY(select_compact(pb, true, nullptr, g_row_index, alpha, g, phi, scores, keep,
                           seg_offsets, perm, g_c, phi_c, alpha_c, zfill ? nullptr : dphi,
                           reinterpret_cast<char*>(workspace) + sel_off, ws_bytes - sel_off,
                           stream, timing, true, planes, false, rnorm, ebound));
  TimingSlots ts;
  ts.gemm = 3;
  ts.reduce = 4;
  ts.prologue = 5;
  return grouped_backward(pb, perm, alpha_c, g_c, phi_c, W, dW, dphi, false, nullptr, nullptr,
                          nullptr, workspace, ws_bytes, stream, timing, fused, ts, false,
                          zfill ? keep : nullptr);
}


// Validation of a gather on an inherited keep set (every host-detectable
// problem); phi_rows: the rows of phi its row index may address.
lrmoe_status check_gather(const lrmoe_problem* pb, const Checked& c, const int32_t* perm,
                          const uint8_t* keep, const int32_t* g_row_index,
                          const int32_t* phi_row_index, const float* alpha, const void* g,
                          const void* phi, void* g_c, void* phi_c, float* alpha_c,
                          float* dphi_zero, const GatherPlanes& planes, int64_t& phi_rows) {
  const int64_t P = pb->P, M = c.M;
  const bool with_g = g != nullptr || g_c != nullptr;   // both NULL: phi rows only
  if (with_g && g_row_index == nullptr && pb->T != P) return LRMOE_ERR_SHAPE;
  if (with_g && M > 0 && pb->T < 1) return LRMOE_ERR_SHAPE;
  // rows of phi: T_phi through a row index, else one per pair
  phi_rows = phi_row_index != nullptr ? pb->T_phi : P;
  if (phi_row_index != nullptr && M > 0 &&
      (pb->T_phi < 1 || pb->T_phi >= (int64_t(1) << 31)))
    return LRMOE_ERR_SHAPE;
  LRMOE_TRY(need(perm, M));
  LRMOE_TRY(need(alpha, P));
  if (with_g) {
    LRMOE_TRY(need(g, M > 0 ? pb->T : 0));
    LRMOE_TRY(need(g_c, M));
  }
  LRMOE_TRY(need(phi, M > 0 ? phi_rows : 0));
  LRMOE_TRY(optional(g_row_index));
  LRMOE_TRY(optional(phi_row_index));
  LRMOE_TRY(need(phi_c, M));
  LRMOE_TRY(need(alpha_c, M));
  LRMOE_TRY(optional(dphi_zero));
  if (dphi_zero != nullptr) LRMOE_TRY(need(keep, P));
  if ((planes.hi != nullptr || planes.f16_g != nullptr || planes.f16_phi != nullptr) && !with_g)
    return LRMOE_ERR_NULL;
  return LRMOE_OK;
}

lrmoe_status launch_gather_timed(const lrmoe_problem* pb, const Checked& c, const int32_t* perm,
                                 const uint8_t* keep, const int32_t* g_row_index,
                                 const int32_t* phi_row_index, const float* alpha,
                                 const void* g, const void* phi, void* g_c, void* phi_c,
                                 float* alpha_c, float* dphi_zero, int64_t phi_rows,
                                 hipStream_t s, const lrmoe_timing* timing,
                                 const GatherPlanes& planes) {
  LRMOE_TRY(mark(timing, false, 2, s));
  LRMOE_TRY(hip_status(launch_gather(pb->dtype, perm, keep, g_row_index, phi_row_index, alpha, g,
                                     phi, g_c, phi_c, alpha_c, dphi_zero, (int32_t)c.M,
                                     (int32_t)pb->P, (int32_t)pb->T, (int32_t)phi_rows,
                                     pb->d_out, pb->d_in, s, planes)));
  return mark(timing, true, 2, s);
}

lrmoe_status gather_compact(const lrmoe_problem* pb, const int32_t* perm, const uint8_t* keep,
                            const int32_t* g_row_index, const int32_t* phi_row_index,
                            const float* alpha, const void* g, const void* phi, void* g_c,
                            void* phi_c, float* alpha_c, float* dphi_zero, void* stream,
                            const lrmoe_timing* timing, const GatherPlanes& planes) {
  Checked c;
  LRMOE_TRY(check_problem(pb, c));
  int64_t phi_rows = 0;
  LRMOE_TRY(check_gather(pb, c, perm, keep, g_row_index, phi_row_index, alpha, g, phi, g_c, phi_c,
                         alpha_c, dphi_zero, planes, phi_rows));
  return launch_gather_timed(pb, c, perm, keep, g_row_index, phi_row_index, alpha, g, phi, g_c,
                             phi_c, alpha_c, dphi_zero, phi_rows,
                             reinterpret_cast<hipStream_t>(stream), timing, planes);
}

// Step 4 + step 5 for a projection on an inherited keep set: the gather also
// writes the GEMM's operand planes (bf16 storage), then the grouped GEMMs.
lrmoe_status gather_backward(const lrmoe_problem* pb, const int32_t* perm, const uint8_t* keep,
                             const int32_t* g_row_index, const int32_t* phi_row_index,
                             const float* alpha, const void* g, const void* phi, const void* W,
                             void* g_c, void* phi_c, float* alpha_c, float* dW, float* dphi,
                             void* workspace, size_t ws_bytes, void* stream,
                             const lrmoe_timing* timing) {
  Checked c;
  LRMOE_TRY(check_problem(pb, c));
  LRMOE_TRY(need(W, 1));
  LRMOE_TRY(need(dW, 1));
  if (c.M > 0 && pb->T < 1) return LRMOE_ERR_SHAPE;
  LRMOE_TRY(need(g, c.M > 0 ? pb->T : 0));   // the GEMM needs g rows: no NULL g here
  LRMOE_TRY(need(g_c, c.M));
  const GemmWorkspace wl = gemm_workspace(pb, c.M);
  if (ws_bytes < workspace_bytes(pb, c)) return LRMOE_ERR_WORKSPACE;
  LRMOE_TRY(need(workspace, (int64_t)wl.total));
  GatherPlanes planes;
  const bool fused = pb->dtype == LRMOE_BF16;   // the gather writes the GEMM's planes
  char* ws = reinterpret_cast<char*>(workspace);
  if (fused) {
    planes.from_phi = wl.alpha_on_phi;
    planes.zero = reinterpret_cast<int32_t*>(ws + wl.heads);
    planes.nzero = kHeadCounters;
    if (wl.f16) {
      if (wl.f16_g) planes.f16_g = reinterpret_cast<uint16_t*>(ws + wl.a_hi);
      if (wl.f16_phi) planes.f16_phi = reinterpret_cast<uint16_t*>(ws + wl.b_hi);
      planes.ebound = reinterpret_cast<float*>(ws + wl.heads + kEmaxOff);
      planes.seg.E = pb->E;
      for (int e = 0; e <= pb->E; ++e) planes.seg.off[e] = c.tab.seg_off[e];
    } else {
      planes.hi = reinterpret_cast<uint16_t*>(ws + wl.b_hi);
      planes.lo = pb->dw_mode == LRMOE_DW_EXACT ? reinterpret_cast<uint16_t*>(ws + wl.b_lo)
                                                : nullptr;
    }
  }
  int64_t phi_rows = 0;
  LRMOE_TRY(check_gather(pb, c, perm, keep, g_row_index, phi_row_index, alpha, g, phi, g_c, phi_c,
                         alpha_c, dphi, planes, phi_rows));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  TimingSlots ts;
  ts.gemm = 3;
  ts.reduce = 4;
  ts.prologue = 5;
  if (fused && wl.f16) {
    // float16 planes: no score pass to take the expert bounds from, so they
    // come from the source rows the gather is about to copy (slot 5)
    LRMOE_TRY(mark(timing, false, ts.prologue, s));
    LRMOE_TRY(hip_status(launch_expert_bounds(
        planes.seg, reinterpret_cast<const uint16_t*>(g), reinterpret_cast<const uint16_t*>(phi),
        alpha, perm, g_row_index, phi_row_index, (int32_t)c.M, (int32_t)pb->P, (int32_t)pb->T,
        (int32_t)phi_rows, pb->d_out, pb->d_in, wl.alpha_on_phi,
        reinterpret_cast<float2*>(ws + wl.rnorm), planes.ebound, s)));
    LRMOE_TRY(mark(timing, true, ts.prologue, s));
  }
  // the dropped pairs' dphi rows: cleared by the gather, or (large fills)
  // inside the grouped GEMM launch
  const bool zfill = dphi != nullptr && zero_in_gemm(pb, c.M);
  planes.stream_out = zfill;
  LRMOE_TRY(launch_gather_timed(pb, c, perm, keep, g_row_index, phi_row_index, alpha, g, phi, g_c,
                                phi_c, alpha_c, zfill ? nullptr : dphi, phi_rows, s, timing,
                                planes));
  return grouped_backward(pb, perm, alpha_c, g_c, phi_c, W, dW, dphi, false, nullptr, nullptr,
                          nullptr, workspace, ws_bytes, stream, timing, fused, ts, false,
                          zfill ? keep : nullptr);
}

}  // namespace

extern "C" {

int32_t lrmoe_abi_version(void) { return LRMOE_ABI_VERSION; }

const char* lrmoe_status_string(lrmoe_status s) {
  switch (s) {
    case LRMOE_OK: return "ok";
    case LRMOE_ERR_NULL: return "a required pointer is NULL";
    case LRMOE_ERR_INVALID: return "invalid expert count, quota, policy or mode";
    case LRMOE_ERR_SHAPE: return "inconsistent or out-of-range sizes";
    case LRMOE_ERR_ALIGN: return "pointer not 16-byte aligned or row length not a multiple of 16 bytes";
    case LRMOE_ERR_DTYPE: return "unknown storage dtype";
    case LRMOE_ERR_WORKSPACE: return "workspace too small";
    case LRMOE_ERR_HIP: return "HIP runtime error";
    case LRMOE_ERR_SCRATCH: return "problem needs more selection scratch than the library's static buffer holds";
  }
  return "unknown status";
}

lrmoe_status lrmoe_plan_quota(int32_t E, const int64_t* counts, const lrmoe_quota_policy* policy,
                              int64_t* quotas_out) {
  if (counts == nullptr || policy == nullptr || quotas_out == nullptr) return LRMOE_ERR_NULL;
  if (E < 1 || E > kMaxE) return LRMOE_ERR_INVALID;
  int64_t P = 0;
  for (int e = 0; e < E; ++e) {
    if (counts[e] < 0 || counts[e] >= (int64_t(1) << 31)) return LRMOE_ERR_INVALID;
    P += counts[e];
  }
  if (policy->mode == LRMOE_QUOTA_RATIO) {
    const int64_t num = policy->num, den = policy->den;
    if (den <= 0 || num < 0 || num > den || den >= (int64_t(1) << 31)) return LRMOE_ERR_INVALID;
    for (int e = 0; e < E; ++e) quotas_out[e] = (counts[e] * num) / den;
  } else if (policy->mode == LRMOE_QUOTA_BUDGET) {
    const int64_t Q = policy->budget_pairs;
    if (Q < 0) return LRMOE_ERR_INVALID;
    for (int e = 0; e < E; ++e) {
      if (P == 0 || Q >= P) {
        quotas_out[e] = counts[e];
      } else {
        // n_e * Q < 2^31 * 2^31: exact in unsigned 128-bit arithmetic
        const unsigned __int128 prod = (unsigned __int128)counts[e] * (unsigned __int128)Q;
        quotas_out[e] = (int64_t)(prod / (unsigned __int128)P);
      }
    }
  } else {
    return LRMOE_ERR_INVALID;
  }
  return LRMOE_OK;
}

lrmoe_status lrmoe_plan_quota_device(int32_t E, const int32_t* expert_ids, int64_t n_ids,
                                     const lrmoe_quota_policy* policy, int64_t* counts_out,
                                     int64_t* quotas_out, int64_t* seg_offsets_out,
                                     int64_t* invalid_out, void* stream) {
  if (policy == nullptr) return LRMOE_ERR_NULL;
  if (E < 1 || E > kMaxE) return LRMOE_ERR_INVALID;
  if (n_ids < 0 || n_ids >= (int64_t(1) << 31)) return LRMOE_ERR_SHAPE;
  if (policy->mode == LRMOE_QUOTA_RATIO) {
    if (policy->den <= 0 || policy->num < 0 || policy->num > policy->den ||
        policy->den >= (int64_t(1) << 31))
      return LRMOE_ERR_INVALID;
  } else if (policy->mode == LRMOE_QUOTA_BUDGET) {
    if (policy->budget_pairs < 0) return LRMOE_ERR_INVALID;
  } else {
    return LRMOE_ERR_INVALID;
  }
  LRMOE_TRY(need(expert_ids, n_ids));
  LRMOE_TRY(need(counts_out, E));
  LRMOE_TRY(need(quotas_out, E));
  LRMOE_TRY(need(seg_offsets_out, E + 1));
  LRMOE_TRY(optional(invalid_out));
  return hip_status(launch_plan_quota_device(
      expert_ids, (int32_t)n_ids, E, policy->mode, policy->num, policy->den,
      policy->budget_pairs, counts_out, quotas_out, seg_offsets_out, invalid_out,
      reinterpret_cast<hipStream_t>(stream)));
}

lrmoe_status lrmoe_workspace_size(const lrmoe_problem* pb, size_t* bytes_out) {
  if (bytes_out == nullptr) return LRMOE_ERR_NULL;
  Checked c;
  LRMOE_TRY(check_problem(pb, c));
  *bytes_out = workspace_bytes(pb, c);
  return LRMOE_OK;
}

lrmoe_status lrmoe_score_select_compact(const lrmoe_problem* pb, const int32_t* g_row_index,
                                        const float* alpha, const void* g, const void* phi,
                                        float* scores, uint8_t* keep, int32_t* seg_offsets,
                                        int32_t* perm, void* g_c, void* phi_c, float* alpha_c,
                                        float* dphi_zero, void* workspace, size_t ws_bytes,
                                        void* stream) {
  return select_compact(pb, true, nullptr, g_row_index, alpha, g, phi, scores, keep, seg_offsets,
                        perm, g_c, phi_c, alpha_c, dphi_zero, workspace, ws_bytes, stream,
                        nullptr);
}

lrmoe_status lrmoe_score_select_compact_timed(const lrmoe_problem* pb, const int32_t* g_row_index,
                                              const float* alpha, const void* g, const void* phi,
                                              float* scores, uint8_t* keep, int32_t* seg_offsets,
                                              int32_t* perm, void* g_c, void* phi_c,
                                              float* alpha_c, float* dphi_zero, void* workspace,
                                              size_t ws_bytes, void* stream,
                                              const lrmoe_timing* timing) {
  return select_compact(pb, true, nullptr, g_row_index, alpha, g, phi, scores, keep, seg_offsets,
                        perm, g_c, phi_c, alpha_c, dphi_zero, workspace, ws_bytes, stream, timing);
}

lrmoe_status lrmoe_score_select_compact_noalloc(const lrmoe_problem* pb,
                                                const int32_t* g_row_index, const float* alpha,
                                                const void* g, const void* phi, float* scores,
                                                uint8_t* keep, int32_t* seg_offsets,
                                                int32_t* perm, void* g_c, void* phi_c,
                                                float* alpha_c, float* dphi_zero, void* stream) {
  return select_compact(pb, true, nullptr, g_row_index, alpha, g, phi, scores, keep, seg_offsets,
                        perm, g_c, phi_c, alpha_c, dphi_zero, nullptr, 0, stream, nullptr, true,
                        GatherPlanes(), true);
}

lrmoe_status lrmoe_select_compact(const lrmoe_problem* pb, const float* scores,
                                  const int32_t* g_row_index, const float* alpha, const void* g,
                                  const void* phi, uint8_t* keep, int32_t* seg_offsets,
                                  int32_t* perm, void* g_c, void* phi_c, float* alpha_c,
                                  float* dphi_zero, void* workspace, size_t ws_bytes,
                                  void* stream) {
  return select_compact(pb, false, scores, g_row_index, alpha, g, phi, nullptr, keep, seg_offsets,
                        perm, g_c, phi_c, alpha_c, dphi_zero, workspace, ws_bytes, stream,
                        nullptr);
}

lrmoe_status lrmoe_select_compact_timed(const lrmoe_problem* pb, const float* scores,
                                        const int32_t* g_row_index, const float* alpha,
                                        const void* g, const void* phi, uint8_t* keep,
                                        int32_t* seg_offsets, int32_t* perm, void* g_c,
                                        void* phi_c, float* alpha_c, float* dphi_zero,
                                        void* workspace, size_t ws_bytes, void* stream,
                                        const lrmoe_timing* timing) {
  return select_compact(pb, false, scores, g_row_index, alpha, g, phi, nullptr, keep, seg_offsets,
                        perm, g_c, phi_c, alpha_c, dphi_zero, workspace, ws_bytes, stream,
                        timing);
}

lrmoe_status lrmoe_score_select(const lrmoe_problem* pb, const int32_t* g_row_index,
                                const float* alpha, const void* g, const void* phi, float* scores,
                                uint8_t* keep, int32_t* seg_offsets, int32_t* perm,
                                void* workspace, size_t ws_bytes, void* stream) {
  return select_compact(pb, true, nullptr, g_row_index, alpha, g, phi, scores, keep, seg_offsets,
                        perm, nullptr, nullptr, nullptr, nullptr, workspace, ws_bytes, stream,
                        nullptr, false);
}

lrmoe_status lrmoe_mask_alpha(int64_t P, const uint8_t* keep, const float* alpha,
                              float* alpha_masked, int32_t* perm_identity, void* stream) {
  if (P < 0 || P >= (int64_t(1) << 31)) return LRMOE_ERR_SHAPE;
  LRMOE_TRY(need(keep, P));
  LRMOE_TRY(need(alpha, P));
  LRMOE_TRY(need(alpha_masked, P));
  LRMOE_TRY(optional(perm_identity));
  return hip_status(launch_mask_alpha((int32_t)P, keep, alpha, alpha_masked, perm_identity,
                                      reinterpret_cast<hipStream_t>(stream)));
}

lrmoe_status lrmoe_gather_compact(const lrmoe_problem* pb, const int32_t* perm,
                                  const uint8_t* keep, const int32_t* g_row_index,
                                  const int32_t* phi_row_index, const float* alpha,
                                  const void* g, const void* phi, void* g_c, void* phi_c,
                                  float* alpha_c, float* dphi_zero, void* stream) {
  return gather_compact(pb, perm, keep, g_row_index, phi_row_index, alpha, g, phi, g_c, phi_c,
                        alpha_c, dphi_zero, stream, nullptr, GatherPlanes());
}

lrmoe_status lrmoe_gather_backward(const lrmoe_problem* pb, const int32_t* perm,
                                   const uint8_t* keep, const int32_t* g_row_index,
                                   const int32_t* phi_row_index, const float* alpha,
                                   const void* g, const void* phi, const void* W, void* g_c,
                                   void* phi_c, float* alpha_c, float* dW, float* dphi,
                                   void* workspace, size_t ws_bytes, void* stream) {
  return gather_backward(pb, perm, keep, g_row_index, phi_row_index, alpha, g, phi, W, g_c,
                         phi_c, alpha_c, dW, dphi, workspace, ws_bytes, stream, nullptr);
}

lrmoe_status lrmoe_gather_backward_timed(const lrmoe_problem* pb, const int32_t* perm,
                                         const uint8_t* keep, const int32_t* g_row_index,
                                         const int32_t* phi_row_index, const float* alpha,
                                         const void* g, const void* phi, const void* W,
                                         void* g_c, void* phi_c, float* alpha_c, float* dW,
                                         float* dphi, void* workspace, size_t ws_bytes,
                                         void* stream, const lrmoe_timing* timing) {
  return gather_backward(pb, perm, keep, g_row_index, phi_row_index, alpha, g, phi, W, g_c,
                         phi_c, alpha_c, dW, dphi, workspace, ws_bytes, stream, timing);
}


lrmoe_status lrmoe_grouped_backward(const lrmoe_problem* pb, const int32_t* perm,
                                    const float* alpha_c, const void* g_c, const void* phi_c,
                                    const void* W, float* dW, float* dphi, void* workspace,
                                    size_t ws_bytes, void* stream) {
  return lrmoe_grouped_backward_timed(pb, perm, alpha_c, g_c, phi_c, W, dW, dphi, workspace,
                                      ws_bytes, stream, nullptr);
}

lrmoe_status lrmoe_grouped_backward_timed(const lrmoe_problem* pb, const int32_t* perm,
                                          const float* alpha_c, const void* g_c,
                                          const void* phi_c, const void* W, float* dW,
                                          float* dphi, void* workspace, size_t ws_bytes,
                                          void* stream, const lrmoe_timing* timing) {
  return grouped_backward(pb, perm, alpha_c, g_c, phi_c, W, dW, dphi, false, nullptr, nullptr,
                          nullptr, workspace, ws_bytes, stream, timing);
}

lrmoe_status lrmoe_pruned_backward(const lrmoe_problem* pb, const int32_t* g_row_index,
                                   const float* alpha, const void* g, const void* phi,
                                   const void* W, float* scores, uint8_t* keep,
                                   int32_t* seg_offsets, int32_t* perm, void* g_c, void* phi_c,
                                   float* alpha_c, float* dW, float* dphi, void* workspace,
                                   size_t ws_bytes, void* stream) {
  return pruned_backward(pb, g_row_index, alpha, g, phi, W, scores, keep, seg_offsets, perm, g_c,
                         phi_c, alpha_c, dW, dphi, workspace, ws_bytes, stream, nullptr);
}

lrmoe_status lrmoe_pruned_backward_timed(const lrmoe_problem* pb, const int32_t* g_row_index,
                                         const float* alpha, const void* g, const void* phi,
                                         const void* W, float* scores, uint8_t* keep,
                                         int32_t* seg_offsets, int32_t* perm, void* g_c,
                                         void* phi_c, float* alpha_c, float* dW, float* dphi,
                                         void* workspace, size_t ws_bytes, void* stream,
                                         const lrmoe_timing* timing) {
  return pruned_backward(pb, g_row_index, alpha, g, phi, W, scores, keep, seg_offsets, perm, g_c,
                         phi_c, alpha_c, dW, dphi, workspace, ws_bytes, stream, timing);
}

lrmoe_status lrmoe_grouped_backward_glu(const lrmoe_problem* pb, const int32_t* perm,
                                        const float* alpha_c, const void* g_c, const void* phi_c,
                                        const void* W, float* dW, const void* act_a,
                                        const void* act_b, void* dgu_c, void* workspace,
                                        size_t ws_bytes, void* stream) {
  return lrmoe_grouped_backward_glu_timed(pb, perm, alpha_c, g_c, phi_c, W, dW, act_a, act_b,
                                          dgu_c, workspace, ws_bytes, stream, nullptr);
}

lrmoe_status lrmoe_grouped_backward_glu_timed(const lrmoe_problem* pb, const int32_t* perm,
                                              const float* alpha_c, const void* g_c,
                                              const void* phi_c, const void* W, float* dW,
                                              const void* act_a, const void* act_b, void* dgu_c,
                                              void* workspace, size_t ws_bytes, void* stream,
                                              const lrmoe_timing* timing) {
  if (pb == nullptr) return LRMOE_ERR_NULL;
  if (pb->dtype != LRMOE_BF16) return LRMOE_ERR_DTYPE;
  return grouped_backward(pb, perm, alpha_c, g_c, phi_c, W, dW, nullptr, true,
                          reinterpret_cast<const uint16_t*>(act_a),
                          reinterpret_cast<const uint16_t*>(act_b), dgu_c, workspace, ws_bytes,
                          stream, timing);
}

lrmoe_status lrmoe_grouped_backward_gate_up(const lrmoe_problem* pb, const int32_t* perm,
                                            const float* alpha_c, const float* dgu_c,
                                            const void* x_c, const void* W, float* dW, float* dx,
                                            void* workspace, size_t ws_bytes, void* stream) {
  return lrmoe_grouped_backward_gate_up_timed(pb, perm, alpha_c, dgu_c, x_c, W, dW, dx, workspace,
                                              ws_bytes, stream, nullptr);
}

lrmoe_status lrmoe_grouped_backward_gate_up_timed(const lrmoe_problem* pb, const int32_t* perm,
                                                  const float* alpha_c, const float* dgu_c,
                                                  const void* x_c, const void* W, float* dW,
                                                  float* dx, void* workspace, size_t ws_bytes,
                                                  void* stream, const lrmoe_timing* timing) {
  return grouped_backward(pb, perm, alpha_c, dgu_c, x_c, W, dW, dx, false, nullptr, nullptr,
                          nullptr, workspace, ws_bytes, stream, timing, false, TimingSlots(),
                          true);
}

}  // extern "C"
