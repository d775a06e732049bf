// C-ABI entry points of liblrmoe: argument validation (all of it on the host,
// before any launch), host-side quota planning, the per-expert tables handed
// to kernels by value, and the stream-ordered launch sequence.
#include <string.h>

#include <algorithm>
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
  if ((pb->dw_mode != LRMOE_DW_EXACT && pb->dw_mode != LRMOE_DW_BF16) || pb->reserved != 0)
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
  c.tab.M = (int32_t)M;
  c.M = M;
  return LRMOE_OK;
}

size_t workspace_bytes(const lrmoe_problem*, const Checked&) { return 0; }

lrmoe_status hip_status(hipError_t e) { return e == hipSuccess ? LRMOE_OK : LRMOE_ERR_HIP; }

int64_t elem_bytes(const lrmoe_problem* pb) { return pb->dtype == LRMOE_BF16 ? 2 : 4; }

// Shared body of the two select entry points.
lrmoe_status select_compact(const lrmoe_problem* pb, bool compute_scores, const float* scores_in,
                            const int32_t* g_row_index, const float* alpha, const void* g,
                            const void* phi, float* scores_out, uint8_t* keep,
                            int32_t* seg_offsets, int32_t* perm, void* g_c, void* phi_c,
                            float* alpha_c, float* dphi_zero, void* workspace, size_t ws_bytes,
                            void* stream) {
  Checked c;
  LRMOE_TRY(check_problem(pb, c));
  const int64_t P = pb->P, M = c.M;
  if (g_row_index == nullptr && pb->T != P) return LRMOE_ERR_SHAPE;
  LRMOE_TRY(need(alpha, P));
  LRMOE_TRY(need(g, P > 0 ? pb->T : 0));
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
  LRMOE_TRY(need(g_c, M));
  LRMOE_TRY(need(phi_c, M));
  LRMOE_TRY(need(alpha_c, M));
  LRMOE_TRY(optional(dphi_zero));
  if (ws_bytes < workspace_bytes(pb, c)) return LRMOE_ERR_WORKSPACE;
  (void)workspace;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const float* scores = scores_in;
  if (compute_scores) {
    LRMOE_TRY(hip_status(launch_score(pb->dtype, g, phi, alpha, g_row_index, (int32_t)P,
                                      pb->d_out, pb->d_in, scores_out, s)));
    scores = scores_out;
  }
  LRMOE_TRY(hip_status(launch_select_scan(c.tab, scores, keep, perm, seg_offsets, s)));
  LRMOE_TRY(hip_status(launch_gather(pb->dtype, perm, keep, g_row_index, nullptr, alpha, g, phi,
                                     g_c, phi_c, alpha_c, dphi_zero, (int32_t)M, (int32_t)P,
                                     pb->d_out, pb->d_in, s)));
  return LRMOE_OK;
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
                        perm, g_c, phi_c, alpha_c, dphi_zero, workspace, ws_bytes, stream);
}

lrmoe_status lrmoe_select_compact(const lrmoe_problem* pb, const float* scores,
                                  const int32_t* g_row_index, const float* alpha, const void* g,
                                  const void* phi, uint8_t* keep, int32_t* seg_offsets,
                                  int32_t* perm, void* g_c, void* phi_c, float* alpha_c,
                                  float* dphi_zero, void* workspace, size_t ws_bytes,
                                  void* stream) {
  return select_compact(pb, false, scores, g_row_index, alpha, g, phi, nullptr, keep, seg_offsets,
                        perm, g_c, phi_c, alpha_c, dphi_zero, workspace, ws_bytes, stream);
}

lrmoe_status lrmoe_gather_compact(const lrmoe_problem* pb, const int32_t* perm,
                                  const uint8_t* keep, const int32_t* g_row_index,
                                  const int32_t* phi_row_index, const float* alpha,
                                  const void* g, const void* phi, void* g_c, void* phi_c,
                                  float* alpha_c, float* dphi_zero, void* stream) {
  Checked c;
  LRMOE_TRY(check_problem(pb, c));
  const int64_t P = pb->P, M = c.M;
  if (g_row_index == nullptr && pb->T != P) return LRMOE_ERR_SHAPE;
  LRMOE_TRY(need(perm, M));
  LRMOE_TRY(need(alpha, P));
  LRMOE_TRY(need(g, M > 0 ? pb->T : 0));
  LRMOE_TRY(need(phi, M));
  LRMOE_TRY(optional(g_row_index));
  LRMOE_TRY(optional(phi_row_index));
  LRMOE_TRY(need(g_c, M));
  LRMOE_TRY(need(phi_c, M));
  LRMOE_TRY(need(alpha_c, M));
  LRMOE_TRY(optional(dphi_zero));
  if (dphi_zero != nullptr) LRMOE_TRY(need(keep, P));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return hip_status(launch_gather(pb->dtype, perm, keep, g_row_index, phi_row_index, alpha, g,
                                  phi, g_c, phi_c, alpha_c, dphi_zero, (int32_t)M, (int32_t)P,
                                  pb->d_out, pb->d_in, s));
}

lrmoe_status lrmoe_grouped_backward(const lrmoe_problem* pb, const int32_t* perm,
                                    const float* alpha_c, const void* g_c, const void* phi_c,
                                    const void* W, float* dW, float* dphi, void* workspace,
                                    size_t ws_bytes, void* stream) {
  Checked c;
  LRMOE_TRY(check_problem(pb, c));
  const int64_t M = c.M;
  LRMOE_TRY(need(alpha_c, M));
  LRMOE_TRY(need(g_c, M));
  LRMOE_TRY(need(phi_c, M));
  LRMOE_TRY(need(W, 1));
  LRMOE_TRY(need(dW, 1));
  LRMOE_TRY(optional(dphi));
  if (dphi != nullptr) LRMOE_TRY(need(perm, M));
  if (ws_bytes < workspace_bytes(pb, c)) return LRMOE_ERR_WORKSPACE;
  (void)workspace;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  const int E = pb->E;
  GemmTable t;
  memset(&t, 0, sizeof(t));
  t.E = E;
  t.tiles_n = (pb->d_in + 127) / 128;
  t.tiles_m_fixed = (pb->d_out + 127) / 128;
  for (int e = 0; e <= E; ++e) t.seg_off[e] = c.tab.seg_off[e];

  // Weight gradient: every expert's tiles (zeros for q_e = 0), heaviest
  // experts first so that the longest K loops start earliest.
  std::vector<int> order(E);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int a, int b) { return pb->quotas[a] > pb->quotas[b]; });
  for (int i = 0; i < E; ++i) t.order[i] = (int16_t)order[i];
  t.dw_tiles = E * t.tiles_m_fixed * t.tiles_n;
  int32_t tiles = 0;
  for (int e = 0; e < E; ++e) {
    t.tile_off[e] = tiles;
    tiles += (int32_t)((pb->quotas[e] + 127) / 128) * t.tiles_n;
  }
  t.tile_off[E] = tiles;
  t.dp_tiles = (dphi != nullptr) ? tiles : 0;
  LRMOE_TRY(hip_status(launch_grouped_backward(pb->dtype, pb->dw_mode, t, perm, alpha_c, g_c,
                                               phi_c, W, dW, dphi, pb->d_out, pb->d_in,
                                               (int32_t)pb->P, s)));
  return LRMOE_OK;
}

}  // extern "C"
