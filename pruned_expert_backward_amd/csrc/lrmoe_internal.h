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
struct ExpertTable {
  int32_t E;
  int32_t M;                      // total kept pairs
  int32_t pair_off[kMaxE + 1];    // first pair of expert e (expert-sorted)
  int32_t seg_off[kMaxE + 1];     // first compacted row of expert e
};

// Tile schedule of the grouped GEMMs (also host-built, by value).
struct GemmTable {
  int32_t E;
  int32_t tiles_n;                // tiles along the output columns (d_in)
  int32_t tiles_m_fixed;          // dW: tiles along d_out (same for all experts)
  int32_t dw_tiles;               // weight-gradient blocks (first in the grid)
  int32_t dp_tiles;               // input-gradient blocks (after them)
  int32_t seg_off[kMaxE + 1];     // compacted segment offsets
  int32_t tile_off[kMaxE + 1];    // dphi: first block of expert e
  int16_t order[kMaxE];           // dW: experts by descending quota
};

// Launchers (return hipSuccess or the launch error).
hipError_t launch_score(int dtype, const void* g, const void* phi, const float* alpha,
                        const int32_t* row_index, int32_t P, int32_t d_out, int32_t d_in,
                        float* scores, hipStream_t s);

hipError_t launch_select_scan(const ExpertTable& tab, const float* scores, uint8_t* keep,
                              int32_t* perm, int32_t* seg_offsets_out, hipStream_t s);

hipError_t launch_gather(int dtype, const int32_t* perm, const uint8_t* keep,
                         const int32_t* g_row_index, const int32_t* phi_row_index,
                         const float* alpha, const void* g, const void* phi, void* g_c,
                         void* phi_c, float* alpha_c, float* dphi_zero, int32_t M,
                         int32_t P, int32_t d_out, int32_t d_in, hipStream_t s);

hipError_t launch_grouped_backward(int dtype, int dw_mode, const GemmTable& tab,
                                   const int32_t* perm, const float* alpha_c, const void* g_c,
                                   const void* phi_c, const void* W, float* dW, float* dphi,
                                   int32_t d_out, int32_t d_in, int32_t P, hipStream_t s);

}  // namespace lrmoe
