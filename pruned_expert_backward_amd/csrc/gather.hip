// Physical compaction: copy the kept g rows, phi rows and routing weights into
// contiguous, expert-segmented, unpadded buffers, and zero the input-gradient
// rows of dropped pairs in the original layout.  The pages stress that the
// gain comes from this repacking, not from masking rows of full-size tensors
// ("LRMoE: Trimming Backward Work in Memory-Bound MoE Training", section "The
// part that is easy to get wrong"; Portuguese write-up, compaction bullet).
//
// HBM-bound copy: one wave64 per row job, 16-byte vector loads and stores.
// Jobs [0, M) gather compacted row j; jobs [M, M + P) zero dphi row u when
// pair u was dropped (only when a zero target is given).
#include "lrmoe_internal.h"

namespace lrmoe {
namespace {

__device__ __forceinline__ void copy_row(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                         int nchunk, int lane) {
  int c = lane;
  for (; c + 192 < nchunk; c += 256) {
    const uint4 a = src[c], b = src[c + 64], d = src[c + 128], f = src[c + 192];
    dst[c] = a; dst[c + 64] = b; dst[c + 128] = d; dst[c + 192] = f;
  }
  for (; c < nchunk; c += 64) dst[c] = src[c];
}

__global__ __launch_bounds__(256) void gather_kernel(
    const int32_t* __restrict__ perm, const uint8_t* __restrict__ keep,
    const int32_t* __restrict__ g_row_index, const int32_t* __restrict__ phi_row_index,
    const float* __restrict__ alpha, const uint4* __restrict__ g, const uint4* __restrict__ phi,
    uint4* __restrict__ g_c, uint4* __restrict__ phi_c, float* __restrict__ alpha_c,
    float4* __restrict__ dphi_zero, int32_t M, int32_t P, int32_t gch, int32_t pch,
    int32_t zch) {
  const int lane = threadIdx.x & 63;
  const int64_t job = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (job < M) {
    const int32_t j = (int32_t)job;
    const int32_t u = perm[j];
    if ((uint32_t)u >= (uint32_t)P) return;   // perm holds pair indices < P
    const int64_t gr = g_row_index ? (int64_t)g_row_index[u] : (int64_t)u;
    const int64_t pr = phi_row_index ? (int64_t)phi_row_index[u] : (int64_t)u;
    if (g_c != nullptr) copy_row(g + gr * gch, g_c + (int64_t)j * gch, gch, lane);
    copy_row(phi + pr * pch, phi_c + (int64_t)j * pch, pch, lane);
    if (lane == 0) alpha_c[j] = alpha[u];
  } else if (dphi_zero != nullptr && job < (int64_t)M + P) {
    const int64_t u = job - M;
    if (!keep[u]) {
      float4* row = dphi_zero + u * zch;
      const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int c = lane; c < zch; c += 64) row[c] = z;
    }
  }
}

// Zero-masked dense alternative: alpha of dropped pairs set to 0 in the
// original layout (and, optionally, the identity permutation), so that the
// same grouped GEMMs run over every routed pair with the dropped ones
// contributing exactly nothing.  The pages weigh this masking against
// compaction and find that it saves neither time nor memory (Portuguese
// write-up, the paragraph after the bullets); this path measures that.
__global__ __launch_bounds__(256) void mask_alpha_kernel(const uint8_t* __restrict__ keep,
                                                         const float* __restrict__ alpha,
                                                         float* __restrict__ alpha_masked,
                                                         int32_t* __restrict__ perm_identity,
                                                         int32_t P) {
  for (int u = blockIdx.x * blockDim.x + threadIdx.x; u < P; u += gridDim.x * blockDim.x) {
    alpha_masked[u] = keep[u] ? alpha[u] : 0.f;
    if (perm_identity != nullptr) perm_identity[u] = u;
  }
}

}  // namespace

hipError_t launch_mask_alpha(int32_t P, const uint8_t* keep, const float* alpha,
                             float* alpha_masked, int32_t* perm_identity, hipStream_t s) {
  if (P <= 0) return hipSuccess;
  int blocks = (P + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(mask_alpha_kernel, dim3(blocks), dim3(256), 0, s, keep, alpha, alpha_masked,
                     perm_identity, P);
  return hipGetLastError();
}

hipError_t launch_gather(int dtype, const int32_t* perm, const uint8_t* keep,
                         const int32_t* g_row_index, const int32_t* phi_row_index,
                         const float* alpha, const void* g, const void* phi, void* g_c,
                         void* phi_c, float* alpha_c, float* dphi_zero, int32_t M,
                         int32_t P, int32_t d_out, int32_t d_in, hipStream_t s) {
  const int per = (dtype == LRMOE_BF16) ? 8 : 4;
  const int64_t jobs = (int64_t)M + (dphi_zero ? (int64_t)P : 0);
  if (jobs == 0) return hipSuccess;
  const int64_t blocks = (jobs + 3) / 4;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(256), 0, s, perm, keep,
                     g_row_index, phi_row_index, alpha, (const uint4*)g, (const uint4*)phi,
                     (uint4*)g_c, (uint4*)phi_c, alpha_c, (float4*)dphi_zero, M, P,
                     d_out / per, d_in / per, d_in / 4);
  return hipGetLastError();
}

}  // namespace lrmoe
