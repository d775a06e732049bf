// Quota planning on the device, from the forward's routing.
//
// The pages fix each expert's backward quota before the backward, from how
// many tokens reached the expert ("LRMoE poda a passagem reversa do MoE e
// acelera o treinamento em 21-45%", bullet "Cotas antes do calculo"; "LRMoE:
// Trimming Backward Work in Memory-Bound MoE Training", section "Backward
// demand is not a constant").  The host planner (lrmoe_plan_quota) takes the
// counts; this one starts from the routing itself -- the expert index of
// every routed token-expert pair, as the forward's top-k produces it -- so
// that the counts never have to visit the host:
//   1. clear the count array;
//   2. histogram: each workgroup counts its slice of the expert indices in
//      LDS, then adds its E bins to the global counts with E atomics (an
//      index outside 0..E-1 is counted as invalid, not routed);
//   3. one workgroup turns counts into quotas with the same integer rules as
//      the host planner (ratio: floor(n_e num / den); budget Q: floor(n_e Q /
//      P) with P the routed pairs, or n_e when Q >= P) and writes the
//      exclusive prefix sum of the quotas.
#include "lrmoe_internal.h"

namespace lrmoe {
namespace {

constexpr int kPlanThreads = 1024;
constexpr int kIdsPerBlock = kPlanThreads * 16;

__global__ void clear_counts_kernel(unsigned long long* counts, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) counts[i] = 0ull;
}

__global__ __launch_bounds__(kPlanThreads) void routing_hist_kernel(
    const int32_t* __restrict__ ids, int32_t n_ids, int32_t E,
    unsigned long long* __restrict__ counts, unsigned long long* __restrict__ invalid) {
  __shared__ uint32_t h[kMaxE + 1];   // bin E: indices outside 0..E-1
  const int tid = threadIdx.x;
  for (int i = tid; i <= E; i += kPlanThreads) h[i] = 0;
  __syncthreads();
  const int lo = blockIdx.x * kIdsPerBlock;
  const int hi = min(lo + kIdsPerBlock, n_ids);
  // the id array is 16-byte aligned and lo is a multiple of 4: int4 loads,
  // with a guarded tail
  for (int a = lo + 4 * tid; a < hi; a += 4 * kPlanThreads) {
    int v[4];
    if (a + 4 <= hi) {
      const int4 x = *reinterpret_cast<const int4*>(ids + a);
      v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = a + j < hi ? ids[a + j] : -2;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (a + j >= hi) break;
      const int e = v[j];
      atomicAdd(&h[(e >= 0 && e < E) ? e : E], 1u);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kPlanThreads)
    if (h[e]) atomicAdd(&counts[e], (unsigned long long)h[e]);
  if (tid == 0 && h[E] && invalid != nullptr) atomicAdd(invalid, (unsigned long long)h[E]);
}

__global__ __launch_bounds__(256) void quota_kernel(
    int32_t E, int32_t mode, int64_t num, int64_t den, int64_t Q,
    const unsigned long long* __restrict__ counts, int64_t* __restrict__ quotas,
    int64_t* __restrict__ seg_offsets) {
  __shared__ int64_t qs[kMaxE];
  __shared__ int64_t total;
  const int tid = threadIdx.x;
  if (tid == 0) {
    int64_t P = 0;
    for (int e = 0; e < E; ++e) P += (int64_t)counts[e];
    total = P;
  }
  __syncthreads();
  const int64_t P = total;
  for (int e = tid; e < E; e += blockDim.x) {
    const int64_t n = (int64_t)counts[e];
    int64_t q;
    if (mode == LRMOE_QUOTA_RATIO) {
      q = (n * num) / den;   // n < 2^31, num <= den < 2^31: exact in 64 bits
    } else if (P == 0 || Q >= P) {
      q = n;
    } else {
      q = (int64_t)((unsigned __int128)n * (unsigned __int128)Q / (unsigned __int128)P);
    }
    qs[e] = q;
    quotas[e] = q;
  }
  __syncthreads();
  if (tid == 0) {   // E <= 256: a serial prefix sum is the simplest exact one
    int64_t s = 0;
    for (int e = 0; e < E; ++e) {
      seg_offsets[e] = s;
      s += qs[e];
    }
    seg_offsets[E] = s;
  }
}

}  // namespace

hipError_t launch_plan_quota_device(const int32_t* ids, int32_t n_ids, int32_t E, int32_t mode,
                                    int64_t num, int64_t den, int64_t Q, int64_t* counts,
                                    int64_t* quotas, int64_t* seg_offsets, int64_t* invalid,
                                    hipStream_t s) {
  unsigned long long* c = reinterpret_cast<unsigned long long*>(counts);
  unsigned long long* bad = reinterpret_cast<unsigned long long*>(invalid);
  hipLaunchKernelGGL(clear_counts_kernel, dim3((E + 255) / 256), dim3(256), 0, s, c, E);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (bad != nullptr) {
    hipLaunchKernelGGL(clear_counts_kernel, dim3(1), dim3(64), 0, s, bad, 1);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (n_ids > 0) {
    const int blocks = (n_ids + kIdsPerBlock - 1) / kIdsPerBlock;
    hipLaunchKernelGGL(routing_hist_kernel, dim3(blocks), dim3(kPlanThreads), 0, s, ids, n_ids,
                       E, c, bad);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  hipLaunchKernelGGL(quota_kernel, dim3(1), dim3(256), 0, s, E, mode, num, den, Q, c, quotas,
                     seg_offsets);
  return hipGetLastError();
}

}  // namespace lrmoe
