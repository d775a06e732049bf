// LRM scoring, per-expert top-quota selection and the compaction scan.
//
// Score: R_u = alpha_u^2 * ||g_t||^2 * ||phi_u||^2, the squared Frobenius norm
// of the rank-one per-pair weight gradient (alpha_u g_t) phi_u^T
// ("LRMoE: Trimming Backward Work in Memory-Bound MoE Training", section
// "LRM: a decomposable contribution score").  It is a pure row-norm pass:
// HBM-bound, one wave64 per pair, 16-byte loads, shuffle-tree reductions.
//
// Select + scan: within each expert's quota the highest-scoring pairs are kept
// (Portuguese write-up "LRMoE poda a passagem reversa do MoE ...", selection
// bullet).  One 1024-thread workgroup per expert runs an MSB-first radix
// select (4 x 8-bit digits) on an order-preserving integer image of the
// float32 scores to find the q_e-th largest key tau_e and how many keys equal
// to tau_e are still needed; ties go to the lower pair index.  The same
// workgroup then scans the expert's pairs in index order, writes the keep
// flags and the compacted permutation (ascending pair index inside the
// segment).
#include "lrmoe_internal.h"

namespace lrmoe {
namespace {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ float sumsq8(uint4 x) {
  float a = 0.f, v;
  v = bf16_lo(x.x); a = fmaf(v, v, a); v = bf16_hi(x.x); a = fmaf(v, v, a);
  v = bf16_lo(x.y); a = fmaf(v, v, a); v = bf16_hi(x.y); a = fmaf(v, v, a);
  v = bf16_lo(x.z); a = fmaf(v, v, a); v = bf16_hi(x.z); a = fmaf(v, v, a);
  v = bf16_lo(x.w); a = fmaf(v, v, a); v = bf16_hi(x.w); a = fmaf(v, v, a);
  return a;
}
__device__ __forceinline__ float sumsq4(float4 x) {
  return fmaf(x.w, x.w, fmaf(x.z, x.z, fmaf(x.y, x.y, x.x * x.x)));
}

// Sum of squares of one row held in 16-byte chunks, lane-strided, four
// independent loads in flight per lane.
template <typename V>
__device__ __forceinline__ float row_sumsq(const V* __restrict__ row, int nchunk, int lane) {
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  int c = lane;
  for (; c + 192 < nchunk; c += 256) {
    const V x0 = row[c], x1 = row[c + 64], x2 = row[c + 128], x3 = row[c + 192];
    if constexpr (sizeof(V) == 16 && __is_same(V, uint4)) {
      a0 += sumsq8(x0); a1 += sumsq8(x1); a2 += sumsq8(x2); a3 += sumsq8(x3);
    } else {
      a0 += sumsq4(x0); a1 += sumsq4(x1); a2 += sumsq4(x2); a3 += sumsq4(x3);
    }
  }
  for (; c < nchunk; c += 64) {
    const V x = row[c];
    if constexpr (__is_same(V, uint4)) a0 += sumsq8(x); else a0 += sumsq4(x);
  }
  return (a0 + a1) + (a2 + a3);
}

template <bool BF16>
__global__ __launch_bounds__(256) void lrm_score_kernel(
    const void* __restrict__ g, const void* __restrict__ phi, const float* __restrict__ alpha,
    const int32_t* __restrict__ row_index, int32_t P, int32_t d_out, int32_t d_in,
    float* __restrict__ scores) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * blockDim.x) >> 6;
  const int per = BF16 ? 8 : 4;  // elements per 16-byte chunk
  const int gc = d_out / per, pc = d_in / per;
  for (int u = wave; u < P; u += nwaves) {
    const int64_t r = row_index ? (int64_t)row_index[u] : (int64_t)u;
    float gs, ps;
    if (BF16) {
      gs = row_sumsq(reinterpret_cast<const uint4*>(g) + r * gc, gc, lane);
      ps = row_sumsq(reinterpret_cast<const uint4*>(phi) + (int64_t)u * pc, pc, lane);
    } else {
      gs = row_sumsq(reinterpret_cast<const float4*>(g) + r * gc, gc, lane);
      ps = row_sumsq(reinterpret_cast<const float4*>(phi) + (int64_t)u * pc, pc, lane);
    }
    gs = wave_sum(gs);
    ps = wave_sum(ps);
    if (lane == 0) {
      const float a = alpha[u];
      scores[u] = ((a * a) * gs) * ps;
    }
  }
}

// Order-preserving map of float32 to uint32 (larger float -> larger key);
// -0.0 is folded onto +0.0 so that equal values have equal keys.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t b = __float_as_uint(s);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelLdsKeys = 24576;   // 96 KiB: experts up to this size select from LDS

__global__ __launch_bounds__(kSelThreads) void select_scan_kernel(
    ExpertTable tab, const float* __restrict__ scores, uint8_t* __restrict__ keep,
    int32_t* __restrict__ perm, int32_t* __restrict__ seg_offsets_out) {
  __shared__ uint32_t hist[kSelWaves][256];
  __shared__ uint32_t sh_digit, sh_k;
  __shared__ uint32_t wcnt[2][kSelWaves];
  __shared__ uint32_t keys_lds[kSelLdsKeys];   // the expert's keys, when they fit

  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int base = tab.pair_off[e];
  const int n = tab.pair_off[e + 1] - base;
  const int seg = tab.seg_off[e];
  const uint32_t q = (uint32_t)(tab.seg_off[e + 1] - seg);

  if (tid == 0) {
    seg_offsets_out[e] = seg;
    if (e == tab.E - 1) seg_offsets_out[tab.E] = tab.seg_off[tab.E];
  }
  if (n == 0) return;
  const bool cached = n <= kSelLdsKeys;
  if (cached) {
    for (int i = tid; i < n; i += kSelThreads) keys_lds[i] = score_key(scores[base + i]);
    __syncthreads();
  }
  auto key_at = [&](int i) -> uint32_t {
    return cached ? keys_lds[i] : score_key(scores[base + i]);
  };

  // ---- radix select: tau = q-th largest key, need = #(key == tau) to keep
  uint32_t tau = 0xFFFFFFFFu, need = 0;   // q == 0: nothing is above or equal
  if (q > 0) {
    uint32_t prefix = 0, mask = 0, k = q;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < kSelWaves * 256; i += kSelThreads) (&hist[0][0])[i] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += kSelThreads) {
        const uint32_t key = key_at(i);
        if ((key & mask) == prefix) atomicAdd(&hist[wave][(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 256) {
        uint32_t s = 0;
#pragma unroll
        for (int w = 0; w < kSelWaves; ++w) s += hist[w][tid];
        hist[0][tid] = s;
      }
      __syncthreads();
      if (wave == 0) {
        // lane l owns bins 4l .. 4l+3; count from the top bin down.
        const uint32_t c0 = hist[0][4 * lane], c1 = hist[0][4 * lane + 1];
        const uint32_t c2 = hist[0][4 * lane + 2], c3 = hist[0][4 * lane + 3];
        const uint32_t local = c0 + c1 + c2 + c3;
        uint32_t suffix = local;  // inclusive sum over lanes >= lane
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t o = __shfl_down(suffix, off, 64);
          if (lane + off < 64) suffix += o;
        }
        const uint32_t above = suffix - local;
        if (above < k && k <= suffix) {
          uint32_t cum = above, d;
          if (cum + c3 >= k) d = 3;
          else if ((cum += c3) + c2 >= k) d = 2;
          else if ((cum += c2) + c1 >= k) d = 1;
          else { cum += c1; d = 0; }
          sh_digit = 4u * lane + d;
          sh_k = k - cum;
        }
      }
      __syncthreads();
      prefix |= sh_digit << shift;
      mask |= 0xFFu << shift;
      k = sh_k;
      __syncthreads();
    }
    tau = prefix;
    need = k;
  }

  // ---- stable scan: keep = key > tau, or key == tau among the first `need`
  uint32_t run_keep = 0, run_eq = 0;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int c0 = 0; c0 < n; c0 += kSelThreads) {
    const int i = c0 + tid;
    const bool valid = i < n;
    const uint32_t key = valid ? key_at(i) : 0u;
    const bool gt = valid && key > tau;
    const bool eq = valid && key == tau;
    const uint64_t beq = __ballot(eq);
    if (lane == 0) wcnt[0][wave] = (uint32_t)__popcll(beq);
    __syncthreads();
    uint32_t eq_before = 0, eq_total = 0;
    for (int w = 0; w < kSelWaves; ++w) {
      const uint32_t v = wcnt[0][w];
      eq_before += (w < wave) ? v : 0u;
      eq_total += v;
    }
    const uint32_t eq_rank = run_eq + eq_before + (uint32_t)__popcll(beq & lt_mask);
    const bool kp = gt || (eq && eq_rank < need);
    const uint64_t bk = __ballot(kp);
    if (lane == 0) wcnt[1][wave] = (uint32_t)__popcll(bk);
    __syncthreads();
    uint32_t k_before = 0, k_total = 0;
    for (int w = 0; w < kSelWaves; ++w) {
      const uint32_t v = wcnt[1][w];
      k_before += (w < wave) ? v : 0u;
      k_total += v;
    }
    if (valid) {
      keep[base + i] = kp ? 1 : 0;
      const uint32_t pos = run_keep + k_before + (uint32_t)__popcll(bk & lt_mask);
      if (kp && pos < q) perm[seg + pos] = base + i;   // pos < q holds by construction
    }
    run_eq += eq_total;
    run_keep += k_total;
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_score(int dtype, const void* g, const void* phi, const float* alpha,
                        const int32_t* row_index, int32_t P, int32_t d_out, int32_t d_in,
                        float* scores, hipStream_t s) {
  if (P <= 0) return hipSuccess;
  const int waves_per_block = 4;
  int blocks = (P + waves_per_block - 1) / waves_per_block;
  if (blocks > 256 * 8) blocks = 256 * 8;   // 32 waves per CU, each looping over pairs
  if (dtype == LRMOE_BF16)
    hipLaunchKernelGGL(lrm_score_kernel<true>, dim3(blocks), dim3(256), 0, s, g, phi, alpha,
                       row_index, P, d_out, d_in, scores);
  else
    hipLaunchKernelGGL(lrm_score_kernel<false>, dim3(blocks), dim3(256), 0, s, g, phi, alpha,
                       row_index, P, d_out, d_in, scores);
  return hipGetLastError();
}

hipError_t launch_select_scan(const ExpertTable& tab, const float* scores, uint8_t* keep,
                              int32_t* perm, int32_t* seg_offsets_out, hipStream_t s) {
  hipLaunchKernelGGL(select_scan_kernel, dim3(tab.E), dim3(kSelThreads), 0, s, tab, scores,
                     keep, perm, seg_offsets_out);
  return hipGetLastError();
}

}  // namespace lrmoe
