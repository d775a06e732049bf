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
#include "row_norm.h"

namespace lrmoe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Zero row (a source row index out of range reads as zeros), and its planes.
__device__ __forceinline__ void zero_row(uint4* __restrict__ dst, uint4* __restrict__ hi,
                                         uint4* __restrict__ lo, int nchunk, int lane) {
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
  for (int c = lane; c < nchunk; c += 64) {
    if (dst != nullptr) dst[c] = z;
    if (hi != nullptr) hi[c] = z;
    if (lo != nullptr) lo[c] = z;
  }
}

__device__ __forceinline__ void copy_row(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                         int nchunk, int lane) {
  int c = lane;
  for (; c + 192 < nchunk; c += 256) {
    const uint4 a = src[c], b = src[c + 64], d = src[c + 128], f = src[c + 192];
    dst[c] = a; dst[c + 64] = b; dst[c + 128] = d; dst[c + 192] = f;
  }
  for (; c < nchunk; c += 64) dst[c] = src[c];
}

// copy_row that also writes the bf16 hi (+ lo) planes of a * row (bf16 rows).
__device__ __forceinline__ void copy_row_split(const uint4* __restrict__ src,
                                               uint4* __restrict__ dst, uint4* __restrict__ hi,
                                               uint4* __restrict__ lo, float a, int nchunk,
                                               int lane) {
  auto split = [&](int c, const uint4& x) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    bf16x8 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const HiLo e0 = alpha_split(a, __uint_as_float(w[i] << 16));
      const HiLo e1 = alpha_split(a, __uint_as_float(w[i] & 0xFFFF0000u));
      h[2 * i] = e0.h; l[2 * i] = e0.l;
      h[2 * i + 1] = e1.h; l[2 * i + 1] = e1.l;
    }
    hi[c] = __builtin_bit_cast(uint4, h);
    if (lo != nullptr) lo[c] = __builtin_bit_cast(uint4, l);
  };
  int c = lane;
  for (; c + 64 < nchunk; c += 128) {
    const uint4 x0 = src[c], x1 = src[c + 64];
    dst[c] = x0; dst[c + 64] = x1;
    split(c, x0); split(c + 64, x1);
  }
  for (; c < nchunk; c += 64) {
    const uint4 x = src[c];
    dst[c] = x;
    split(c, x);
  }
}

// ---- float16 weight-gradient planes
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// 8 bf16 of a 16-byte chunk -> float16 of 2^s * a * x: the product rounded
// once to float32 (exact when a == 1), the power of two exact, then one
// rounding to float16 (nearest even).
__device__ __forceinline__ uint4 f16_chunk(const uint4& x, float a, int s) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  f16x8 h;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[2 * i] = (_Float16)__builtin_amdgcn_ldexpf(a * __uint_as_float(w[i] << 16), s);
    h[2 * i + 1] = (_Float16)__builtin_amdgcn_ldexpf(a * __uint_as_float(w[i] & 0xFFFF0000u), s);
  }
  return __builtin_bit_cast(uint4, h);
}

// 16-byte store; NT marks it non-temporal (the line is not kept in the
// caches for reuse).
template <bool NT>
__device__ __forceinline__ void store16(uint4* __restrict__ p, const uint4& v) {
  if constexpr (NT) {
    typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(p));
  } else {
    *p = v;
  }
}

// Copy of one bf16 row (dst may be null) and its float16 plane row.  NT:
// non-temporal stores.  Where the grouped GEMM launch also clears the
// dropped pairs' dphi rows (the 655 360-pair workload), the gather's 1.4 GB
// of cached stores pushed the lines the GEMM re-reads out of the caches:
// non-temporal ones cost the gather about 15 us and save the GEMM 30-55 us;
// on a 32 768-pair workload without that fill they cost 23 us and saved 4-15.
template <bool NT = false>
__device__ __forceinline__ void copy_row_f16(const uint4* __restrict__ src,
                                             uint4* __restrict__ dst, uint4* __restrict__ pl,
                                             float a, int s, int nchunk, int lane) {
  int c = lane;
  for (; c + 64 < nchunk; c += 128) {
    const uint4 x0 = src[c], x1 = src[c + 64];
    if (dst != nullptr) {
      store16<NT>(dst + c, x0);
      store16<NT>(dst + c + 64, x1);
    }
    store16<NT>(pl + c, f16_chunk(x0, a, s));
    store16<NT>(pl + c + 64, f16_chunk(x1, a, s));
  }
  for (; c < nchunk; c += 64) {
    const uint4 x = src[c];
    if (dst != nullptr) store16<NT>(dst + c, x);
    store16<NT>(pl + c, f16_chunk(x, a, s));
  }
}

struct F16Planes {
  uint4* g;              // [M, d_out / 8] chunks, or null
  uint4* phi;            // [M, d_in / 8], or null; both null: no float16 planes
  const float* ebound;   // [E][2]
  SegTable seg;
  int nt;                // non-temporal stores of the copies and the planes
};

__global__ __launch_bounds__(256) void gather_kernel(
    const int32_t* __restrict__ perm, const uint8_t* __restrict__ keep,
    const int32_t* __restrict__ g_row_index, const int32_t* __restrict__ phi_row_index,
    const float* __restrict__ alpha, const uint4* __restrict__ g, const uint4* __restrict__ phi,
    uint4* __restrict__ g_c, uint4* __restrict__ phi_c, float* __restrict__ alpha_c,
    float4* __restrict__ dphi_zero, int32_t M, int32_t P, int32_t g_rows, int32_t phi_rows,
    int32_t gch, int32_t pch, int32_t zch, uint4* __restrict__ pl_hi, uint4* __restrict__ pl_lo,
    int pl_from_phi, int32_t* __restrict__ zero, int nzero, F16Planes f16) {
  const int lane = threadIdx.x & 63;
  if (blockIdx.x == 0 && (int)threadIdx.x < nzero) zero[threadIdx.x] = 0;
  const int64_t job = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (job < M) {
    const int32_t j = (int32_t)job;
    const int32_t u = perm[j];
    if ((uint32_t)u >= (uint32_t)P) return;   // perm holds pair indices < P
    const int64_t gr = g_row_index ? (int64_t)g_row_index[u] : (int64_t)u;
    const int64_t pr = phi_row_index ? (int64_t)phi_row_index[u] : (int64_t)u;
    // source rows outside g's / phi's rows read as zeros
    const bool g_ok = (uint64_t)gr < (uint64_t)g_rows;
    const bool p_ok = (uint64_t)pr < (uint64_t)phi_rows;
    const float a = alpha[u];
    uint4* gdst = g_c != nullptr ? g_c + (int64_t)j * gch : nullptr;
    uint4* pdst = phi_c + (int64_t)j * pch;
    if (f16.g != nullptr || f16.phi != nullptr) {   // float16 weight-gradient planes
      const int e = expert_of_row(f16.seg, j);
      const int sa = f16_scale_exp(f16.ebound[2 * e]), sb = f16_scale_exp(f16.ebound[2 * e + 1]);
      uint4* pg = f16.g != nullptr ? f16.g + (int64_t)j * gch : nullptr;
      uint4* pp = f16.phi != nullptr ? f16.phi + (int64_t)j * pch : nullptr;
      const float ag = pl_from_phi ? 1.f : a, ap = pl_from_phi ? a : 1.f;
      if (!g_ok) zero_row(gdst, pg, nullptr, gch, lane);
      else if (pg != nullptr && f16.nt) copy_row_f16<true>(g + gr * gch, gdst, pg, ag, sa, gch, lane);
      else if (pg != nullptr) copy_row_f16(g + gr * gch, gdst, pg, ag, sa, gch, lane);
      else if (gdst != nullptr) copy_row(g + gr * gch, gdst, gch, lane);
      if (!p_ok) zero_row(pdst, pp, nullptr, pch, lane);
      else if (pp != nullptr && f16.nt) copy_row_f16<true>(phi + pr * pch, pdst, pp, ap, sb, pch, lane);
      else if (pp != nullptr) copy_row_f16(phi + pr * pch, pdst, pp, ap, sb, pch, lane);
      else copy_row(phi + pr * pch, pdst, pch, lane);
    } else if (pl_hi != nullptr && !pl_from_phi) {
      uint4* h = pl_hi + (int64_t)j * gch;
      uint4* l = pl_lo ? pl_lo + (int64_t)j * gch : nullptr;
      if (g_ok) copy_row_split(g + gr * gch, gdst, h, l, a, gch, lane);
      else zero_row(gdst, h, l, gch, lane);
    } else if (gdst != nullptr) {
      if (g_ok) copy_row(g + gr * gch, gdst, gch, lane);
      else zero_row(gdst, nullptr, nullptr, gch, lane);
    }
    if (f16.g != nullptr || f16.phi != nullptr) {
      // written above
    } else if (pl_hi != nullptr && pl_from_phi) {
      uint4* h = pl_hi + (int64_t)j * pch;
      uint4* l = pl_lo ? pl_lo + (int64_t)j * pch : nullptr;
      if (p_ok) copy_row_split(phi + pr * pch, pdst, h, l, a, pch, lane);
      else zero_row(pdst, h, l, pch, lane);
    } else {
      if (p_ok) copy_row(phi + pr * pch, pdst, pch, lane);
      else zero_row(pdst, nullptr, nullptr, pch, lane);
    }
    if (lane == 0) alpha_c[j] = a;
  } else if (dphi_zero != nullptr && job < (int64_t)M + P) {
    const int64_t u = job - M;
    if (!keep[u]) {
      float4* row = dphi_zero + u * zch;
      const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int c = lane; c < zch; c += 64) row[c] = z;
    }
  }
}

// Float16 weight-gradient mode, step 1: the Euclidean norms of both
// weight-gradient operand rows of every compacted row j into rn[j] = {|A
// row|, |B row|} (A the g row, B the phi row, the side carrying alpha times
// |alpha|), one wave per row, grid-strided.  The rows are read from the
// compacted buffers (perm null: row j, alpha[j] = alpha_c[j]), or through
// perm from the source rows the gather is about to copy.  Either way the
// values are bit for bit the score pass's per-pair norms (pair_sumsq_bf16);
// rows outside the sources read as zero rows, as in the gather.
__global__ __launch_bounds__(256) void row_norms_kernel(
    const uint4* __restrict__ g, const uint4* __restrict__ phi, const float* __restrict__ alpha,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ g_row_index,
    const int32_t* __restrict__ phi_row_index, int32_t M, int32_t P, int32_t g_rows,
    int32_t phi_rows, int32_t gch, int32_t pch, int alpha_on_phi, float2* __restrict__ rn) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * blockDim.x) >> 6;
  for (int j = wave; j < M; j += nwaves) {
    int64_t gr = j, pr = j;
    int32_t u = j;
    bool ok = true;
    if (perm != nullptr) {
      u = perm[j];
      ok = (uint32_t)u < (uint32_t)P;
      if (ok) {
        gr = g_row_index ? (int64_t)g_row_index[u] : (int64_t)u;
        pr = phi_row_index ? (int64_t)phi_row_index[u] : (int64_t)u;
      }
    }
    const bool g_ok = ok && (uint64_t)gr < (uint64_t)g_rows;
    const bool p_ok = ok && (uint64_t)pr < (uint64_t)phi_rows;
    const float2 sq = pair_sumsq_bf16(g + (g_ok ? gr : 0) * gch, gch, g_ok,
                                      phi + (p_ok ? pr : 0) * pch, pch, p_ok, lane);
    const float na = sqrtf(wave_sum(sq.x)), nb = sqrtf(wave_sum(sq.y));
    if (lane == 0) {
      const float aa = ok ? fabsf(alpha[u]) : 0.f;
      rn[j] = alpha_on_phi ? make_float2(na, aa * nb) : make_float2(aa * na, nb);
    }
  }
}

// Step 2: ebound[e] = the largest rn over expert e's rows (0 when it has
// none), one 1024-thread workgroup per expert, four independent loads in
// flight per thread (one workgroup streams a 10 K-row expert in three
// rounds, where 256 threads with one load each at a time took about 40).
constexpr int kBoundT = 1024;
__global__ __launch_bounds__(kBoundT) void expert_bound_kernel(SegTable seg,
                                                               const float2* __restrict__ rn,
                                                               float* __restrict__ ebound) {
  __shared__ uint32_t part[2][kBoundT / 64];
  const int e = blockIdx.x, tid = threadIdx.x;
  const int lo = seg.off[e], hi = seg.off[e + 1];
  uint32_t a = 0u, b = 0u;   // non-negative float32 bit patterns order like their values
  for (int j = lo + tid; j < hi; j += 4 * kBoundT) {
    float2 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = j + i * kBoundT;
      v[i] = r < hi ? rn[r] : make_float2(0.f, 0.f);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a = max(a, __float_as_uint(v[i].x));
      b = max(b, __float_as_uint(v[i].y));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    a = max(a, (uint32_t)__shfl_xor((int)a, off, 64));
    b = max(b, (uint32_t)__shfl_xor((int)b, off, 64));
  }
  if ((tid & 63) == 0) {
    part[0][tid >> 6] = a;
    part[1][tid >> 6] = b;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t ma = 0u, mb = 0u;
#pragma unroll
    for (int w = 0; w < kBoundT / 64; ++w) {
      ma = max(ma, part[0][w]);
      mb = max(mb, part[1][w]);
    }
    ebound[2 * e] = __uint_as_float(ma);
    ebound[2 * e + 1] = __uint_as_float(mb);
  }
}

// Step 2: the float16 planes from the compacted rows (either may be null),
// one wave per row (bit for bit the gather's planes of the one-call path).
__global__ __launch_bounds__(256) void split_f16_kernel(
    SegTable seg, const uint4* __restrict__ g_c, const uint4* __restrict__ phi_c,
    const float* __restrict__ alpha_c, int32_t M, int32_t gch, int32_t pch, int alpha_on_phi,
    const float* __restrict__ ebound, uint4* __restrict__ pa, uint4* __restrict__ pb) {
  const int lane = threadIdx.x & 63;
  const int64_t j = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (j >= M) return;
  const int e = expert_of_row(seg, (int)j);
  const float a = alpha_c[j];
  if (pa != nullptr)
    copy_row_f16(g_c + j * gch, nullptr, pa + j * gch, alpha_on_phi ? 1.f : a,
                 f16_scale_exp(ebound[2 * e]), gch, lane);
  if (pb != nullptr)
    copy_row_f16(phi_c + j * pch, nullptr, pb + j * pch, alpha_on_phi ? a : 1.f,
                 f16_scale_exp(ebound[2 * e + 1]), pch, lane);
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
                         int32_t P, int32_t g_rows, int32_t phi_rows, int32_t d_out,
                         int32_t d_in, hipStream_t s, const GatherPlanes& planes) {
  const int per = (dtype == LRMOE_BF16) ? 8 : 4;
  if ((planes.hi != nullptr || planes.f16_g != nullptr || planes.f16_phi != nullptr) &&
      dtype != LRMOE_BF16)
    return hipErrorInvalidValue;
  F16Planes f16{(uint4*)planes.f16_g, (uint4*)planes.f16_phi, planes.ebound, planes.seg,
                planes.stream_out ? 1 : 0};
  const int64_t jobs = (int64_t)M + (dphi_zero ? (int64_t)P : 0);
  if (jobs == 0) return planes.nzero > 0 ? launch_zero(planes.zero, planes.nzero, s) : hipSuccess;
  const int64_t blocks = (jobs + 3) / 4;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(256), 0, s, perm, keep,
                     g_row_index, phi_row_index, alpha, (const uint4*)g, (const uint4*)phi,
                     (uint4*)g_c, (uint4*)phi_c, alpha_c, (float4*)dphi_zero, M, P, g_rows,
                     phi_rows, d_out / per, d_in / per, d_in / 4, (uint4*)planes.hi, (uint4*)planes.lo,
                     planes.from_phi ? 1 : 0, planes.zero, planes.nzero, f16);
  return hipGetLastError();
}

hipError_t launch_expert_bounds(const SegTable& seg, const uint16_t* g, const uint16_t* phi,
                                const float* alpha, const int32_t* perm,
                                const int32_t* g_row_index, const int32_t* phi_row_index,
                                int32_t M, int32_t P, int32_t g_rows, int32_t phi_rows,
                                int32_t d_out, int32_t d_in, bool alpha_on_phi, float2* rn,
                                float* ebound, hipStream_t s) {
  if (M > 0) {
    // one row per wave, as in the score pass (fresh workgroups balance the CUs
    // better than waves looping over rows); grid-strided beyond 4 M rows
    int blocks = (M + 3) / 4;
    if (blocks > 256 * 4096) blocks = 256 * 4096;
    hipLaunchKernelGGL(row_norms_kernel, dim3(blocks), dim3(256), 0, s, (const uint4*)g,
                       (const uint4*)phi, alpha, perm, g_row_index, phi_row_index, M, P, g_rows,
                       phi_rows, d_out / 8, d_in / 8, alpha_on_phi ? 1 : 0, rn);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(expert_bound_kernel, dim3(seg.E), dim3(kBoundT), 0, s, seg, rn, ebound);
  return hipGetLastError();
}

hipError_t launch_split_f16(const SegTable& seg, const uint16_t* g_c, const uint16_t* phi_c,
                            const float* alpha_c, int32_t M, int32_t d_out, int32_t d_in,
                            bool alpha_on_phi, const float* ebound, uint16_t* f16_g,
                            uint16_t* f16_phi, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL(split_f16_kernel, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, s, seg,
                     (const uint4*)g_c, (const uint4*)phi_c, alpha_c, M, d_out / 8, d_in / 8,
                     alpha_on_phi ? 1 : 0, ebound, (uint4*)f16_g, (uint4*)f16_phi);
  return hipGetLastError();
}

}  // namespace lrmoe
