// Sums of squares of bf16 rows, reduced over the wave64 that reads them.
// Shared by the score pass and the float16 weight-gradient planes' bounds, so
// that both compute bit for bit the same row norms.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lrmoe {

// Value of lane l ^ 1, l ^ 2 (quad permutes), the mirror lane inside each
// 8-lane half row and inside each 16-lane row: four DPP steps combine every
// row of 16 lanes without touching the LDS.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

// Sum over the wave: rows of 16 by DPP, the four row sums read with
// v_readlane (uniform result, fixed order).
__device__ __forceinline__ float wave_sum(float v) {
  v += __uint_as_float(dpp<0xB1>(__float_as_uint(v)));    // quad_perm [1,0,3,2]
  v += __uint_as_float(dpp<0x4E>(__float_as_uint(v)));    // quad_perm [2,3,0,1]
  v += __uint_as_float(dpp<0x141>(__float_as_uint(v)));   // row_half_mirror
  v += __uint_as_float(dpp<0x140>(__float_as_uint(v)));   // row_mirror
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));

// 16-byte load; NT marks it non-temporal (streamed once: the line is not kept
// in the caches for reuse).
template <bool NT>
__device__ __forceinline__ uint4 load16(const uint4* __restrict__ p) {
  if constexpr (NT) {
    const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
  } else {
    return *p;
  }
}

// Sum of squares of 8 bf16 values: one packed bf16 dot product per pair
// (v_dot2c_f32_bf16: both products exact in float32, accumulated in float32).
__device__ __forceinline__ float dot2sq(uint32_t w, float acc) {
  const bf16x2_t b = __builtin_bit_cast(bf16x2_t, w);
  return __builtin_amdgcn_fdot2_f32_bf16(b, b, acc, false);
}
__device__ __forceinline__ float sumsq8(uint4 x) {
  return dot2sq(x.w, dot2sq(x.z, dot2sq(x.y, dot2sq(x.x, 0.f))));
}

// This lane's shares of the sums of squares of a pair's two bf16 rows: the
// g row (gc 16-byte chunks) and the phi row (pc chunks), read as one
// sequence of chunks c = lane + 64 k (c < gc from g, else chunk c - gc of
// phi), sixteen loads in flight per lane (one round trip for a GLM pair's
// 688 chunks; with eight, two, and the score pass ran 2.4 % slower on the
// 655 360-pair workload despite twice the waves per SIMD).  Chunk i of a
// batch adds into accumulator i % 4 in increasing i, so the sums do not
// depend on the batch size.  A row that is not there (g_ok / p_ok
// false) reads as zeros but keeps its chunk positions, so the other row's
// sum is the same either way.  {x: g, y: phi}; reduce each with wave_sum.
// NT: non-temporal loads, for the score pass, which streams every routed
// row once (cached loads there left the previous step's dirty lines to be
// written back under it: 8 % slower on the 655 360-pair workload, 29 % on
// the 32 768-pair one).
template <bool NT = false>
__device__ __forceinline__ float2 pair_sumsq_bf16(const uint4* __restrict__ g, int gc, bool g_ok,
                                                  const uint4* __restrict__ phi, int pc,
                                                  bool p_ok, int lane) {
  float ag[4] = {0.f, 0.f, 0.f, 0.f}, ap[4] = {0.f, 0.f, 0.f, 0.f};
  const int n = gc + pc;
  for (int base = lane; base < n; base += 64 * 16) {
    uint4 x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c = base + 64 * i;
      const bool in_g = c < gc;
      const uint4* src = in_g ? g + c : phi + (c - gc);
      const bool ok = c < n && (in_g ? g_ok : p_ok);
      x[i] = ok ? load16<NT>(src) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float v = sumsq8(x[i]);
      if (base + 64 * i < gc) ag[i & 3] += v;
      else ap[i & 3] += v;
    }
  }
  return make_float2((ag[0] + ag[1]) + (ag[2] + ag[3]), (ap[0] + ap[1]) + (ap[2] + ap[3]));
}

}  // namespace lrmoe
