// Sum of squares of one bf16 row, reduced over the wave64 that reads it.
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

// Sum of squares of 8 bf16 values: one packed bf16 dot product per pair
// (v_dot2c_f32_bf16: both products exact in float32, accumulated in float32).
__device__ __forceinline__ float dot2sq(uint32_t w, float acc) {
  const bf16x2_t b = __builtin_bit_cast(bf16x2_t, w);
  return __builtin_amdgcn_fdot2_f32_bf16(b, b, acc, false);
}
__device__ __forceinline__ float sumsq8(uint4 x) {
  return dot2sq(x.w, dot2sq(x.z, dot2sq(x.y, dot2sq(x.x, 0.f))));
}

// The lane's last 1..3 chunks of a row at once (zeros past the row end), so
// that a short tail costs one memory round trip, not one per chunk.
template <typename V>
__device__ __forceinline__ void tail3(const V* __restrict__ row, int c, int nchunk, V& x0, V& x1,
                                      V& x2) {
  const V z = {};
  x0 = row[c];
  x1 = c + 64 < nchunk ? row[c + 64] : z;
  x2 = c + 128 < nchunk ? row[c + 128] : z;
}

// This lane's share of the sum of squares of a bf16 row of nchunk 16-byte
// chunks (lane-strided, four independent loads in flight per lane); the
// caller reduces it with wave_sum.
__device__ __forceinline__ float row_sumsq_bf16(const uint4* __restrict__ row, int nchunk,
                                                int lane) {
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  int c = lane;
  for (; c + 192 < nchunk; c += 256) {
    const uint4 x0 = row[c], x1 = row[c + 64], x2 = row[c + 128], x3 = row[c + 192];
    a0 += sumsq8(x0); a1 += sumsq8(x1); a2 += sumsq8(x2); a3 += sumsq8(x3);
  }
  if (c < nchunk) {
    uint4 x0, x1, x2;
    tail3(row, c, nchunk, x0, x1, x2);
    a0 += sumsq8(x0); a1 += sumsq8(x1); a2 += sumsq8(x2);
  }
  return (a0 + a1) + (a2 + a3);
}

// Euclidean norm of a bf16 row (an upper bound of its largest |x|; wave
// uniform).
__device__ __forceinline__ float row_norm_bf16(const uint4* __restrict__ row, int nchunk,
                                               int lane) {
  return sqrtf(wave_sum(row_sumsq_bf16(row, nchunk, lane)));
}

}  // namespace lrmoe
