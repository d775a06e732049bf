// Variable-length grouped GEMMs over the compacted, expert-segmented buffers.
//
// The kept row counts q_e drive the GEMM sizes directly, with no padded rows
// ("LRMoE: Trimming Backward Work in Memory-Bound MoE Training", section "The
// part that is easy to get wrong").  Two products per expert e, with
// segment rows j in [s_e, s_e + q_e):
//
//   weight gradient  dW_e[o][i] = sum_j (alpha_j g_c[j][o]) phi_c[j][i]
//                    (the per-pair outer product (alpha_u g_t) phi_u^T of
//                    section "LRM: a decomposable contribution score", summed
//                    over kept pairs): M = d_out, N = d_in, K = q_e (varlen).
//   input gradient   dphi[perm[j]][i] = alpha_j sum_o g_c[j][o] W_e[o][i]
//                    (alpha_u W_e^T g_t, scattered back to the original pair
//                    row -- Portuguese write-up, compaction bullet): M = q_e
//                    (varlen), N = d_in, K = d_out.
//
// gfx950 mapping
//   * 256-thread workgroups (4 wave64s, 2x2) own a 128x128 fp32 tile; each
//     wave accumulates 64x64 with v_mfma_f32_32x32x16_bf16 (fp32 accumulate).
//   * Every operand is a bf16 plane in global memory.  alpha multiplies the
//     reduction index of dW, so it cannot be applied after the product: a
//     prologue writes alpha * (the narrower of g_c, phi_c) as bf16 hi + lo
//     planes (exact mode; hi only in single-rounding mode), and float32
//     storage is pre-split into hi + lo planes.  Products of split operands
//     sum hi*hi + hi*lo + lo*hi.  The MFMA loop does no conversions.
//   * Operand tiles of one K step (32) live in LDS in the global layout:
//     "KC" tiles (rows along M/N, K contiguous: g_c rows of the input
//     gradient) are read with 16-byte ds_read_b128 fragments; "MC" tiles
//     (rows along K, M/N contiguous: both operands of the weight gradient, W
//     of the input gradient) are read with ds_read_b64_tr_b16, which
//     transposes 4x16 bf16 blocks across each 16-lane group, so no operand is
//     ever transposed in memory.  16-byte chunks are XOR-swizzled per row so
//     that fragment reads spread over the LDS banks.
//   * Two LDS stages, one barrier per K step; global loads run two K steps
//     ahead of the MFMAs through two register stages.
//   * Scheduling: dW and dphi tiles share one launch.  Tiles are grouped in
//     blocks of an expert's tile grid that share operand panels; group g runs
//     on XCD g % 8 (workgroups are dispatched round-robin over the 8 XCDs), so
//     a group's panels are fetched into one L2.  dW groups come first, heaviest
//     experts first; the uniform dphi groups fill the tail.
#include "lrmoe_internal.h"

namespace lrmoe {
namespace {

#define LDS_AS __attribute__((address_space(3)))

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int kThreads = 256;
constexpr int kPlaneBytes = 128 * BK * 2;   // one bf16 operand plane of one K step

// ------------------------------------------------------------ LDS layouts
// KC: row r (0..127) holds K 0..31 as 4 chunks of 16 B.
__device__ __forceinline__ int kc_off(int r, int c) {
  return r * 64 + ((c ^ (((r >> 1) ^ (r >> 3)) & 3)) << 4);
}
// MC: row k (0..31) holds M/N 0..127 as 16 chunks of 16 B.
__device__ __forceinline__ int mc_off(int k, int c) { return k * 256 + ((c ^ ((k & 3) << 2)) << 4); }

// Fragment: 8 bf16 along K for MN index (mb + lane%32), K = kb + 8*(lane/32) + 0..7.
__device__ __forceinline__ i16x8 frag_kc(LDS_AS const char* t, int mb, int kb, int lane) {
  const int r = mb + (lane & 31);
  const int c = (kb >> 3) + (lane >> 5);
  return *reinterpret_cast<LDS_AS const i16x8*>(t + kc_off(r, c));
}

// ds_read_b64_tr_b16: within each 16-lane group, source lane s reads 4 bf16
// of row k0 + s/4 at columns n + 4*(s%4); lane l then holds column n + l%16
// for rows k0 .. k0+3.
__device__ __forceinline__ i16x8 frag_mc(LDS_AS const char* t, int mb, int kb, int lane) {
  const int G = lane >> 4, s = lane & 15;
  const int c = (mb >> 3) + 2 * (G & 1) + ((s & 3) >> 1);
  const int half = (s & 1) * 8;
  const int k0 = kb + 8 * (G >> 1) + (s >> 2);
  LDS_AS char* base = const_cast<LDS_AS char*>(t);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<LDS_AS i16x4*>(base + mc_off(k0, c) + half));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<LDS_AS i16x4*>(base + mc_off(k0 + 4, c) + half));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <bool MC>
__device__ __forceinline__ i16x8 frag(LDS_AS const char* t, int mb, int kb, int lane) {
  if constexpr (MC) return frag_mc(t, mb, kb, lane);
  else return frag_kc(t, mb, kb, lane);
}

__device__ __forceinline__ f32x16 mfma(i16x8 a, i16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

struct TileJob {
  int e, m0, n0;
};

// Decode the workgroup's tile from the group schedule; false = idle slot.
__device__ __forceinline__ bool decode(const GemmTable& tab, bool& is_dw, TileJob& job) {
  const int b = blockIdx.x;
  const int x = b % kXcds, i = b / kXcds;
  const int g = (i / kGroupSlots) * kXcds + x;   // group of this XCD's queue
  const int t = i % kGroupSlots;                 // slot inside the group
  if (g >= tab.total_groups) return false;
  is_dw = g < tab.dw_groups;
  const int32_t* goff = is_dw ? tab.dw_goff : tab.dp_goff;
  int lo = 0, hi = tab.E - 1;   // last rank r with goff[r] <= g
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (goff[mid] <= g) lo = mid; else hi = mid - 1;
  }
  const int e = is_dw ? (int)tab.order[lo] : lo;
  const int lg = g - goff[lo];
  const int gm = is_dw ? tab.dw_gm : tab.dp_gm;
  const int gn = is_dw ? tab.dw_gn : tab.dp_gn;
  if (t >= gm * gn) return false;
  const int ngn = (tab.tiles_n + gn - 1) / gn;
  const int tm = (lg / ngn) * gm + t / gn;
  const int tn = (lg % ngn) * gn + t % gn;
  const int q = tab.seg_off[e + 1] - tab.seg_off[e];
  const int tiles_m = is_dw ? tab.dw_tiles_m : (q + BM - 1) / BM;
  if (tm >= tiles_m || tn >= tab.tiles_n) return false;
  job.e = e;
  job.m0 = tm * BM;
  job.n0 = tn * BN;
  return true;
}

template <int PA, int PB>
struct Stage {
  u32x4 a[PA][2], b[PB][2];
};

struct Args {
  GemmOperands ops;
  const float* alpha_c;
  const int32_t* perm;
  float* dW;
  float* dphi;
  int32_t d_out, d_in, P;
};

// Buffer resource over [base, base + bytes): loads at or beyond `bytes`
// return zero, which masks ragged row and column edges without branches.
constexpr uint32_t kBufferFlags = 0x00020000u;   // gfx9 family: raw 32-bit data
constexpr uint32_t kOutOfRange = 0x80000000u;     // voffset that is never in range

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const uint16_t* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (int)(bytes > 0x7FFFFFFF ? 0x7FFFFFFF : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, n,
                                           (int)kBufferFlags);
}

__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
}

// One 128x128 output tile.  IS_DW: A (MC, rows = K) and B (MC, rows = K) are
// [M, d_out] / [M, d_in] segment rows.  Else A (KC, rows = M) = g_c segment
// rows and B (MC) = W_e.  PA/PB: bf16 planes of each operand.
template <bool IS_DW, int PA, int PB>
__device__ __forceinline__ void gemm_tile(const Args& args, const GemmTable& tab,
                                          const TileJob& job, LDS_AS char* smem) {
  constexpr bool A_MC = IS_DW;
  constexpr int kStage = (PA + PB) * kPlaneBytes;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int d_out = args.d_out, d_in = args.d_in;
  const int e = job.e, m0 = job.m0, n0 = job.n0;
  const int seg = tab.seg_off[e];
  const int q = tab.seg_off[e + 1] - seg;
  const int K = IS_DW ? q : d_out;

  const uint16_t* A[2];
  const uint16_t* B[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    A[p] = IS_DW ? args.ops.dw_a[p] : args.ops.dp_a[p];
    B[p] = IS_DW ? args.ops.dw_b[p] : args.ops.dp_b[p];
  }
  // Per-thread byte offsets inside one K step (fixed over the loop).
  uint32_t aoff[2], boff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int idx = tid + h * kThreads;
    if (A_MC) {   // row k of the step, 8-element chunk along M (o)
      const int k = idx >> 4, col = m0 + 8 * (idx & 15);
      aoff[h] = col < d_out ? (uint32_t)(k * d_out + col) * 2u : kOutOfRange;
    } else {      // row r of the tile, chunk along K (o); K offset added per step
      const int r = idx >> 2;
      aoff[h] = (uint32_t)(r * d_out + 8 * (idx & 3)) * 2u;
    }
    const int k = idx >> 4, col = n0 + 8 * (idx & 15);
    boff[h] = col < d_in ? (uint32_t)(k * d_in + col) * 2u : kOutOfRange;
  }

  // ---- global -> registers for the K step starting at k0
  auto gload = [&](int k0, Stage<PA, PB>& st) {
    const int krows = K - k0 < BK ? K - k0 : BK;
    __amdgpu_buffer_rsrc_t ra[PA], rb[PB];
#pragma unroll
    for (int p = 0; p < PA; ++p) {
      if (A_MC) ra[p] = rsrc(A[p] + ((int64_t)seg + k0) * d_out, (int64_t)krows * d_out * 2);
      else ra[p] = rsrc(A[p] + ((int64_t)seg + m0) * d_out, (int64_t)(q - m0) * d_out * 2);
    }
#pragma unroll
    for (int p = 0; p < PB; ++p) {
      const uint16_t* b0 = IS_DW ? B[p] + ((int64_t)seg + k0) * d_in
                                 : B[p] + ((int64_t)e * d_out + k0) * d_in;
      rb[p] = rsrc(b0, (int64_t)krows * d_in * 2);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t ao = aoff[h];
      if (!A_MC) {   // K columns of this step; past d_out reads zero
        const int kcol = k0 + 8 * ((tid + h * kThreads) & 3);
        ao = kcol < K ? ao + (uint32_t)k0 * 2u : kOutOfRange;
      }
#pragma unroll
      for (int p = 0; p < PA; ++p) st.a[p][h] = bload(ra[p], ao);
#pragma unroll
      for (int p = 0; p < PB; ++p) st.b[p][h] = bload(rb[p], boff[h]);
    }
  };
  // ---- registers -> one LDS stage: A planes then B planes
  auto lstore = [&](const Stage<PA, PB>& st, LDS_AS char* stage) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int idx = tid + h * kThreads;
      const int ao = A_MC ? mc_off(idx >> 4, idx & 15) : kc_off(idx >> 2, idx & 3);
      const int bo = mc_off(idx >> 4, idx & 15);
#pragma unroll
      for (int p = 0; p < PA; ++p)
        *reinterpret_cast<LDS_AS u32x4*>(stage + p * kPlaneBytes + ao) = st.a[p][h];
#pragma unroll
      for (int p = 0; p < PB; ++p)
        *reinterpret_cast<LDS_AS u32x4*>(stage + (PA + p) * kPlaneBytes + bo) = st.b[p][h];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  // ---- MFMAs of one K step: hi*hi (+ hi*lo_B) (+ lo_A*hi)
  auto compute = [&](LDS_AS const char* stage) {
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      i16x8 fb[PB][2], fa[PA][2];
#pragma unroll
      for (int p = 0; p < PB; ++p)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          fb[p][b] = frag_mc(stage + (PA + p) * kPlaneBytes, wn * 64 + b * 32, kk, lane);
#pragma unroll
      for (int p = 0; p < PA; ++p)
#pragma unroll
        for (int a = 0; a < 2; ++a)
          fa[p][a] = frag<A_MC>(stage + p * kPlaneBytes, wm * 64 + a * 32, kk, lane);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          acc[a][b] = mfma(fa[0][a], fb[0][b], acc[a][b]);
          if (PB == 2) acc[a][b] = mfma(fa[0][a], fb[PB - 1][b], acc[a][b]);
          if (PA == 2) acc[a][b] = mfma(fa[PA - 1][a], fb[0][b], acc[a][b]);
        }
    }
  };

  // ---- pipeline: loads two steps ahead, two LDS stages, one barrier per
  // step; unrolled by two so that each register stage has a fixed name.
  const int nk = (K + BK - 1) / BK;
  Stage<PA, PB> r0, r1;
  LDS_AS char* st0 = smem;
  LDS_AS char* st1 = smem + kStage;
  if (nk > 0) {
    gload(0, r0);
    gload(BK, r1);
    lstore(r0, st0);
    __syncthreads();
  }
  // Loads past the end of K see an empty buffer and return zeros without
  // touching memory, so they are issued unconditionally: branch-free code
  // lets each wait cover exactly the older register stage.
  for (int kt = 0; kt < nk; kt += 2) {
    gload((kt + 2) * BK, r0);
    compute(st0);
    lstore(r1, st1);
    __syncthreads();
    if (kt + 1 >= nk) break;
    gload((kt + 3) * BK, r1);
    compute(st1);
    lstore(r0, st0);
    __syncthreads();
  }

  // ---- epilogue: D[i][j] sits in lane j + 32*((i/4)%2), register (i%4) + 4*(i/8)
  const int fl = lane & 31;
  LDS_AS int32_t* s_perm = reinterpret_cast<LDS_AS int32_t*>(smem);
  LDS_AS float* s_alpha = reinterpret_cast<LDS_AS float*>(smem + BM * 4);
  if (!IS_DW) {   // destination row and alpha of the tile's 128 rows, via LDS
    if (tid < BM) {
      const bool ok = m0 + tid < q;
      const int32_t u = ok ? args.perm[seg + m0 + tid] : -1;
      s_perm[tid] = (uint32_t)u < (uint32_t)args.P ? u : -1;   // perm holds pair indices < P
      s_alpha[tid] = ok ? args.alpha_c[seg + m0 + tid] : 0.f;
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 2; ++a) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      const int mrow = m0 + wm * 64 + a * 32 + i;
      if (IS_DW) {
        if (mrow < d_out) {
          float* orow = args.dW + ((int64_t)e * d_out + mrow) * d_in;
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            const int col = n0 + wn * 64 + b * 32 + fl;
            if (col < d_in) orow[col] = acc[a][b][r];
          }
        }
      } else {
        const int lr = mrow - m0;
        const int32_t u = s_perm[lr];
        const float al = s_alpha[lr];
        if (u >= 0) {
          float* orow = args.dphi + (int64_t)u * d_in;
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            const int col = n0 + wn * 64 + b * 32 + fl;
            if (col < d_in) orow[col] = al * acc[a][b][r];
          }
        }
      }
    }
  }
}

template <int DW_PA, int DW_PB, int DP_PA, int DP_PB>
struct Cfg {
  static constexpr int dw_bytes = 2 * (DW_PA + DW_PB) * kPlaneBytes;
  static constexpr int dp_bytes = 2 * (DP_PA + DP_PB) * kPlaneBytes;
  static constexpr int bytes = dw_bytes > dp_bytes ? dw_bytes : dp_bytes;
};

template <int DW_PA, int DW_PB, int DP_PA, int DP_PB>
__global__ __launch_bounds__(kThreads, 2) void grouped_backward_kernel(Args args, GemmTable tab) {
  __shared__ __attribute__((aligned(16))) char smem_raw[Cfg<DW_PA, DW_PB, DP_PA, DP_PB>::bytes];
  LDS_AS char* smem = (LDS_AS char*)(smem_raw);
  bool is_dw;
  TileJob job;
  if (!decode(tab, is_dw, job)) return;
  if (is_dw)
    gemm_tile<true, DW_PA, DW_PB>(args, tab, job, smem);
  else
    gemm_tile<false, DP_PA, DP_PB>(args, tab, job, smem);
}

template <int DW_PA, int DW_PB, int DP_PA, int DP_PB>
hipError_t launch(const Args& args, const GemmTable& tab, hipStream_t s) {
  const int64_t queue = (tab.total_groups + kXcds - 1) / kXcds;
  const int64_t blocks = queue * kXcds * kGroupSlots;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_backward_kernel<DW_PA, DW_PB, DP_PA, DP_PB>), dim3((unsigned)blocks),
                     dim3(kThreads), 0, s, args, tab);
  return hipGetLastError();
}

// ------------------------------------------------------------ operand prologue
// hi/lo bf16 planes of alpha[row] * src[row][4c .. 4c+3].
template <bool F32>
__global__ __launch_bounds__(256) void split_kernel(const void* __restrict__ src, int64_t rows,
                                                    int32_t cols, const float* __restrict__ alpha,
                                                    uint16_t* __restrict__ hi,
                                                    uint16_t* __restrict__ lo) {
  const int64_t quads = rows * (cols / 4);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t qd = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; qd < quads; qd += stride) {
    const int64_t row = qd / (cols / 4);
    float x[4];
    if (F32) {
      const f32x4 v = reinterpret_cast<const f32x4*>(src)[qd];
      x[0] = v[0]; x[1] = v[1]; x[2] = v[2]; x[3] = v[3];
    } else {
      const u32x2 v = reinterpret_cast<const u32x2*>(src)[qd];
      x[0] = __uint_as_float(v[0] << 16); x[1] = __uint_as_float(v[0] & 0xFFFF0000u);
      x[2] = __uint_as_float(v[1] << 16); x[3] = __uint_as_float(v[1] & 0xFFFF0000u);
    }
    const float a = alpha ? alpha[row] : 1.f;
    bf16x8 hl;   // hi in 0..3, lo in 4..7
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float y = a * x[i];
      hl[i] = (__bf16)y;
      hl[4 + i] = (__bf16)(y - (float)hl[i]);
    }
    const u32x4 w = __builtin_bit_cast(u32x4, hl);
    reinterpret_cast<u32x2*>(hi)[qd] = u32x2{w[0], w[1]};
    if (lo) reinterpret_cast<u32x2*>(lo)[qd] = u32x2{w[2], w[3]};
  }
}

}  // namespace

hipError_t launch_split(int src_dtype, const void* src, int64_t rows, int32_t cols,
                        const float* alpha, uint16_t* hi, uint16_t* lo, hipStream_t s) {
  const int64_t quads = rows * (cols / 4);
  if (quads <= 0) return hipSuccess;
  int64_t blocks = (quads + 255) / 256;
  if (blocks > 256 * 16) blocks = 256 * 16;
  if (src_dtype == LRMOE_F32)
    hipLaunchKernelGGL(split_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, src, rows,
                       cols, alpha, hi, lo);
  else
    hipLaunchKernelGGL(split_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, src, rows,
                       cols, alpha, hi, lo);
  return hipGetLastError();
}

hipError_t launch_grouped_backward(const GemmTable& tab, const GemmOperands& ops,
                                   const int32_t* perm, const float* alpha_c, float* dW,
                                   float* dphi, int32_t d_out, int32_t d_in, int32_t P,
                                   hipStream_t s) {
  const Args args{ops, alpha_c, perm, dW, dphi, d_out, d_in, P};
  const int key = ops.dw_pa * 1000 + ops.dw_pb * 100 + ops.dp_pa * 10 + ops.dp_pb;
  switch (key) {
    case 1211: return launch<1, 2, 1, 1>(args, tab, s);   // bf16, alpha folded into phi
    case 2111: return launch<2, 1, 1, 1>(args, tab, s);   // bf16, alpha folded into g
    case 1111: return launch<1, 1, 1, 1>(args, tab, s);   // bf16, single rounding
    case 2222: return launch<2, 2, 2, 2>(args, tab, s);   // float32 storage
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lrmoe
