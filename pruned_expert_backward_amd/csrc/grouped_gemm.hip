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
// gfx950 mapping: 256-thread workgroups (4 wave64s in a 2x2 grid) own a
// 128x128 fp32 output tile; each wave accumulates 64x64 with
// v_mfma_f32_32x32x16_bf16.  Operand tiles are staged through LDS as bf16 in
// a K-contiguous layout when global memory is K-contiguous (g_c rows for the
// input gradient; 16-byte fragment reads), and in the global MN-contiguous
// layout otherwise (g_c, phi_c and W rows), read back K-wise.  Global loads
// of the next K step are issued before the MFMAs of the current one.
//
// Exact alpha folding: alpha multiplies the reduction index of dW, so it
// cannot be applied after the product.  alpha*g is formed in fp32 and split
// into bf16 hi + lo (two MFMA terms); float32 storage splits both operands
// (three terms: hi*hi + hi*lo + lo*hi).  The single-rounding mode keeps only
// the hi term.
#include "lrmoe_internal.h"

namespace lrmoe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int KC_LD = BK + 8;      // bf16 per row of a K-contiguous tile (80 B)
constexpr int MC_LD = 128 + 4;     // bf16 per K row of an MN-contiguous tile (264 B)
constexpr int kThreads = 256;

template <bool MC>
struct TileSize;
template <> struct TileSize<true> { static constexpr int elems = BK * MC_LD; };
template <> struct TileSize<false> { static constexpr int elems = BM * KC_LD; };

// Eight consecutive global elements of one operand row, widened to fp32.
template <typename TIn>
struct Raw8 {
  float v[8];
};

template <typename TIn>
__device__ __forceinline__ void load8(const TIn* __restrict__ p, int valid_elems, Raw8<TIn>& r);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* __restrict__ p, int valid_elems,
                                                Raw8<uint16_t>& r) {
  uint4 w = make_uint4(0, 0, 0, 0);
  if (valid_elems >= 8) w = *reinterpret_cast<const uint4*>(p);
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r.v[2 * i] = __uint_as_float(ws[i] << 16);
    r.v[2 * i + 1] = __uint_as_float(ws[i] & 0xFFFF0000u);
  }
}

template <>
__device__ __forceinline__ void load8<float>(const float* __restrict__ p, int valid_elems,
                                             Raw8<float>& r) {
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
  if (valid_elems >= 4) a = *reinterpret_cast<const float4*>(p);
  if (valid_elems >= 8) b = *reinterpret_cast<const float4*>(p + 4);
  r.v[0] = a.x; r.v[1] = a.y; r.v[2] = a.z; r.v[3] = a.w;
  r.v[4] = b.x; r.v[5] = b.y; r.v[6] = b.z; r.v[7] = b.w;
}

// Write 8 values as bf16 hi (and lo residual) planes into LDS.
template <int SPLIT>
__device__ __forceinline__ void store8(const float (&x)[8], __bf16* hi, __bf16* lo, bool aligned16) {
  __bf16 h[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h[i] = (__bf16)x[i];
    if (SPLIT == 2) l[i] = (__bf16)(x[i] - (float)h[i]);
  }
  if (aligned16) {
    *reinterpret_cast<bf16x8*>(hi) = *reinterpret_cast<const bf16x8*>(h);
    if (SPLIT == 2) *reinterpret_cast<bf16x8*>(lo) = *reinterpret_cast<const bf16x8*>(l);
  } else {
    uint2* dh = reinterpret_cast<uint2*>(hi);
    dh[0] = reinterpret_cast<const uint2*>(h)[0];
    dh[1] = reinterpret_cast<const uint2*>(h)[1];
    if (SPLIT == 2) {
      uint2* dl = reinterpret_cast<uint2*>(lo);
      dl[0] = reinterpret_cast<const uint2*>(l)[0];
      dl[1] = reinterpret_cast<const uint2*>(l)[1];
    }
  }
}

// MFMA operand fragment (8 bf16 along K) for MN index mn, K offset k.
template <bool MC>
__device__ __forceinline__ bf16x8 frag(const __bf16* tile, int mn, int k);

template <>
__device__ __forceinline__ bf16x8 frag<false>(const __bf16* tile, int mn, int k) {
  return *reinterpret_cast<const bf16x8*>(tile + mn * KC_LD + k);
}

template <>
__device__ __forceinline__ bf16x8 frag<true>(const __bf16* tile, int mn, int k) {
  bf16x8 f;
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = tile[(k + i) * MC_LD + mn];
  return f;
}

struct GemmArgs {
  const void* a;         // dW: g_c (MC)   dphi: g_c (KC)
  const void* b;         // dW: phi_c (MC) dphi: W (MC)
  const float* alpha_c;
  const int32_t* perm;
  float* out;            // dW or dphi
  int32_t d_out, d_in;
  int32_t P;             // rows of dphi
};

// One operand tile of one K step, held in registers between the global load
// and the LDS store.
template <typename TIn>
struct Stage {
  Raw8<TIn> r[2];
  float s[2];
};

template <bool IS_DW, int SPLIT_A, int SPLIT_B>
struct TileLds {
  static constexpr int a_elems = TileSize<IS_DW>::elems;
  static constexpr int b_elems = TileSize<true>::elems;
  static constexpr int bytes = 2 * (SPLIT_A * a_elems + SPLIT_B * b_elems);
};

// One 128x128 output tile.  IS_DW: weight gradient (A = alpha * g_c,
// MN-contiguous) else input gradient (A = g_c, K-contiguous).  B is
// MN-contiguous in both.  `bid` indexes this product's tiles.
template <typename TIn, bool IS_DW, int SPLIT_A, int SPLIT_B>
__device__ __forceinline__ void gemm_tile(const GemmArgs& args, const GemmTable& tab, int bid,
                                          __bf16* lds) {
  constexpr bool A_MC = IS_DW;
  using L = TileLds<IS_DW, SPLIT_A, SPLIT_B>;
  __bf16* lds_a[2] = {lds, lds + (SPLIT_A - 1) * L::a_elems};
  __bf16* lds_b[2] = {lds + SPLIT_A * L::a_elems, lds + SPLIT_A * L::a_elems + (SPLIT_B - 1) * L::b_elems};

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int d_out = args.d_out, d_in = args.d_in;

  // ---- which expert / tile this workgroup owns
  int e, m0, n0, seg, q;
  if (IS_DW) {
    const int tpe = tab.tiles_m_fixed * tab.tiles_n;
    e = tab.order[bid / tpe];
    const int t = bid % tpe;
    m0 = (t / tab.tiles_n) * BM;
    n0 = (t % tab.tiles_n) * BN;
  } else {
    int lo = 0, hi = tab.E - 1;   // largest e with tile_off[e] <= bid
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tab.tile_off[mid] <= bid) lo = mid; else hi = mid - 1;
    }
    e = lo;
    const int t = bid - tab.tile_off[e];
    m0 = (t / tab.tiles_n) * BM;
    n0 = (t % tab.tiles_n) * BN;
  }
  seg = tab.seg_off[e];
  q = tab.seg_off[e + 1] - seg;
  const int K = IS_DW ? q : d_out;

  const TIn* A = reinterpret_cast<const TIn*>(args.a);
  const TIn* B = reinterpret_cast<const TIn*>(args.b);
  if (!IS_DW) B += (int64_t)e * d_out * d_in;

  // ---- global -> register staging
  auto load_a = [&](int k0, Stage<TIn>& st) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = tid + h * kThreads;
      if (A_MC) {   // rows are K (segment rows), columns are M (= o)
        const int k = c >> 4, mn = (c & 15) * 8;
        const bool kv = (k0 + k) < K;
        const int valid = kv ? (d_out - (m0 + mn)) : 0;
        const int64_t row = (int64_t)seg + k0 + k;
        load8<TIn>(A + row * d_out + m0 + mn, valid, st.r[h]);
        st.s[h] = kv ? args.alpha_c[row] : 0.f;
      } else {      // rows are M (segment rows), columns are K (= o)
        const int r = c >> 2, kc = (c & 3) * 8;
        const bool rv = (m0 + r) < q;
        const int valid = rv ? (K - (k0 + kc)) : 0;
        load8<TIn>(A + ((int64_t)seg + m0 + r) * d_out + k0 + kc, valid, st.r[h]);
        st.s[h] = 1.f;
      }
    }
  };
  auto load_b = [&](int k0, Stage<TIn>& st) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = tid + h * kThreads;
      const int k = c >> 4, mn = (c & 15) * 8;
      const bool kv = (k0 + k) < K;
      const int valid = kv ? (d_in - (n0 + mn)) : 0;
      const int64_t row = IS_DW ? ((int64_t)seg + k0 + k) : (int64_t)(k0 + k);
      load8<TIn>(B + row * d_in + n0 + mn, valid, st.r[h]);
      st.s[h] = 1.f;
    }
  };
  auto store_a = [&](const Stage<TIn>& st) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = tid + h * kThreads;
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = IS_DW ? st.s[h] * st.r[h].v[i] : st.r[h].v[i];
      if (A_MC) {
        const int k = c >> 4, mn = (c & 15) * 8;
        store8<SPLIT_A>(x, lds_a[0] + k * MC_LD + mn, lds_a[1] + k * MC_LD + mn, false);
      } else {
        const int r = c >> 2, kc = (c & 3) * 8;
        store8<SPLIT_A>(x, lds_a[0] + r * KC_LD + kc, lds_a[1] + r * KC_LD + kc, true);
      }
    }
  };
  auto store_b = [&](const Stage<TIn>& st) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = tid + h * kThreads;
      const int k = c >> 4, mn = (c & 15) * 8;
      store8<SPLIT_B>(st.r[h].v, lds_b[0] + k * MC_LD + mn, lds_b[1] + k * MC_LD + mn, false);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int nk = (K + BK - 1) / BK;
  Stage<TIn> sa, sb;
  if (nk > 0) {
    load_a(0, sa);
    load_b(0, sb);
  }
  const int fl = lane & 31, fk = 8 * (lane >> 5);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
    store_a(sa);
    store_b(sb);
    __syncthreads();
    if (kt + 1 < nk) {
      load_a((kt + 1) * BK, sa);
      load_b((kt + 1) * BK, sb);
    }
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 fa[SPLIT_A][2], fb[SPLIT_B][2];
#pragma unroll
      for (int s = 0; s < SPLIT_A; ++s)
#pragma unroll
        for (int a = 0; a < 2; ++a) fa[s][a] = frag<A_MC>(lds_a[s], wm * 64 + a * 32 + fl, kk + fk);
#pragma unroll
      for (int s = 0; s < SPLIT_B; ++s)
#pragma unroll
        for (int b = 0; b < 2; ++b) fb[s][b] = frag<true>(lds_b[s], wn * 64 + b * 32 + fl, kk + fk);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[0][a], fb[0][b], acc[a][b], 0, 0, 0);
          if (SPLIT_B == 2)
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[0][a], fb[SPLIT_B - 1][b], acc[a][b], 0, 0, 0);
          if (SPLIT_A == 2)
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[SPLIT_A - 1][a], fb[0][b], acc[a][b], 0, 0, 0);
        }
    }
  }

  // ---- epilogue: D[i][j] sits in lane j + 32*((i/4)%2), register (i%4) + 4*(i/8)
#pragma unroll
  for (int a = 0; a < 2; ++a) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      const int mrow = m0 + wm * 64 + a * 32 + i;
      if (IS_DW) {
        if (mrow < d_out) {
          float* orow = args.out + ((int64_t)e * d_out + mrow) * d_in;
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            const int col = n0 + wn * 64 + b * 32 + fl;
            if (col < d_in) orow[col] = acc[a][b][r];
          }
        }
      } else if (mrow < q) {
        const int64_t jj = (int64_t)seg + mrow;
        const int32_t u = args.perm[jj];
        const float al = args.alpha_c[jj];
        if ((uint32_t)u < (uint32_t)args.P) {   // perm holds pair indices < P
          float* orow = args.out + (int64_t)u * d_in;
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

// One launch for both products: blocks [0, dw_tiles) are weight-gradient
// tiles (heaviest experts first), the rest are input-gradient tiles, which
// have uniform work and fill the tail left by skewed expert sizes.
template <typename TIn, int DW_SA, int DW_SB, int DP_SA, int DP_SB>
__global__ __launch_bounds__(kThreads, 2) void grouped_backward_kernel(GemmArgs dw, GemmArgs dp,
                                                                       GemmTable tab) {
  constexpr int kDw = TileLds<true, DW_SA, DW_SB>::bytes;
  constexpr int kDp = TileLds<false, DP_SA, DP_SB>::bytes;
  __shared__ __attribute__((aligned(16))) __bf16 lds[(kDw > kDp ? kDw : kDp) / 2];
  const int bid = blockIdx.x;
  if (bid < tab.dw_tiles)
    gemm_tile<TIn, true, DW_SA, DW_SB>(dw, tab, bid, lds);
  else
    gemm_tile<TIn, false, DP_SA, DP_SB>(dp, tab, bid - tab.dw_tiles, lds);
}

template <typename TIn, int DW_SA, int DW_SB, int DP_SA, int DP_SB>
hipError_t launch(const GemmArgs& dw, const GemmArgs& dp, const GemmTable& tab, hipStream_t s) {
  const int blocks = tab.dw_tiles + tab.dp_tiles;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_backward_kernel<TIn, DW_SA, DW_SB, DP_SA, DP_SB>), dim3(blocks),
                     dim3(kThreads), 0, s, dw, dp, tab);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_backward(int dtype, int dw_mode, const GemmTable& tab,
                                   const int32_t* perm, const float* alpha_c, const void* g_c,
                                   const void* phi_c, const void* W, float* dW, float* dphi,
                                   int32_t d_out, int32_t d_in, int32_t P, hipStream_t s) {
  GemmArgs dw{g_c, phi_c, alpha_c, nullptr, dW, d_out, d_in, P};
  GemmArgs dp{g_c, W, alpha_c, perm, dphi, d_out, d_in, P};
  if (dtype == LRMOE_F32) return launch<float, 2, 2, 2, 2>(dw, dp, tab, s);
  if (dw_mode == LRMOE_DW_BF16) return launch<uint16_t, 1, 1, 1, 1>(dw, dp, tab, s);
  return launch<uint16_t, 2, 1, 1, 1>(dw, dp, tab, s);
}

}  // namespace lrmoe
