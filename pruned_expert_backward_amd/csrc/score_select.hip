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
// select (12 + 12 + 8-bit digits) on an order-preserving integer image of the
// float32 scores to find the q_e-th largest key tau_e and how many keys equal
// to tau_e are still needed; ties go to the lower pair index.  Keys of experts
// up to 24576 pairs are cached in LDS.  For larger experts the first digit is
// counted by many workgroups at once (select_hist_kernel, one per 16384-pair
// chunk, histograms in the workspace), and only the keys in that digit's bin
// are gathered into LDS for the later digits.  The same
// workgroup then scans the expert's pairs in index order (8 consecutive keys
// per thread, one workgroup prefix sum per 8192 keys), writes the keep flags
// and the compacted permutation (ascending pair index inside the segment).
// Global score reads are 16-byte vectors from an aligned start (a single
// workgroup's bandwidth is bounded by its vector memory instructions).
#include "lrmoe_internal.h"
#include "row_norm.h"

namespace lrmoe {
namespace {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float sumsq4(float4 x) {
  return fmaf(x.w, x.w, fmaf(x.z, x.z, fmaf(x.y, x.y, x.x * x.x)));
}
__device__ __forceinline__ float sumabs8(uint4 x) {
  // |bf16| = clear the sign bit of each half
  const float a = (bf16_lo(x.x & 0x7FFF7FFFu) + bf16_hi(x.x & 0x7FFF7FFFu)) +
                  (bf16_lo(x.y & 0x7FFF7FFFu) + bf16_hi(x.y & 0x7FFF7FFFu));
  const float b = (bf16_lo(x.z & 0x7FFF7FFFu) + bf16_hi(x.z & 0x7FFF7FFFu)) +
                  (bf16_lo(x.w & 0x7FFF7FFFu) + bf16_hi(x.w & 0x7FFF7FFFu));
  return a + b;
}
__device__ __forceinline__ float sumabs4(float4 x) {
  return (fabsf(x.x) + fabsf(x.y)) + (fabsf(x.z) + fabsf(x.w));
}

template <bool ABS, typename V>
__device__ __forceinline__ float reduce16(const V& x) {
  if constexpr (__is_same(V, uint4)) return ABS ? sumabs8(x) : sumsq8(x);
  else return ABS ? sumabs4(x) : sumsq4(x);
}

// Sum of squares (ABS: of absolute values) of one row held in 16-byte
// chunks, lane-strided, four independent loads in flight per lane.
template <bool ABS = false, typename V>
__device__ __forceinline__ float row_sumsq(const V* __restrict__ row, int nchunk, int lane) {
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  int c = lane;
  for (; c + 192 < nchunk; c += 256) {
    const V x0 = row[c], x1 = row[c + 64], x2 = row[c + 128], x3 = row[c + 192];
    a0 += reduce16<ABS>(x0); a1 += reduce16<ABS>(x1);
    a2 += reduce16<ABS>(x2); a3 += reduce16<ABS>(x3);
  }
  if (c < nchunk) {
    V x0, x1, x2;
    tail3(row, c, nchunk, x0, x1, x2);
    a0 += reduce16<ABS>(x0); a1 += reduce16<ABS>(x1); a2 += reduce16<ABS>(x2);
  }
  return (a0 + a1) + (a2 + a3);
}

// MODE: LRMOE_SCORE_LRM (alpha^2 ||g||^2 ||phi||^2), _GRAD_SQNORM (||g||^2)
// or _GRAD_L1 (sum |g_i|); the gradient-only rules never touch phi, unless
// RNORM.  RNORM (bf16 storage, the float16 weight-gradient mode): also write
// per pair the Euclidean norms of the two weight-gradient operand rows,
// rnorm[u] = {|A row|, |B row|}, A = the g row, B = the phi row, the side
// that carries alpha (alpha_on_phi) times |alpha_u|.  A row norm bounds the
// row's largest magnitude; the float16 planes' scales come from them.
template <bool BF16, int MODE, bool RNORM = false>
__global__ __launch_bounds__(256) void lrm_score_kernel(
    const void* __restrict__ g, const void* __restrict__ phi, const float* __restrict__ alpha,
    const int32_t* __restrict__ row_index, int32_t P, int32_t T, int32_t d_out, int32_t d_in,
    float* __restrict__ scores, float2* __restrict__ rnorm, int alpha_on_phi) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * blockDim.x) >> 6;
  const int per = BF16 ? 8 : 4;  // elements per 16-byte chunk
  const int gc = d_out / per, pc = d_in / per;
  constexpr bool L1 = MODE == LRMOE_SCORE_GRAD_L1;
  constexpr bool LRM = MODE == LRMOE_SCORE_LRM;
  for (int u = wave; u < P; u += nwaves) {
    const int64_t r = row_index ? (int64_t)row_index[u] : (int64_t)u;
    // a row index outside g's T rows reads as a zero row: no load at all
    const int gcr = (uint64_t)r < (uint64_t)T ? gc : 0;
    float gs, ps = 1.f;   // wave totals
    if constexpr (BF16) {
      const uint4* grow = reinterpret_cast<const uint4*>(g) + r * gc;
      const uint4* prow = reinterpret_cast<const uint4*>(phi) + (int64_t)u * pc;
      // both rows in one pass (phi only where the rule or the norms need it)
      constexpr bool WITH_PHI = LRM || RNORM;
      float gsq = 0.f, psq = 0.f;
      if (!L1 || RNORM) {
        const float2 sq = pair_sumsq_bf16(grow, gc, gcr > 0, prow, WITH_PHI ? pc : 0, true, lane);
        gsq = wave_sum(sq.x);
        if (WITH_PHI) psq = wave_sum(sq.y);
      }
      gs = L1 ? wave_sum(row_sumsq<true>(grow, gcr, lane)) : gsq;
      if (LRM) ps = psq;
      if (RNORM && lane == 0) {
        const float aa = fabsf(alpha[u]);
        const float ng = sqrtf(gsq), np = sqrtf(psq);
        rnorm[u] = alpha_on_phi ? make_float2(ng, aa * np) : make_float2(aa * ng, np);
      }
    } else {
      gs = wave_sum(row_sumsq<L1>(reinterpret_cast<const float4*>(g) + r * gc, gcr, lane));
      if (LRM)
        ps = wave_sum(row_sumsq(reinterpret_cast<const float4*>(phi) + (int64_t)u * pc, pc, lane));
    }
    if (lane == 0) {
      if (LRM) {
        const float a = alpha[u];
        scores[u] = ((a * a) * gs) * ps;
      } else {
        scores[u] = gs;
      }
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

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
// kSelLdsKeys (96 KiB): keys of one expert, or first-digit candidates
constexpr int kBins = kHistBins;     // first and second digits: 12 bits; last digit: 8 bits
constexpr int kHistPer = kHistChunk / kSelThreads;   // keys per thread in a histogram chunk
constexpr int kScanPer = 8;          // keys per thread per scan tile
constexpr int kScanTile = kSelThreads * kScanPer;
constexpr int kCandLoads = 16;       // 16-byte score loads in flight per thread (candidates)

// Inclusive prefix sum of v over the workgroup in thread order; `total`
// receives the workgroup sum.  wsum: kSelWaves LDS words.
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* wsum, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  uint32_t before = 0, t = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const uint32_t sw = wsum[w];
    before += (w < wave) ? sw : 0u;
    t += sw;
  }
  __syncthreads();   // wsum may be reused
  total = t;
  return before + x;
}

// Largest of v over the workgroup (every thread gets it).  wsum: kSelWaves
// LDS words.
__device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  if (lane == 0) wsum[wave] = v;
  __syncthreads();
  uint32_t m = 0u;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) m = max(m, wsum[w]);
  __syncthreads();   // wsum may be reused
  return m;
}

// Largest operand row norms of expert e's kept pairs (float16 weight-gradient
// mode): the workgroup's accumulators reduced and stored (whole expert) or
// merged with atomicMax (one chunk of a large expert; non-negative float32
// bit patterns order like their values).
__device__ __forceinline__ void put_kept_bound(const uint32_t (&kbound)[2], uint32_t* wsum,
                                             float* ebound, int e, bool merge) {
  const uint32_t a = block_max(kbound[0], wsum);
  const uint32_t b = block_max(kbound[1], wsum);
  if (threadIdx.x == 0) {
    if (merge) {
      atomicMax(reinterpret_cast<uint32_t*>(ebound) + 2 * e, a);
      atomicMax(reinterpret_cast<uint32_t*>(ebound) + 2 * e + 1, b);
    } else {
      ebound[2 * e] = __uint_as_float(a);
      ebound[2 * e + 1] = __uint_as_float(b);
    }
  }
}

struct Digit {
  uint32_t digit;   // bin holding the k-th largest key among the counted ones
  uint32_t k;       // its rank inside that bin (1-based, from the top)
  uint32_t count;   // keys in that bin
};

// Given a histogram of `nbins` (<= 4 per thread) bins in LDS, find the bin
// that holds the k-th largest counted key.  Thread t owns the 4 bins just
// below bin nbins - 4t, so the thread-order scan counts from the top bin.
__device__ __forceinline__ Digit find_digit(const uint32_t* hist, int nbins, uint32_t k,
                                            uint32_t* wsum, Digit* out) {
  const int tid = threadIdx.x;
  const int top = nbins - 4 * tid;   // this thread's bins: top-1 .. top-4
  uint32_t c[4] = {0u, 0u, 0u, 0u};
  if (top > 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = hist[top - 1 - j];
  }
  const uint32_t local = c[0] + c[1] + c[2] + c[3];
  uint32_t total;
  const uint32_t incl = block_scan(local, wsum, total);
  const uint32_t above = incl - local;
  if (local > 0 && above < k && k <= incl) {
    uint32_t cum = above;
    int j = 0;
    while (cum + c[j] < k) cum += c[j++];   // terminates: cum + sum(c) >= k
    out->digit = (uint32_t)(top - 1 - j);
    out->k = k - cum;
    out->count = c[j];
  }
  __syncthreads();
  const Digit d = *out;
  __syncthreads();
  return d;
}

// First-digit (key bits 31..20) histogram of one kHistChunk-pair chunk of a
// large expert, written to hist[chunk][kBins].
__global__ __launch_bounds__(kSelThreads) void select_hist_kernel(
    ExpertTable tab, const float* __restrict__ scores, uint32_t* __restrict__ hist_out) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[kBins];
  const int b = blockIdx.x, tid = threadIdx.x;
  int e = 0;
  while (e + 1 < tab.E && tab.hist_off[e + 1] <= b) ++e;   // chunk b belongs to expert e
  const int lo = tab.pair_off[e] + (b - tab.hist_off[e]) * kHistChunk;
  const int hi = min(lo + kHistChunk, tab.pair_off[e + 1]);
  for (int i = tid; i < kBins; i += kSelThreads) hist[i] = 0;
  __syncthreads();
  float v[kHistPer];
#pragma unroll
  for (int j = 0; j < kHistPer; ++j) {
    const int i = lo + j * kSelThreads + tid;
    v[j] = i < hi ? scores[i] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < kHistPer; ++j)
    if (lo + j * kSelThreads + tid < hi) atomicAdd(&hist[score_key(v[j]) >> 20], 1u);
  __syncthreads();
  reinterpret_cast<u32x4*>(hist_out + (size_t)b * kBins)[tid] =
      reinterpret_cast<const u32x4*>(hist)[tid];
}

// Scores [a, a + 4) for a multiple of 4 (the score array is 16-byte
// aligned), zeros past its end P.
__device__ __forceinline__ float4 load4(const float* __restrict__ scores, int a, int P) {
  if (a + 4 <= P) return *reinterpret_cast<const float4*>(scores + a);
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (a < P) v.x = scores[a];
  if (a + 1 < P) v.y = scores[a + 1];
  if (a + 2 < P) v.z = scores[a + 2];
  return v;
}

// ---- stable scan in pair order over pairs [base, end) of one expert: keep =
// key > tau, or key == tau among the first `need` of the expert's equal keys;
// kept pairs get consecutive compacted rows from seg.  run_gt / run_eq: the
// expert's keys above / equal to tau before `base`.  Keys come from keys_lds
// (pair g at keys_lds[g - lds_base]) or, when keys_lds is null, from the
// global scores.  Tiles start at the aligned index base & ~3; thread t owns 8
// consecutive pairs of a tile (those outside [base, end) are skipped); one
// workgroup scan of (#gt, #eq) per tile gives every position.  The next
// tile's loads go out before this tile is scanned.
//
// rnorm (or null): per-pair operand row norms of the float16 weight-gradient
// mode; the thread's largest over its kept pairs accumulate into kbound
// (float32 bits).
__device__ __forceinline__ void scan_keep(const uint32_t* keys_lds, const float* __restrict__ scores,
                                          int P, int base, int end, int lds_base, uint32_t tau,
                                          uint32_t need, uint32_t run_gt, uint32_t run_eq,
                                          uint32_t q, int seg, uint8_t* __restrict__ keep,
                                          int32_t* __restrict__ perm, uint32_t* wsum,
                                          const float2* __restrict__ rnorm, uint32_t (&kbound)[2]) {
  const int tid = threadIdx.x;
  const int gbeg = base & ~3;
  const bool cached = keys_lds != nullptr;
  auto load_tile = [&](int c, uint32_t (&kk)[kScanPer]) {
    const int g0 = c + tid * kScanPer;
    if (cached) {
#pragma unroll
      for (int j = 0; j < kScanPer; ++j) {
        const int g = g0 + j;
        kk[j] = (g >= base && g < end) ? keys_lds[g - lds_base] : 0u;
      }
    } else {
      // a tile wholly inside the score array: plain vector loads (load4's
      // per-lane bounds branch would wait for each load in turn)
      const bool full = c + kScanTile <= P;   // workgroup-uniform
#pragma unroll
      for (int h = 0; h < kScanPer / 4; ++h) {
        const float4 v = full ? *reinterpret_cast<const float4*>(scores + g0 + 4 * h)
                              : load4(scores, g0 + 4 * h, P);
        kk[4 * h] = score_key(v.x);
        kk[4 * h + 1] = score_key(v.y);
        kk[4 * h + 2] = score_key(v.z);
        kk[4 * h + 3] = score_key(v.w);
      }
    }
  };
  // operand row norms of the tile's pairs, loaded with its keys (loaded
  // only for kept pairs, each was a dependent load inside the scan)
  auto load_rn = [&](int c, float2 (&r)[kScanPer]) {
    if (rnorm == nullptr) return;
    const int g0 = c + tid * kScanPer;
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      const int g = g0 + j;
      r[j] = (g >= base && g < end) ? rnorm[g] : make_float2(0.f, 0.f);
    }
  };
  uint32_t key[kScanPer], key_next[kScanPer];
  float2 rn[kScanPer], rn_next[kScanPer];
  load_tile(gbeg, key);
  load_rn(gbeg, rn);
  for (int c = gbeg; c < end; c += kScanTile) {
    const int g0 = c + tid * kScanPer;
    if (c + kScanTile < end) {
      load_tile(c + kScanTile, key_next);
      load_rn(c + kScanTile, rn_next);
    }
    uint32_t ngt = 0, neq = 0;
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      const bool ok = g0 + j >= base && g0 + j < end;
      ngt += (ok && key[j] > tau) ? 1u : 0u;
      neq += (ok && key[j] == tau) ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t incl = block_scan((ngt << 16) | neq, wsum, tot);   // per tile < 2^16 each
    const uint32_t excl = incl - ((ngt << 16) | neq);
    uint32_t gt_before = run_gt + (excl >> 16);
    uint32_t eq_before = run_eq + (excl & 0xFFFFu);
    // kept keys before this thread: every greater key, and the equal keys
    // among the first `need` equal ones
    uint32_t pos = gt_before + (eq_before < need ? eq_before : need);
    uint32_t kept_bits = 0, valid_bits = 0;
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      const int g = g0 + j;
      if (g >= base && g < end) {
        const bool gt = key[j] > tau, eq = key[j] == tau;
        const bool kp = gt || (eq && eq_before < need);
        eq_before += eq ? 1u : 0u;
        valid_bits |= 1u << j;
        kept_bits |= (kp ? 1u : 0u) << j;
        if (kp) {
          if (pos < q) perm[seg + pos] = g;   // pos < q holds by construction
          ++pos;
          if (rnorm != nullptr) {
            kbound[0] = max(kbound[0], __float_as_uint(rn[j].x));
            kbound[1] = max(kbound[1], __float_as_uint(rn[j].y));
          }
        }
      }
    }
    // keep flags: whole 4-byte groups at once when the range owns all four
#pragma unroll
    for (int h = 0; h < kScanPer / 4; ++h) {
      const uint32_t vb = (valid_bits >> (4 * h)) & 15u, kb = (kept_bits >> (4 * h)) & 15u;
      const int g = g0 + 4 * h;
      if (vb == 15u) {
        *reinterpret_cast<uint32_t*>(keep + g) =
            (kb & 1u) | ((kb & 2u) << 7) | ((kb & 4u) << 14) | ((kb & 8u) << 21);
      } else if (vb != 0u) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (vb & (1u << t)) keep[g + t] = (kb >> t) & 1u;
      }
    }
    run_gt += tot >> 16;
    run_eq += tot & 0xFFFFu;
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      key[j] = key_next[j];
      rn[j] = rn_next[j];
    }
  }
}

__global__ __launch_bounds__(kSelThreads) void select_scan_kernel(
    ExpertTable tab, const float* __restrict__ scores, uint8_t* __restrict__ keep,
    int32_t* __restrict__ perm, int32_t* __restrict__ seg_offsets_out,
    const uint32_t* __restrict__ hist_in, uint32_t* __restrict__ tau_need,
    const float2* __restrict__ rnorm, float* __restrict__ ebound) {
  __shared__ uint32_t keys_lds[kSelLdsKeys];   // the expert's keys, or the candidates
  __shared__ __attribute__((aligned(16))) uint32_t hist[kBins];
  __shared__ uint32_t wsum[kSelWaves];
  __shared__ uint32_t cand_n;
  __shared__ Digit dig;

  const int e = blockIdx.x;
  const int tid = threadIdx.x;
  const int P = tab.pair_off[tab.E];
  const int base = tab.pair_off[e];
  const int end = tab.pair_off[e + 1];
  const int n = end - base;
  const int gbeg = base & ~3;   // 16-byte aligned start for vector reads of global scores
  const int seg = tab.seg_off[e];
  const uint32_t q = (uint32_t)(tab.seg_off[e + 1] - seg);

  const bool cached = n <= kSelLdsKeys;
  if (tid == 0) {
    seg_offsets_out[e] = seg;
    if (e == tab.E - 1) seg_offsets_out[tab.E] = tab.seg_off[tab.E];
    // largest kept row norms: an empty expert keeps 0; a large one starts at 0 and
    // its chunk scans merge into it
    if (ebound != nullptr && (n == 0 || !cached)) {
      ebound[2 * e] = 0.f;
      ebound[2 * e + 1] = 0.f;
    }
  }
  if (n == 0) return;
  if (cached) {
    for (int a = gbeg + 4 * tid; a < end; a += 4 * kSelThreads) {
      const float4 v = load4(scores, a, P);
      const float x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (a + j >= base && a + j < end) keys_lds[a + j - base] = score_key(x[j]);
    }
    __syncthreads();
  }

  // ---- radix select, most significant digit first: 12 + 12 + 8 bits.
  // tau = the q-th largest key; need = how many keys equal to tau are kept.
  uint32_t tau = 0xFFFFFFFFu, need = 0;   // q == 0: no key is above or equal
  if (q > 0) {
    // digit 1 (key bits 31..20) over every key: counted here from the LDS
    // cache, or summed from the chunk histograms of select_hist_kernel
    if (cached) {
      for (int i = tid; i < kBins; i += kSelThreads) hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += kSelThreads) atomicAdd(&hist[keys_lds[i] >> 20], 1u);
    } else {
      // eight chunk histograms in flight per thread (one at a time, the
      // latency of each load was paid in full)
      u32x4 h = {0u, 0u, 0u, 0u};
      const int c1 = tab.hist_off[e + 1];
      for (int c = tab.hist_off[e]; c < c1; c += 8) {
        u32x4 t[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          t[j] = c + j < c1 ? reinterpret_cast<const u32x4*>(hist_in + (size_t)(c + j) * kBins)[tid]
                            : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 8; ++j) h += t[j];
      }
      reinterpret_cast<u32x4*>(hist)[tid] = h;   // kSelThreads * 4 == kBins
    }
    __syncthreads();
    Digit d1 = find_digit(hist, kBins, q, wsum, &dig);
    uint32_t prefix = d1.digit << 20;
    uint32_t k = d1.k;

    // Remaining digits look only at keys whose top bits equal `prefix`: the
    // cached keys, or (large experts) the first-digit candidates collected
    // into LDS, or -- if there are too many of those -- all keys again.
    int nlist = n;
    bool from_global = false;
    if (!cached) {
      if (d1.count <= (uint32_t)kSelLdsKeys) {
        if (tid == 0) cand_n = 0;
        __syncthreads();
        // one workgroup streams the expert, kCandLoads 16-byte loads in
        // flight per thread; steps wholly inside the score array use plain
        // vector loads (no per-lane bounds branch).  This phase is bound by
        // what one CU can stream (about 35 GB/s measured: 9 us per 256 KiB
        // step) and by the LDS atomics of the appends; on a 286k-pair expert
        // it is still the selection's longest (about 45 us).
        for (int a0 = gbeg; a0 < end; a0 += 4 * kCandLoads * kSelThreads) {
          float4 v[kCandLoads];
          if (a0 + 4 * kCandLoads * kSelThreads <= P) {   // workgroup-uniform
#pragma unroll
            for (int j = 0; j < kCandLoads; ++j)
              v[j] = *reinterpret_cast<const float4*>(scores + a0 + 4 * (j * kSelThreads + tid));
          } else {
#pragma unroll
            for (int j = 0; j < kCandLoads; ++j)
              v[j] = load4(scores, a0 + 4 * (j * kSelThreads + tid), P);
          }
#pragma unroll
          for (int j = 0; j < kCandLoads; ++j) {
            const int a = a0 + 4 * (j * kSelThreads + tid);
            const float x[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const uint32_t key = score_key(x[t]);
              if (a + t >= base && a + t < end && (key >> 20) == d1.digit)
                keys_lds[atomicAdd(&cand_n, 1u)] = key;
            }
          }
        }
        __syncthreads();
        nlist = (int)d1.count;   // == cand_n
      } else {
        from_global = true;
      }
    }
    auto list_key = [&](int i) -> uint32_t {
      return from_global ? score_key(scores[base + i]) : keys_lds[i];
    };
    // digit 2 (bits 19..8), then digit 3 (bits 7..0)
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
      const int shift = pass == 0 ? 8 : 0;
      const int nb = pass == 0 ? kBins : 256;
      const uint32_t pmask = pass == 0 ? 0xFFF00000u : 0xFFFFFF00u;
      for (int i = tid; i < nb; i += kSelThreads) hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < nlist; i += kSelThreads) {
        const uint32_t key = list_key(i);
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & (uint32_t)(nb - 1)], 1u);
      }
      __syncthreads();
      const Digit dd = find_digit(hist, nb, k, wsum, &dig);
      prefix |= dd.digit << shift;
      k = dd.k;
    }
    tau = prefix;
    need = k;
  }

  if (!cached) {   // the chunk kernels scan large experts, many workgroups at once
    if (tid == 0) {
      tau_need[2 * e] = tau;
      tau_need[2 * e + 1] = need;
    }
    return;
  }
  uint32_t kbound[2] = {0u, 0u};
  scan_keep(keys_lds, scores, P, base, end, base, tau, need, 0u, 0u, q, seg, keep, perm, wsum,
            ebound != nullptr ? rnorm : nullptr, kbound);
  if (ebound != nullptr) put_kept_bound(kbound, wsum, ebound, e, false);
}

// Large experts (more than kSelLdsKeys pairs), after select_scan_kernel has
// found their tau and need: chunk b (the kHistChunk pairs of select_hist_kernel's
// chunk b) counts its keys above and equal to tau ...
__global__ __launch_bounds__(kSelThreads) void select_chunk_count_kernel(
    ExpertTable tab, const float* __restrict__ scores, const uint32_t* __restrict__ tau_need,
    uint32_t* __restrict__ counts) {
  __shared__ uint32_t wsum[kSelWaves];
  const int b = blockIdx.x, tid = threadIdx.x;
  int e = 0;
  while (e + 1 < tab.E && tab.hist_off[e + 1] <= b) ++e;
  const int lo = tab.pair_off[e] + (b - tab.hist_off[e]) * kHistChunk;
  const int hi = min(lo + kHistChunk, tab.pair_off[e + 1]);
  const uint32_t tau = tau_need[2 * e];
  uint32_t ngt = 0, neq = 0;
  float v[kHistPer];   // every load of the chunk in flight at once
#pragma unroll
  for (int j = 0; j < kHistPer; ++j) {
    const int i = lo + j * kSelThreads + tid;
    v[j] = i < hi ? scores[i] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < kHistPer; ++j) {
    const uint32_t k = score_key(v[j]);
    const bool ok = lo + j * kSelThreads + tid < hi;
    ngt += ok && k > tau ? 1u : 0u;
    neq += ok && k == tau ? 1u : 0u;
  }
  uint32_t tot;
  block_scan((ngt << 16) | neq, wsum, tot);   // chunk < 2^16 pairs
  if (tid == 0) {
    counts[2 * b] = tot >> 16;
    counts[2 * b + 1] = tot & 0xFFFFu;
  }
}

// ... and then scans its pairs, starting from the counts of the expert's
// earlier chunks: keep flags and compacted rows of many chunks at once.
__global__ __launch_bounds__(kSelThreads) void select_chunk_scan_kernel(
    ExpertTable tab, const float* __restrict__ scores, uint8_t* __restrict__ keep,
    int32_t* __restrict__ perm, const uint32_t* __restrict__ tau_need,
    const uint32_t* __restrict__ counts, const float2* __restrict__ rnorm,
    float* __restrict__ ebound) {
  __shared__ uint32_t wsum[kSelWaves];
  const int b = blockIdx.x;
  int e = 0;
  while (e + 1 < tab.E && tab.hist_off[e + 1] <= b) ++e;
  const int lo = tab.pair_off[e] + (b - tab.hist_off[e]) * kHistChunk;
  const int hi = min(lo + kHistChunk, tab.pair_off[e + 1]);
  // counts of the expert's earlier chunks, summed over the workgroup (one
  // load per thread instead of a serial chain of them)
  uint32_t pgt = 0, peq = 0;
  for (int c = tab.hist_off[e] + (int)threadIdx.x; c < b; c += kSelThreads) {
    pgt += counts[2 * c];
    peq += counts[2 * c + 1];
  }
  uint32_t run_gt, run_eq;
  block_scan(pgt, wsum, run_gt);
  block_scan(peq, wsum, run_eq);
  const int seg = tab.seg_off[e];
  const uint32_t q = (uint32_t)(tab.seg_off[e + 1] - seg);
  uint32_t kbound[2] = {0u, 0u};
  scan_keep(nullptr, scores, tab.pair_off[tab.E], lo, hi, 0, tau_need[2 * e],
            tau_need[2 * e + 1], run_gt, run_eq, q, seg, keep, perm, wsum,
            ebound != nullptr ? rnorm : nullptr, kbound);
  if (ebound != nullptr) put_kept_bound(kbound, wsum, ebound, e, true);
}

}  // namespace

template <int MODE>
void launch_score_mode(int dtype, dim3 grid, hipStream_t s, const void* g, const void* phi,
                       const float* alpha, const int32_t* row_index, int32_t P, int32_t T,
                       int32_t d_out, int32_t d_in, float* scores, float2* rnorm,
                       int alpha_on_phi) {
  if (dtype == LRMOE_BF16 && rnorm != nullptr)
    hipLaunchKernelGGL((lrm_score_kernel<true, MODE, true>), grid, dim3(256), 0, s, g, phi, alpha,
                       row_index, P, T, d_out, d_in, scores, rnorm, alpha_on_phi);
  else if (dtype == LRMOE_BF16)
    hipLaunchKernelGGL((lrm_score_kernel<true, MODE>), grid, dim3(256), 0, s, g, phi, alpha,
                       row_index, P, T, d_out, d_in, scores, rnorm, alpha_on_phi);
  else
    hipLaunchKernelGGL((lrm_score_kernel<false, MODE>), grid, dim3(256), 0, s, g, phi, alpha,
                       row_index, P, T, d_out, d_in, scores, rnorm, alpha_on_phi);
}

hipError_t launch_score(int dtype, int mode, const void* g, const void* phi, const float* alpha,
                        const int32_t* row_index, int32_t P, int32_t T, int32_t d_out,
                        int32_t d_in, float* scores, hipStream_t s, float2* rnorm,
                        int alpha_on_phi) {
  if (P <= 0) return hipSuccess;
  const int waves_per_block = 4;
  int blocks = (P + waves_per_block - 1) / waves_per_block;
  // 8 workgroups (32 waves) fit on a CU at a time; eight times that many
  // let the dispatcher balance CUs and channels as workgroups finish (a
  // streaming read reaches 6.3 TB/s so, against 5.9 with one resident wave
  // per slot looping over the whole range)
  if (blocks > 256 * 64) blocks = 256 * 64;
  const dim3 grid(blocks);
  if (mode == LRMOE_SCORE_GRAD_SQNORM)
    launch_score_mode<LRMOE_SCORE_GRAD_SQNORM>(dtype, grid, s, g, phi, alpha, row_index, P, T,
                                               d_out, d_in, scores, rnorm, alpha_on_phi);
  else if (mode == LRMOE_SCORE_GRAD_L1)
    launch_score_mode<LRMOE_SCORE_GRAD_L1>(dtype, grid, s, g, phi, alpha, row_index, P, T,
                                           d_out, d_in, scores, rnorm, alpha_on_phi);
  else
    launch_score_mode<LRMOE_SCORE_LRM>(dtype, grid, s, g, phi, alpha, row_index, P, T, d_out,
                                       d_in, scores, rnorm, alpha_on_phi);
  return hipGetLastError();
}

hipError_t launch_select_scan(const ExpertTable& tab, const float* scores, uint8_t* keep,
                              int32_t* perm, int32_t* seg_offsets_out, uint32_t* hist,
                              hipStream_t s, const float2* rnorm, float* ebound) {
  const int chunks = tab.hist_off[tab.E];
  // workspace: chunk histograms, then tau / need per expert, then per-chunk counts
  uint32_t* tau_need = hist + (size_t)chunks * kBins;
  uint32_t* counts = tau_need + 2 * kMaxE;
  if (chunks > 0) {
    hipLaunchKernelGGL(select_hist_kernel, dim3(chunks), dim3(kSelThreads), 0, s, tab, scores,
                       hist);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(select_scan_kernel, dim3(tab.E), dim3(kSelThreads), 0, s, tab, scores,
                     keep, perm, seg_offsets_out, hist, tau_need, rnorm, ebound);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || chunks == 0) return err;
  hipLaunchKernelGGL(select_chunk_count_kernel, dim3(chunks), dim3(kSelThreads), 0, s, tab,
                     scores, tau_need, counts);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(select_chunk_scan_kernel, dim3(chunks), dim3(kSelThreads), 0, s, tab,
                     scores, keep, perm, tau_need, counts, rnorm, ebound);
  return hipGetLastError();
}

}  // namespace lrmoe
