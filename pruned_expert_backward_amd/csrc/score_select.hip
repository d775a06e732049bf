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
// bullet).  An MSB-first radix select (12 + 12 + 8-bit digits) on an
// order-preserving integer image of the float32 scores finds each expert's
// q_e-th largest key tau_e and how many keys equal to tau_e are still
// needed; ties go to the lower pair index.  Every expert's pairs are cut into
// chunks of 4096, and every pass runs one 256-thread workgroup per chunk:
// three digit passes (each chunk counts its digit in LDS and adds the
// nonzero bins into the expert's histogram in the workspace; the next pass
// finds the digit from it), a count pass (keys above and equal to tau per
// chunk) and a stable scan in pair order (each chunk starts from the counts
// of the expert's earlier chunks) that writes the keep flags and the
// compacted permutation (ascending pair index inside the segment).  One
// workgroup per expert, as an earlier design had it, streams scores it did
// not write at only about 35 GB/s, which made the largest expert the
// critical path.
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

// Non-temporal 16-byte load of a uint4 or float4 chunk (the score pass
// streams every row once).
template <typename V>
__device__ __forceinline__ V ld_stream(const V* __restrict__ p) {
  const uint4 w = load16<true>(reinterpret_cast<const uint4*>(p));
  return __builtin_bit_cast(V, w);
}

// Sum of squares (ABS: of absolute values) of one row held in 16-byte
// chunks, lane-strided, four independent loads in flight per lane.
template <bool ABS = false, typename V>
__device__ __forceinline__ float row_sumsq(const V* __restrict__ row, int nchunk, int lane) {
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  int c = lane;
  for (; c + 192 < nchunk; c += 256) {
    const V x0 = ld_stream(row + c), x1 = ld_stream(row + c + 64), x2 = ld_stream(row + c + 128),
            x3 = ld_stream(row + c + 192);
    a0 += reduce16<ABS>(x0); a1 += reduce16<ABS>(x1);
    a2 += reduce16<ABS>(x2); a3 += reduce16<ABS>(x3);
  }
  if (c < nchunk) {
    V x0, x1, x2;
    const V z = {};   // the lane's last 1..3 chunks at once (zeros past the row end)
    x0 = ld_stream(row + c);
    x1 = c + 64 < nchunk ? ld_stream(row + c + 64) : z;
    x2 = c + 128 < nchunk ? ld_stream(row + c + 128) : z;
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
        const float2 sq =
            pair_sumsq_bf16<true>(grow, gc, gcr > 0, prow, WITH_PHI ? pc : 0, true, lane);
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

// Selection: every expert's pairs are cut into chunks of kSelChunk, one
// 256-thread workgroup per chunk in every pass.
constexpr int kSelT = 256;
constexpr int kSelW = kSelT / 64;
constexpr int kKeysPer = kSelChunk / kSelT;   // 16 keys per thread
constexpr int kB12 = 4096;                    // bins of digits 1 and 2 (12 bits)
constexpr int kB8 = 256;                      // bins of digit 3 (8 bits)
static_assert(kSelChunk % (4 * kSelT) == 0, "chunk shape");

// Selection workspace: per expert the three digit histograms (h1, h2, h3
// contiguous), the state of the radix select st[8e + ...] = {prefix after
// digit 1, its rank, prefix after digit 2, its rank, tau, need}, and two
// counts per chunk (keys above and equal to tau).
struct SelWs {
  uint32_t* h1;        // [E][kB12]
  uint32_t* h2;        // [E][kB12]
  uint32_t* h3;        // [E][kB8]
  uint32_t* st;        // [E][8]
  uint32_t* counts;    // [chunks][2]
};

// Inclusive prefix sum of v over a workgroup of W waves in thread order;
// `total` receives the workgroup sum.  wsum: W LDS words.
template <int W = kSelW>
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
  for (int w = 0; w < W; ++w) {
    const uint32_t sw = wsum[w];
    before += (w < wave) ? sw : 0u;
    t += sw;
  }
  __syncthreads();   // wsum may be reused
  total = t;
  return before + x;
}

// Largest of v over a workgroup of W waves (every thread gets it).
template <int W = kSelW>
__device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  if (lane == 0) wsum[wave] = v;
  __syncthreads();
  uint32_t m = 0u;
#pragma unroll
  for (int w = 0; w < W; ++w) m = max(m, wsum[w]);
  __syncthreads();   // wsum may be reused
  return m;
}

struct Digit {
  uint32_t digit;   // bin holding the k-th largest counted key
  uint32_t k;       // its rank inside that bin (1-based, from the top)
};

// Bin of the k-th largest key of a global histogram of NB bins (1 <= k <=
// the histogram's total).  Thread t owns the NB / kSelT bins just below bin
// NB - (NB / kSelT) t, so the thread-order scan counts from the top bin.
template <int NB>
__device__ __forceinline__ Digit find_digit(const uint32_t* __restrict__ hist, uint32_t k,
                                            uint32_t* wsum, Digit* out) {
  constexpr int PER = NB / kSelT;
  const int tid = threadIdx.x;
  const int top = NB - PER * tid;   // this thread's bins: top-1 .. top-PER
  uint32_t c[PER];
  if constexpr (PER % 4 == 0) {
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
      const u32x4 v = reinterpret_cast<const u32x4*>(hist + top - PER)[q];
      // bins top-PER+4q .. +3 -> c[PER-1-4q] .. c[PER-4-4q]
      c[PER - 1 - 4 * q] = v[0];
      c[PER - 2 - 4 * q] = v[1];
      c[PER - 3 - 4 * q] = v[2];
      c[PER - 4 - 4 * q] = v[3];
    }
  } else {
#pragma unroll
    for (int j = 0; j < PER; ++j) c[j] = hist[top - 1 - j];
  }
  uint32_t local = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) local += c[j];
  if (tid == 0) *out = Digit{0u, 1u};   // stays only if the counts are inconsistent
  uint32_t total;
  const uint32_t incl = block_scan(local, wsum, total);   // its barriers order the write above
  const uint32_t above = incl - local;
  if (local > 0 && above < k && k <= incl) {
    uint32_t cum = above;
    bool found = false;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (!found && cum + c[j] >= k) {
        found = true;
        *out = Digit{(uint32_t)(top - 1 - j), k - cum};
      }
      if (!found) cum += c[j];
    }
  }
  __syncthreads();
  const Digit d = *out;
  __syncthreads();
  return d;
}

// Chunk b -> its expert e and pair range [lo, hi).
struct Chunk {
  int e, lo, hi;
};
__device__ __forceinline__ Chunk chunk_of(const ExpertTable& tab, int b) {
  int e = 0;
  while (e + 1 < tab.E && tab.chunk_off[e + 1] <= b) ++e;
  const int lo = tab.pair_off[e] + (b - tab.chunk_off[e]) * kSelChunk;
  return Chunk{e, lo, min(lo + kSelChunk, tab.pair_off[e + 1])};
}

// The chunk's keys, kKeysPer per thread, thread-strided (key j of thread t is
// pair lo + j kSelT + t); pairs past hi read as 0 and are not valid.
__device__ __forceinline__ void load_keys(const float* __restrict__ scores, const Chunk& ch,
                                          uint32_t (&key)[kKeysPer]) {
  float v[kKeysPer];
#pragma unroll
  for (int j = 0; j < kKeysPer; ++j) {
    const int i = ch.lo + j * kSelT + (int)threadIdx.x;
    v[j] = i < ch.hi ? scores[i] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < kKeysPer; ++j) key[j] = score_key(v[j]);
}
__device__ __forceinline__ bool key_valid(const Chunk& ch, int j) {
  return ch.lo + j * kSelT + (int)threadIdx.x < ch.hi;
}

// Clears the digit histograms, writes seg_offsets and zeroes the expert
// bounds that the scans merge into.
__global__ __launch_bounds__(256) void select_init_kernel(ExpertTable tab, SelWs w,
                                                          int32_t* __restrict__ seg_offsets_out,
                                                          float* __restrict__ ebound) {
  const int n = tab.E * (2 * kB12 + kB8);   // h1, h2, h3 are contiguous
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) w.h1[i] = 0u;
  if (blockIdx.x == 0) {
    for (int e = threadIdx.x; e <= tab.E; e += 256) seg_offsets_out[e] = tab.seg_off[e];
    if (ebound != nullptr)
      for (int i = threadIdx.x; i < 2 * tab.E; i += 256) ebound[i] = 0.f;
  }
}

// Radix pass PASS (1, 2, 3) over one chunk: the histogram of digit PASS
// (key bits 31..20, 19..8, 7..0) of the chunk's keys that carry the prefix
// found so far, counted in LDS and added into the expert's global histogram.
// Passes 2 and 3 first find the previous digit from the previous pass's
// global histogram (every chunk of the expert does, and gets the same; the
// expert's first chunk records it).  Experts that keep nothing are skipped.
template <int PASS>
__global__ __launch_bounds__(kSelT) void select_digit_kernel(ExpertTable tab,
                                                             const float* __restrict__ scores,
                                                             SelWs w) {
  constexpr int NB = PASS == 3 ? kB8 : kB12;
  constexpr int SHIFT = PASS == 1 ? 20 : PASS == 2 ? 8 : 0;
  constexpr uint32_t PMASK = PASS == 1 ? 0u : PASS == 2 ? 0xFFF00000u : 0xFFFFFF00u;
  __shared__ __attribute__((aligned(16))) uint32_t hist[NB];
  __shared__ uint32_t wsum[kSelW];
  __shared__ Digit dig;
  const Chunk ch = chunk_of(tab, blockIdx.x);
  const int e = ch.e;
  const uint32_t q = (uint32_t)(tab.seg_off[e + 1] - tab.seg_off[e]);
  if (q == 0) return;   // workgroup-uniform
  uint32_t key[kKeysPer];
  load_keys(scores, ch, key);   // in flight while the previous digit is found
  const bool first = (int)blockIdx.x == tab.chunk_off[e];
  uint32_t prefix = 0u;
  if (PASS == 2) {
    const Digit d1 = find_digit<kB12>(w.h1 + (size_t)e * kB12, q, wsum, &dig);
    prefix = d1.digit << 20;
    if (first && threadIdx.x == 0) {
      w.st[8 * e + 0] = prefix;
      w.st[8 * e + 1] = d1.k;
    }
  } else if (PASS == 3) {
    const Digit d2 = find_digit<kB12>(w.h2 + (size_t)e * kB12, w.st[8 * e + 1], wsum, &dig);
    prefix = w.st[8 * e + 0] | (d2.digit << 8);
    if (first && threadIdx.x == 0) {
      w.st[8 * e + 2] = prefix;
      w.st[8 * e + 3] = d2.k;
    }
  }
  for (int i = threadIdx.x; i < NB; i += kSelT) hist[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kKeysPer; ++j)
    if (key_valid(ch, j) && (key[j] & PMASK) == prefix)
      atomicAdd(&hist[(key[j] >> SHIFT) & (uint32_t)(NB - 1)], 1u);
  __syncthreads();
  uint32_t* gh = (PASS == 1 ? w.h1 : PASS == 2 ? w.h2 : w.h3) + (size_t)e * NB;
  for (int i = threadIdx.x; i < NB; i += kSelT) {
    const uint32_t c = hist[i];
    if (c != 0u) atomicAdd(gh + i, c);
  }
}

// Last digit -> tau (the q-th largest key) and need (how many keys equal to
// tau are kept: the first `need` of them in pair order); then the chunk's
// counts of keys above and equal to tau.
__global__ __launch_bounds__(kSelT) void select_count_kernel(ExpertTable tab,
                                                             const float* __restrict__ scores,
                                                             SelWs w) {
  __shared__ uint32_t wsum[kSelW];
  __shared__ Digit dig;
  const int b = blockIdx.x;
  const Chunk ch = chunk_of(tab, b);
  const int e = ch.e;
  const uint32_t q = (uint32_t)(tab.seg_off[e + 1] - tab.seg_off[e]);
  const bool first = b == tab.chunk_off[e];
  uint32_t key[kKeysPer];
  load_keys(scores, ch, key);
  uint32_t tau = 0xFFFFFFFFu, need = 0u;   // q == 0: no key is above or equal
  if (q > 0) {
    const Digit d3 = find_digit<kB8>(w.h3 + (size_t)e * kB8, w.st[8 * e + 3], wsum, &dig);
    tau = w.st[8 * e + 2] | d3.digit;
    need = d3.k;
  }
  if (first && threadIdx.x == 0) {
    w.st[8 * e + 4] = tau;
    w.st[8 * e + 5] = need;
  }
  uint32_t ngt = 0, neq = 0;
#pragma unroll
  for (int j = 0; j < kKeysPer; ++j) {
    const bool ok = key_valid(ch, j);
    ngt += ok && key[j] > tau ? 1u : 0u;
    neq += ok && key[j] == tau ? 1u : 0u;
  }
  uint32_t tot;
  block_scan((ngt << 16) | neq, wsum, tot);   // a chunk has < 2^16 keys
  if (threadIdx.x == 0) {
    w.counts[2 * b] = tot >> 16;
    w.counts[2 * b + 1] = tot & 0xFFFFu;
  }
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

// Stable scan of one chunk in pair order: keep = key > tau, or key == tau
// among the first `need` of the expert's equal keys; kept pairs get
// consecutive compacted rows from seg (ascending pair index in the segment).
// The counts of the expert's earlier chunks give the chunk's start.  Thread t
// owns 16 consecutive pairs of a tile that starts at an aligned index (so
// that keep flags go out as whole 4-byte words), and one workgroup scan per
// tile places them; a chunk that starts unaligned takes a second, short
// tile.  In the float16 mode the largest row norms of the kept pairs are
// merged into the expert's bounds.
__global__ __launch_bounds__(kSelT) void select_scan_kernel(
    ExpertTable tab, const float* __restrict__ scores, uint8_t* __restrict__ keep,
    int32_t* __restrict__ perm, SelWs w, const float2* __restrict__ rnorm,
    float* __restrict__ ebound) {
  __shared__ uint32_t wsum[kSelW];
  const int b = blockIdx.x, tid = threadIdx.x;
  const Chunk ch = chunk_of(tab, b);
  const int e = ch.e;
  const int P = tab.pair_off[tab.E];
  const int seg = tab.seg_off[e];
  const uint32_t q = (uint32_t)(tab.seg_off[e + 1] - seg);
  const uint32_t tau = w.st[8 * e + 4], need = w.st[8 * e + 5];
  // keys above / equal to tau in the expert's earlier chunks
  uint32_t pgt = 0, peq = 0;
  for (int c = tab.chunk_off[e] + tid; c < b; c += kSelT) {
    pgt += w.counts[2 * c];
    peq += w.counts[2 * c + 1];
  }
  uint32_t run_gt, run_eq;
  block_scan(pgt, wsum, run_gt);
  block_scan(peq, wsum, run_eq);
  uint32_t kbound[2] = {0u, 0u};
  for (int c = ch.lo & ~3; c < ch.hi; c += kSelChunk) {
    const int g0 = c + tid * kKeysPer;
    const bool full = c + kSelChunk <= P;   // workgroup-uniform: plain vector loads
    uint32_t key[kKeysPer];
#pragma unroll
    for (int h = 0; h < kKeysPer / 4; ++h) {
      const float4 v = full ? *reinterpret_cast<const float4*>(scores + g0 + 4 * h)
                            : load4(scores, g0 + 4 * h, P);
      key[4 * h] = score_key(v.x);
      key[4 * h + 1] = score_key(v.y);
      key[4 * h + 2] = score_key(v.z);
      key[4 * h + 3] = score_key(v.w);
    }
    float2 rn[kKeysPer];
    if (rnorm != nullptr) {
#pragma unroll
      for (int j = 0; j < kKeysPer; ++j) {
        const int g = g0 + j;
        rn[j] = (g >= ch.lo && g < ch.hi) ? rnorm[g] : make_float2(0.f, 0.f);
      }
    }
    uint32_t ngt = 0, neq = 0;
#pragma unroll
    for (int j = 0; j < kKeysPer; ++j) {
      const bool ok = g0 + j >= ch.lo && g0 + j < ch.hi;
      ngt += (ok && key[j] > tau) ? 1u : 0u;
      neq += (ok && key[j] == tau) ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t incl = block_scan((ngt << 16) | neq, wsum, tot);   // per tile < 2^16 each
    const uint32_t excl = incl - ((ngt << 16) | neq);
    uint32_t eq_before = run_eq + (excl & 0xFFFFu);
    // kept keys before this thread: every greater key, and the equal keys
    // among the first `need` equal ones
    uint32_t pos = run_gt + (excl >> 16) + (eq_before < need ? eq_before : need);
    uint32_t kept_bits = 0, valid_bits = 0;
#pragma unroll
    for (int j = 0; j < kKeysPer; ++j) {
      const int g = g0 + j;
      if (g >= ch.lo && g < ch.hi) {
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
    // keep flags: whole 4-byte groups at once when the chunk owns all four
#pragma unroll
    for (int h = 0; h < kKeysPer / 4; ++h) {
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
  }
  if (ebound != nullptr) {   // non-negative float32 bit patterns order like their values
    const uint32_t a = block_max(kbound[0], wsum);
    const uint32_t m = block_max(kbound[1], wsum);
    if (tid == 0) {
      atomicMax(reinterpret_cast<uint32_t*>(ebound) + 2 * e, a);
      atomicMax(reinterpret_cast<uint32_t*>(ebound) + 2 * e + 1, m);
    }
  }
}

// ---- Problems whose experts all have at most kSelLdsKeys pairs: one
// 1024-thread workgroup per expert does the whole selection with the keys in
// LDS, in one launch (the chunked passes above cost about 45 us in six
// launches whatever the size; this takes about 23 us on 32 K-pair problems).
constexpr int kLdsT = 1024;
constexpr int kLdsW = kLdsT / 64;
constexpr int kLdsPer = 8;                 // keys per thread per scan tile
constexpr int kLdsTile = kLdsT * kLdsPer;

// Bin of the k-th largest key of an LDS histogram of nbins <= 4 kLdsT bins:
// thread t owns the 4 bins just below bin nbins - 4 t.
__device__ __forceinline__ Digit find_digit_lds(const uint32_t* hist, int nbins, uint32_t k,
                                                uint32_t* wsum, Digit* out) {
  const int tid = threadIdx.x;
  const int top = nbins - 4 * tid;
  uint32_t c[4] = {0u, 0u, 0u, 0u};
  if (top > 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = hist[top - 1 - j];
  }
  const uint32_t local = c[0] + c[1] + c[2] + c[3];
  if (tid == 0) *out = Digit{0u, 1u};   // stays only if the counts are inconsistent
  uint32_t total;
  const uint32_t incl = block_scan<kLdsW>(local, wsum, total);
  const uint32_t above = incl - local;
  if (local > 0 && above < k && k <= incl) {
    uint32_t cum = above;
    bool found = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (!found && cum + c[j] >= k) {
        found = true;
        *out = Digit{(uint32_t)(top - 1 - j), k - cum};
      }
      if (!found) cum += c[j];
    }
  }
  __syncthreads();
  const Digit d = *out;
  __syncthreads();
  return d;
}

__global__ __launch_bounds__(kLdsT) void select_lds_kernel(
    ExpertTable tab, const float* __restrict__ scores, uint8_t* __restrict__ keep,
    int32_t* __restrict__ perm, int32_t* __restrict__ seg_offsets_out,
    const float2* __restrict__ rnorm, float* __restrict__ ebound) {
  __shared__ uint32_t keys_lds[kSelLdsKeys];
  __shared__ __attribute__((aligned(16))) uint32_t hist[kB12];
  __shared__ uint32_t wsum[kLdsW];
  __shared__ Digit dig;
  const int e = blockIdx.x, tid = threadIdx.x;
  const int P = tab.pair_off[tab.E];
  const int base = tab.pair_off[e], end = tab.pair_off[e + 1];
  const int n = end - base;
  const int gbeg = base & ~3;   // 16-byte aligned start for vector reads
  const int seg = tab.seg_off[e];
  const uint32_t q = (uint32_t)(tab.seg_off[e + 1] - seg);
  if (tid == 0) {
    seg_offsets_out[e] = seg;
    if (e == tab.E - 1) seg_offsets_out[tab.E] = tab.seg_off[tab.E];
    if (ebound != nullptr && n == 0) {   // an empty expert keeps nothing
      ebound[2 * e] = 0.f;
      ebound[2 * e + 1] = 0.f;
    }
  }
  if (n == 0) return;
  for (int a = gbeg + 4 * tid; a < end; a += 4 * kLdsT) {
    const float4 v = load4(scores, a, P);
    const float x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (a + j >= base && a + j < end) keys_lds[a + j - base] = score_key(x[j]);
  }
  __syncthreads();
  // radix select, most significant digit first: 12 + 12 + 8 bits
  uint32_t tau = 0xFFFFFFFFu, need = 0u;   // q == 0: no key is above or equal
  if (q > 0) {
    uint32_t prefix = 0u, k = q;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 20 : pass == 1 ? 8 : 0;
      const int nb = pass == 2 ? kB8 : kB12;
      const uint32_t pmask = pass == 0 ? 0u : pass == 1 ? 0xFFF00000u : 0xFFFFFF00u;
      for (int i = tid; i < nb; i += kLdsT) hist[i] = 0u;
      __syncthreads();
      for (int i = tid; i < n; i += kLdsT) {
        const uint32_t key = keys_lds[i];
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & (uint32_t)(nb - 1)], 1u);
      }
      __syncthreads();
      const Digit d = find_digit_lds(hist, nb, k, wsum, &dig);
      prefix |= d.digit << shift;
      k = d.k;
    }
    tau = prefix;
    need = k;
  }
  // stable scan in pair order, 8 consecutive keys per thread, one workgroup
  // scan per 8192 keys
  uint32_t run_gt = 0, run_eq = 0;
  uint32_t kbound[2] = {0u, 0u};
  for (int c = gbeg; c < end; c += kLdsTile) {
    const int g0 = c + tid * kLdsPer;
    uint32_t key[kLdsPer];
    float2 rn[kLdsPer];
#pragma unroll
    for (int j = 0; j < kLdsPer; ++j) {
      const int g = g0 + j;
      const bool ok = g >= base && g < end;
      key[j] = ok ? keys_lds[g - base] : 0u;
      if (rnorm != nullptr) rn[j] = ok ? rnorm[g] : make_float2(0.f, 0.f);
    }
    uint32_t ngt = 0, neq = 0;
#pragma unroll
    for (int j = 0; j < kLdsPer; ++j) {
      const bool ok = g0 + j >= base && g0 + j < end;
      ngt += (ok && key[j] > tau) ? 1u : 0u;
      neq += (ok && key[j] == tau) ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t incl = block_scan<kLdsW>((ngt << 16) | neq, wsum, tot);   // < 2^16 each
    const uint32_t excl = incl - ((ngt << 16) | neq);
    uint32_t eq_before = run_eq + (excl & 0xFFFFu);
    uint32_t pos = run_gt + (excl >> 16) + (eq_before < need ? eq_before : need);
    uint32_t kept_bits = 0, valid_bits = 0;
#pragma unroll
    for (int j = 0; j < kLdsPer; ++j) {
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
#pragma unroll
    for (int h = 0; h < kLdsPer / 4; ++h) {
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
  }
  if (ebound != nullptr) {
    const uint32_t a = block_max<kLdsW>(kbound[0], wsum);
    const uint32_t m = block_max<kLdsW>(kbound[1], wsum);
    if (tid == 0) {
      ebound[2 * e] = __uint_as_float(a);
      ebound[2 * e + 1] = __uint_as_float(m);
    }
  }
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
  // One pair per wave: the dispatcher hands out fresh workgroups as others
  // finish, which balances CUs and memory channels better than waves that
  // loop over many pairs (655 360-pair workload: 1214 us, against 1274 us
  // with 64 workgroups per CU looping and 1330 us with 16).  Beyond 4 M
  // pairs the waves loop (grid-stride).
  if (blocks > 256 * 4096) blocks = 256 * 4096;
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

// The chunked passes serve problems with an expert above kSelLdsKeys pairs;
// the others take the one-launch LDS path, which needs no workspace.
static bool select_chunked(const ExpertTable& tab) {
  for (int e = 0; e < tab.E; ++e)
    if (tab.pair_off[e + 1] - tab.pair_off[e] > kSelLdsKeys) return true;
  return false;
}

size_t select_workspace_bytes(const ExpertTable& tab) {
  if (!select_chunked(tab)) return 0;
  return ((size_t)tab.E * (2 * kB12 + kB8 + 8) + 2 * (size_t)tab.chunk_off[tab.E]) *
         sizeof(uint32_t);
}

hipError_t launch_select(const ExpertTable& tab, const float* scores, uint8_t* keep,
                         int32_t* perm, int32_t* seg_offsets_out, uint32_t* ws, hipStream_t s,
                         const float2* rnorm, float* ebound) {
  if (!select_chunked(tab)) {
    hipLaunchKernelGGL(select_lds_kernel, dim3(tab.E), dim3(kLdsT), 0, s, tab, scores, keep,
                       perm, seg_offsets_out, rnorm, ebound);
    return hipGetLastError();
  }
  SelWs w;
  w.h1 = ws;
  w.h2 = w.h1 + (size_t)tab.E * kB12;
  w.h3 = w.h2 + (size_t)tab.E * kB12;
  w.st = w.h3 + (size_t)tab.E * kB8;
  w.counts = w.st + 8 * (size_t)tab.E;
  const int chunks = tab.chunk_off[tab.E];
  const int init_words = tab.E * (2 * kB12 + kB8);
  int init_blocks = (init_words + 4 * 256 - 1) / (4 * 256);
  if (init_blocks < 1) init_blocks = 1;
  hipLaunchKernelGGL(select_init_kernel, dim3(init_blocks), dim3(256), 0, s, tab, w,
                     seg_offsets_out, ebound);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || chunks == 0) return err;
  hipLaunchKernelGGL(select_digit_kernel<1>, dim3(chunks), dim3(kSelT), 0, s, tab, scores, w);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(select_digit_kernel<2>, dim3(chunks), dim3(kSelT), 0, s, tab, scores, w);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(select_digit_kernel<3>, dim3(chunks), dim3(kSelT), 0, s, tab, scores, w);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(select_count_kernel, dim3(chunks), dim3(kSelT), 0, s, tab, scores, w);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(select_scan_kernel, dim3(chunks), dim3(kSelT), 0, s, tab, scores, keep,
                     perm, w, rnorm, ebound);
  return hipGetLastError();
}

}  // namespace lrmoe
