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
//   * 256-thread workgroups (4 wave64s, 2 x 2, one per SIMD) own a 256x256
//     fp32 tile; each wave accumulates 128x128 in its 256 accumulation
//     registers with v_mfma_f32_32x32x16_bf16 (fp32 accumulate).  Large wave
//     tiles keep LDS bytes per MFMA low (the LDS, not the matrix cores, bounds
//     a 128x64 wave tile).  With one wave per SIMD the K loop is software
//     pipelined by hand: fragments are double-buffered in registers by half
//     K step, and LDS reads and global->LDS loads are placed between MFMAs
//     (see Tile).  Accumulators hold each 32x32 block transposed (lane = row,
//     register quad = 4 consecutive columns), so results leave as 16-byte
//     stores; adjacent lanes swap one quad each first, so that every store
//     instruction writes 64-byte row pieces from adjacent lane pairs.
//   * Every operand is a bf16 plane in global memory.  alpha multiplies the
//     reduction index of dW, so it cannot be applied after the product: a
//     prologue writes alpha * (the narrower of g_c, phi_c) as bf16 hi + lo
//     planes (exact mode; hi only in single-rounding mode), and float32
//     storage is pre-split into hi + lo planes.  Products of split operands
//     sum hi*hi + hi*lo + lo*hi.  In the float16 weight-gradient mode the
//     operand with alpha is a scaled float16 plane, and the other one either
//     a plane too or (narrow problems) its bf16 rows, converted to scaled
//     float16 in registers inside the MFMA loop; no other mode converts.
//   * Operand tiles of one K step (32) live in LDS in the global layout:
//     "KC" tiles (rows along M/N, K contiguous: g_c rows of the input
//     gradient) are read with 16-byte ds_read_b128 fragments; "MC" tiles
//     (rows along K, M/N contiguous: both operands of the weight gradient, W
//     of the input gradient) are read with ds_read_b64_tr_b16, which
//     transposes 4x16 bf16 blocks across each 16-lane group, so no operand is
//     ever transposed in memory.  16-byte chunks are XOR-swizzled per row so
//     that fragment reads spread over the LDS banks.
//   * Operands move global -> LDS with buffer_load_dwordx4 ... lds (no
//     register staging): each wave instruction fills one 1 KiB LDS block, lane
//     i writing bytes 16i..16i+15, so each lane fetches the global chunk that
//     the swizzled layout puts in its slot; lanes past a row or column edge
//     get an out-of-range offset and write zeros.  Each tile kind gets as
//     many LDS stages as fit in 144 KiB, up to four: two planes (dphi, and dW
//     in single-rounding mode) -> 4 stages; three planes (dW with a hi + lo
//     operand) -> 3; four (float32 storage) -> 2.  Each K step crosses one
//     barrier, between its two halves.
//   * Scheduling: dW and dphi tiles share one persistent launch, one
//     workgroup per CU.  Tiles are grouped in blocks of an expert's tile grid
//     that share operand panels.  The host deals the groups, longest first,
//     to the XCD with the least work so far; workgroup b runs on XCD b % 8
//     (dispatch is round-robin over the 8 XCDs) and drains that XCD's queue
//     through an atomic counter, so a group's panels are fetched into one L2.
//     A workgroup whose queue is empty takes tiles from the other XCDs'
//     queues.  An expert whose kept rows exceed one K chunk has its dW split
//     along K: each chunk writes an fp32 partial tile and a second kernel
//     sums them in chunk order, so the result does not depend on timing.
//   * SiLU-GLU variant (GLU = 1: bf16 output, 2: float32 output): the
//     input-gradient tiles write the gate/up output gradient of the expert
//     MLP, compacted, instead of dphi (see Tile::glu_epilogue).
//   * The gate/up projection behind it reads that gradient as float32: a
//     prologue splits alpha * g_c into bf16 hi + lo planes that feed both
//     products (PA = 2 for the input gradient too), and the input-gradient
//     epilogue then applies no alpha (dp_alpha_folded).
#include "lrmoe_internal.h"

namespace lrmoe {
namespace {

#define LDS_AS __attribute__((address_space(3)))

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = kTile, BN = kTile, BK = 32;
// Four waves per tile, each computing a 128 x 128 block (one wave per SIMD,
// 256 accumulators each).  A square tile stacks them 2 x 2; the tall edge
// tile (512 x 128, for a last column that holds at most 128 columns) stacks
// them 4 x 1.  2 x 4 waves of 128 x 64 (two waves per SIMD) were measured as
// well: correct, and no faster (the second wave hides no more than the extra
// fragment reads cost).
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int WTM = 128;                   // rows of one wave's block
constexpr int WTN = 128;                   // columns of one wave's block
constexpr int kMB = WTM / 32;              // 32x32 accumulator blocks per wave: kMB x kNB
constexpr int kNB = WTN / 32;
constexpr int kPlaneBytes = kTile * BK * 2;   // one bf16 operand plane of one K step (16 KB)

// ------------------------------------------------------------ LDS layouts
// KC: row r (0..255) holds K 0..31 as 4 chunks of 16 B; chunk c of row r
// sits at slot c ^ kc_swz(r).  A fragment read (ds_read_b128) serves 16
// consecutive lanes = 16 consecutive rows per LDS cycle; this swizzle gives
// them 16 distinct 16-byte bank slots (measured on gfx950: twice the read
// rate of the ((r >> 1) ^ (r >> 3)) & 3 variant, and the same rate as a
// linear b128 read).
__device__ __forceinline__ int kc_swz(int r) { return (r ^ (r >> 2)) & 3; }
__device__ __forceinline__ int kc_off(int r, int c) { return r * 64 + ((c ^ kc_swz(r)) << 4); }
// MC: row k (0..31) holds the tile's M or N extent (128, 256 or 512) as
// RB / 16 chunks of 16 B, RB bytes per row.  The swizzle moves rows k and
// k + 1 .. k + 3 by 4 chunks each; every row width is a multiple of 256 B,
// so all widths see the same bank pattern.
template <int RB>
__device__ __forceinline__ int mc_off(int k, int c) { return k * RB + ((c ^ ((k & 3) << 2)) << 4); }

// Fragments (8 bf16 per lane), read at precomputed LDS byte addresses (the
// tile's la / lb).
//   KC: lane l holds MN index mb + l%32 and K = kb + 8*(l/32) + 0..7: one
//       16-byte read at kc_off(mb + l%32, kb/8 + l/32).
//   MC: ds_read_b64_tr_b16 -- within each 16-lane group G = l/16, source lane
//       s = l%16 reads 4 bf16 of row k0 = kb + 8*(G/2) + s/4 at chunk
//       mb/8 + 2*(G%2) + (s%4)/2, half (s%2)*8 bytes; after the transpose lane
//       l holds one MN column for rows k0 .. k0 + 3.  Two such reads 4 rows
//       (4 * RB bytes) apart give the 8 K values.
template <int RB>
__device__ __forceinline__ i16x8 frag_mc_at(uint32_t addr) {
  LDS_AS char* p = (LDS_AS char*)(uintptr_t)addr;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<LDS_AS i16x4*>(p));
  const i16x4 hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<LDS_AS i16x4*>(p + 4 * RB));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ i16x8 frag_kc_at(uint32_t addr) {
  return *reinterpret_cast<LDS_AS const i16x8*>((LDS_AS char*)(uintptr_t)addr);
}

__device__ __forceinline__ f32x16 mfma(i16x8 a, i16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
// float16 operands (the float16 weight-gradient mode): same shape and rate
__device__ __forceinline__ f32x16 mfma_f16(i16x8 a, i16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

struct TileJob {
  int e, m0, n0;
  int chunk, chunks;   // dW K chunk of this tile and the expert's chunk count
  bool tall;           // 512 x 128 edge tile over row tiles m0 / 256 and m0 / 256 + 1
  bool half;           // 256 x 128 weight-gradient edge tile (waves of 128 x 64)
};

// Queue length of XCD x in item slots.
__device__ __forceinline__ int queue_items(const GemmTable& tab, int x) {
  if (tab.use_table) return (tab.qoff[x + 1] - tab.qoff[x]) * kGroupSlots;
  const int ng = tab.total_groups > x ? (tab.total_groups - 1 - x) / kXcds + 1 : 0;
  return ng * kGroupSlots;
}

// Item `i` of XCD x's queue -> tile; false for an idle slot.  With `tall`,
// the last input-gradient column tile (and with `tall_dw` the last
// weight-gradient one) of every even row tile becomes a 512 x 128 tile that
// also covers the odd row tile below it, whose slot then idles.  With
// `half_dw` the last weight-gradient column tile is a 256 x 128 tile.
__device__ __forceinline__ bool decode(const GemmTable& tab, int x, int i, bool& is_dw,
                                      TileJob& job, bool tall, bool tall_dw, bool half_dw) {
  const int p = i / kGroupSlots, t = i % kGroupSlots;
  int e, chunk, lg;
  if (tab.use_table) {
    const uint32_t d = tab.groups[tab.qoff[x] + p];
    is_dw = (d >> 31) != 0;
    e = (int)((d >> 23) & 0xFF);
    chunk = (int)((d >> 15) & 0xFF);
    lg = (int)(d & 0x7FFF);
  } else {
    const int g = p * kXcds + x;   // global group order: dW (LPT) then dphi
    is_dw = g < tab.dw_groups;
    const int32_t* goff = is_dw ? tab.f.dw_goff : tab.f.dp_goff;
    int lo = 0, hi = tab.E - 1;   // last rank r with goff[r] <= g
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (goff[mid] <= g) lo = mid; else hi = mid - 1;
    }
    e = is_dw ? (int)tab.f.order[lo] : lo;
    lg = g - goff[lo];
    chunk = 0;
  }
  const int gm = is_dw ? tab.dw_gm : tab.dp_gm;
  const int gn = is_dw ? tab.dw_gn : tab.dp_gn;
  if (t >= gm * gn) return false;
  const int ngn = (tab.tiles_n + gn - 1) / gn;
  const int q = tab.seg_off[e + 1] - tab.seg_off[e];
  int chunks = 1;
  if (is_dw) {
    chunks = dw_chunks(q, tab.kc);
    if (!tab.use_table) {   // formula order: the expert's groups are chunk-major
      const int per_chunk = ((tab.dw_tiles_m + gm - 1) / gm) * ngn;
      chunk = lg / per_chunk;
      lg -= chunk * per_chunk;
    }
  }
  const int tm = (lg / ngn) * gm + t / gn;
  const int tn = (lg % ngn) * gn + t % gn;
  const int tiles_m = is_dw ? tab.dw_tiles_m : (q + BM - 1) / BM;
  if (tm >= tiles_m || tn >= tab.tiles_n) return false;
  job.tall = tall && (!is_dw || tall_dw) && tn == tab.tiles_n - 1;
  job.half = half_dw && is_dw && tab.tall != 0 && tn == tab.tiles_n - 1;
  if (job.tall && (tm & 1)) return false;
  job.e = e;
  job.m0 = tm * BM;
  job.n0 = tn * BN;
  job.chunk = chunk;
  job.chunks = chunks;
  return true;
}

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

// global -> LDS copy of 16 bytes per lane: lane i writes LDS bytes
// [lds + 16i, lds + 16i + 16).  Issued as inline asm so that the compiler
// does not treat later LDS reads of other stages as waiting on it; the
// explicit wait + barrier below orders every stage.  M0 is not used by the
// compiler anywhere in these kernels.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds), "v"(voff),
               "s"(r)
               : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t lds_addr(LDS_AS const char* p) {
  return (uint32_t)(uintptr_t)p;
}

// Workgroup barrier that waits for this wave's LDS accesses only (not for
// global loads or stores still in flight).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most N of this wave's loads are outstanding, then cross the
// workgroup barrier.  One asm block, so that the compiler adds no wait of its
// own for the loads still in flight into other LDS stages.
template <int N>
__device__ __forceinline__ void wait_loads_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// dphi epilogue: destination row + alpha of each of the (at most 512) tile rows
constexpr int kMaxRows = 2 * kTile;
constexpr int kPermBytes = kMaxRows * 8;

// Everything one tile needs, derived from its job.  IS_DW: A (MC, rows = K)
// and B (MC, rows = K) are [M, d_out] / [M, d_in] segment rows.  Else A (KC,
// rows = M) = g_c segment rows and B (MC) = W_e.  PA/PB: bf16 planes of each
// operand; NS: LDS stages.
//
// Software pipeline of one K step kt (stage S = kt % NS), per wave:
//   phase 1  MFMAs of half 0 (registers f0), interleaved with the LDS reads
//            of half 1 of stage S into f1;
//   barrier  wait for this wave's loads of stage kt + 1 and its LDS reads,
//            then s_barrier: stage kt + 1 is in LDS and nobody reads stage S
//            any more;
//   phase 3  MFMAs of half 1 (f1), interleaved with the LDS reads of half 0
//            of stage kt + 1 into f0 and with this wave's loads of stage
//            kt + NS into buffer S.
// The matrix core always has independent MFMAs queued while fragments and
// stages move, and the global loads trickle out between MFMAs instead of
// stalling the wave in a burst.
// F16 (weight-gradient tiles only): float16 MFMAs, and the epilogue undoes
// the expert's power-of-two scales.  The operand that carries alpha comes as
// a scaled float16 plane.  The other one is a scaled float16 plane too
// (F16 == 3), or the compacted bf16 buffer itself, converted in registers
// after its LDS fragment reads (A for F16 == 1, B for F16 == 2; see
// cvt_slot).
// TALL: a 512 x 128 tile (waves stacked 4 x 1) instead of 256 x 256.
template <bool IS_DW, int PA, int PB, int NS, int GLU = 0, int F16 = 0, bool TALL = false,
          bool HALF = false>
struct Tile {
  static constexpr bool A_MC = IS_DW;
  static constexpr int TBM = TALL ? 2 * kTile : kTile;   // tile rows (M)
  static constexpr int TBN = TALL || HALF ? kTile / 2 : kTile;   // tile columns (N)
  static constexpr int WN = HALF ? WTN / 2 : WTN;       // columns of one wave's block
  static constexpr int NB = WN / 32;                    // its 32-column accumulator blocks
  static constexpr int kWN = TBN / WN;                  // wave columns (1 or 2)
  static_assert((TBM / WTM) * kWN == kWaves, "wave grid");
  // One K step of an operand plane: TBM (A) or TBN (B) values per K row.
  // MC rows are RA / RB bytes long (RA: weight-gradient tiles, 256 or 512
  // wide); KC rows are 64 bytes.
  static constexpr int RA = 2 * TBM, RB = 2 * TBN;
  static constexpr int kPlaneA = TBM * BK * 2, kPlaneB = TBN * BK * 2;
  static constexpr int kStage = PA * kPlaneA + PB * kPlaneB;
  // 1 KiB LDS blocks of one plane filled by each wave
  static constexpr int kPwA = kPlaneA / 1024 / kWaves, kPwB = kPlaneB / 1024 / kWaves;
  static constexpr int kLoads = PA * kPwA + PB * kPwB;   // load instructions per stage per wave
  static constexpr int kTerms = 1 + (PA == 2) + (PB == 2);
  static constexpr int kHalfMfmas = kMB * NB * kTerms; // per wave per half step
  static constexpr int kFrags = PA * kMB + PB * NB;     // fragments per half step
  static_assert(kFrags <= kHalfMfmas && kLoads <= kHalfMfmas, "interleave slots");
  // float16 mode: one term, and a converted fragment's 4 dwords spread over
  // the 4 MFMAs of the fragment before it
  static constexpr bool kCvt = IS_DW && (F16 == 1 || F16 == 2);
  static_assert(!kCvt || (kTerms == 1 && kMB == 4 && NB == 4), "float16 slots");

  struct Frags {
    i16x8 a[PA][kMB];
    i16x8 b[PB][NB];
  };

  int e, m0, n0, chunk, chunks, q, seg, K, mrows, nk;
  int lane, wave, wm, wn;
  int cvs;   // float16 mode: power of two applied to the converted operand
  const uint16_t* A[2];
  const uint16_t* B[2];
  uint32_t aoff[kPwA], boff[kPwB];
  int acol[kPwA];
  // LDS byte addresses of this lane's fragment reads in stage 0, plane 0:
  // MC operands: one per 32-wide fragment (half 0; half 1 is 16 rows on);
  // KC operand: one per half (fragment a is +2 KiB * a).
  uint32_t la[kMB], lb[NB];
  LDS_AS char* sink;   // kWaves x 1 KiB of LDS that only dead loads write

  __device__ __forceinline__ Tile(const Args& args, const GemmTable& tab, const TileJob& job,
                                  LDS_AS char* smem, LDS_AS char* sink_) : sink(sink_) {
    const int tid = threadIdx.x;
    lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    wm = wave / kWN;   // wave block rows wm*WTM, columns wn*WN
    wn = wave % kWN;
    // Tile coordinates are workgroup-uniform; say so, so that buffer
    // descriptors and LDS bases stay in scalar registers.
    e = __builtin_amdgcn_readfirstlane(job.e);
    m0 = __builtin_amdgcn_readfirstlane(job.m0);
    n0 = __builtin_amdgcn_readfirstlane(job.n0);
    chunk = __builtin_amdgcn_readfirstlane(job.chunk);
    chunks = __builtin_amdgcn_readfirstlane(job.chunks);
    const int d_out = args.d_out, d_in = args.d_in;
    q = tab.seg_off[e + 1] - tab.seg_off[e];
    // dW: this chunk's rows of the segment; dphi: the whole segment (M) and d_out (K)
    const int kbeg = IS_DW ? chunk * tab.kc : 0;
    seg = tab.seg_off[e] + kbeg;
    K = IS_DW ? (q - kbeg < tab.kc ? q - kbeg : tab.kc) : d_out;
    mrows = IS_DW ? d_out : q;
    nk = (K + BK - 1) / BK;
    cvs = 0;
    if constexpr (kCvt)
      cvs = __builtin_amdgcn_readfirstlane(f16_scale_exp(args.ops.dw_ebound[2 * e + (F16 == 2)]));
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      A[p] = IS_DW ? args.ops.dw_a[p] : args.ops.dp_a[p];
      B[p] = IS_DW ? args.ops.dw_b[p] : args.ops.dp_b[p];
    }
    // Byte offsets (within one K step) of the global chunk each lane fetches
    // for each of its LDS blocks: block wave*kPwA + j of an A plane, wave*kPwB
    // + j of a B plane.  An MC block holds 1024 / RB K rows of RB / 16 chunks
    // (lane -> row lane / (RB/16), physical chunk lane % (RB/16)).
#pragma unroll
    for (int j = 0; j < kPwB; ++j) {
      constexpr int cpr = RB / 16;
      const int k = (64 / cpr) * (wave * kPwB + j) + lane / cpr, pc = lane % cpr;
      const int col = n0 + 8 * (pc ^ ((k & 3) << 2));
      boff[j] = col < d_in ? (uint32_t)(k * d_in + col) * 2u : kOutOfRange;
    }
#pragma unroll
    for (int j = 0; j < kPwA; ++j) {
      const int blk = wave * kPwA + j;
      if (A_MC) {   // MC block: 1024 / RA K rows of RA / 16 chunks each
        constexpr int cpr = RA / 16;
        const int k = (64 / cpr) * blk + lane / cpr, pc = lane % cpr;
        const int acolm = m0 + 8 * (pc ^ ((k & 3) << 2));
        aoff[j] = acolm < d_out ? (uint32_t)(k * d_out + acolm) * 2u : kOutOfRange;
      } else {   // KC block: rows 16*blk .. +15 of the tile, 4 chunks each
        const int r = 16 * blk + (lane >> 2), pc = lane & 3;
        const int lc = pc ^ kc_swz(r);
        acol[j] = 8 * lc;
        aoff[j] = (uint32_t)(r * d_out + 8 * lc) * 2u;
      }
    }
    // Fragment addresses (lane layouts: see the fragment reads above).
    const uint32_t base = lds_addr(smem);
    {
      const int G = lane >> 4, s = lane & 15;
      const int k0 = 8 * (G >> 1) + (s >> 2);
      const int cl = 2 * (G & 1) + ((s & 3) >> 1);
      const int half = (s & 1) * 8;
#pragma unroll
      for (int f = 0; f < NB; ++f)
        lb[f] = base + (uint32_t)(mc_off<RB>(k0, (wn * WN + f * 32) / 8 + cl) + half);
      if (A_MC) {
#pragma unroll
        for (int f = 0; f < kMB; ++f)
          la[f] = base + (uint32_t)(mc_off<RA>(k0, (wm * WTM + f * 32) / 8 + cl) + half);
      }
    }
    if (!A_MC) {
      const int r = wm * WTM + (lane & 31);
#pragma unroll
      for (int h = 0; h < 2; ++h) la[h] = base + (uint32_t)kc_off(r, 2 * h + (lane >> 5));
#pragma unroll
      for (int h = 2; h < kMB; ++h) la[h] = 0;
    }
  }

  // ---- global -> LDS: load instruction `idx` (0 .. kLoads-1) of this wave
  // for the K step starting at k0.  Instructions 0 .. PA*kPwA-1 fill block
  // wave * kPwA + idx % kPwA of A plane idx / kPwA; the rest fill the B
  // planes the same way.  When !live the instruction keeps its place in the
  // stream but reads an empty range and writes only zeros, into this wave's
  // sink block.
  __device__ __forceinline__ void issue_one(const Args& args, int k0, LDS_AS char* stage,
                                            int idx, bool live = true) const {
    const int d_out = args.d_out, d_in = args.d_in;
    const int krows = live ? (K - k0 < BK ? K - k0 : BK) : 0;
    if (idx < PA * kPwA) {
      const int p = idx / kPwA, j = idx % kPwA;
      LDS_AS char* dst = live ? stage + p * kPlaneA + (wave * kPwA + j) * 1024 : sink + wave * 1024;
      __amdgpu_buffer_rsrc_t r =
          A_MC ? rsrc(A[p] + ((int64_t)seg + k0) * d_out, (int64_t)krows * d_out * 2)
               : rsrc(A[p] + ((int64_t)seg + m0) * d_out,
                      live ? (int64_t)(q - m0) * d_out * 2 : 0);
      uint32_t off = aoff[j];
      if (!A_MC) off = (k0 + acol[j]) < K ? off + (uint32_t)k0 * 2u : kOutOfRange;
      load_lds16(r, lds_addr(dst), off);
    } else {
      const int p = (idx - PA * kPwA) / kPwB, j = (idx - PA * kPwA) % kPwB;
      LDS_AS char* dst = live ? stage + PA * kPlaneA + p * kPlaneB + (wave * kPwB + j) * 1024
                              : sink + wave * 1024;
      const uint16_t* b0 = IS_DW ? B[p] + ((int64_t)seg + k0) * d_in
                                 : B[p] + ((int64_t)e * d_out + k0) * d_in;
      load_lds16(rsrc(b0, (int64_t)krows * d_in * 2), lds_addr(dst), boff[j]);
    }
  }

  // First min(NS, nk) stages.
  __device__ __forceinline__ void prologue(const Args& args, LDS_AS char* smem) const {
#pragma unroll
    for (int d = 0; d < NS; ++d)
      if (d < nk) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) issue_one(args, d * BK, smem + d * kStage, i);
      }
  }

  // ---- fragment i (0 .. kFrags-1) of half h of stage s: A fragments first.
  __device__ __forceinline__ void read_frag(int s, int h, Frags& f, int i) const {
    const uint32_t so = (uint32_t)(s * kStage);
    if (i < PA * kMB) {
      const int p = i / kMB, a = i % kMB;
      const uint32_t po = so + (uint32_t)(p * kPlaneA);
      if (A_MC) f.a[p][a] = frag_mc_at<RA>(la[a] + po + (uint32_t)(h * 16 * RA));
      else f.a[p][a] = frag_kc_at(la[h] + po + (uint32_t)(a * 2048));
    } else {
      const int p = (i - PA * kMB) / NB, b = (i - PA * kMB) % NB;
      f.b[p][b] =
          frag_mc_at<RB>(lb[b] + so + (uint32_t)(PA * kPlaneA + p * kPlaneB + h * 16 * RB));
    }
  }

  // ---- MFMA i (0 .. kHalfMfmas-1) of a half: terms hi*hi, hi*lo_B, lo_A*hi.
  // The B fragment goes in the MFMA's first operand slot, so each 32x32
  // accumulator holds the block transposed: lane = tile row (M), registers =
  // columns (N), four consecutive columns per register quad.  That lets the
  // epilogue write 16 bytes per lane.  Within a term the MFMAs run A fragment
  // by A fragment, or (F16 == 2) B fragment by B fragment: the converted
  // operand's fragments are used one after the other.
  __device__ __forceinline__ static void mfma_i(const Frags& f, f32x16 (&acc)[kMB][kNB], int i) {
    const int t = i / (kMB * NB), r = i % (kMB * NB);
    const int a = (IS_DW && F16 == 2) ? r % kMB : r / NB;
    const int b = (IS_DW && F16 == 2) ? r / kMB : r % NB;
    const int pa = (t == 2 || (t == 1 && PB == 1)) ? PA - 1 : 0;
    const int pb = (t == 1 && PB == 2) ? 1 : 0;
    if constexpr (IS_DW && F16) acc[a][b] = mfma_f16(f.b[pb][b], f.a[pa][a], acc[a][b]);
    else acc[a][b] = mfma(f.b[pb][b], f.a[pa][a], acc[a][b]);
  }

  // ---- float16 mode: bf16 -> float16 of 2^cvs * x, in place, for the two
  // values of dword p of fragment x (the power of two is exact; one rounding
  // to nearest even, the same as the scaled float16 planes get).
  __device__ __forceinline__ void cvt_piece(i16x8& x, int p) const {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    u32x4 w = __builtin_bit_cast(u32x4, x);
    const uint32_t d = w[p];
    const float lo = __builtin_amdgcn_ldexpf(__uint_as_float(d << 16), cvs);
    const float hi = __builtin_amdgcn_ldexpf(__uint_as_float(d & 0xFFFF0000u), cvs);
    const f16x2 h = {(_Float16)lo, (_Float16)hi};
    w[p] = __builtin_bit_cast(uint32_t, h);
    x = __builtin_bit_cast(i16x8, w);
  }
  // Conversion work of MFMA slot i of a half that multiplies fragments F
  // while G (the next half) is read: dword i % 4 of the converted operand's
  // next fragment of F, and in the last 4 slots of G's first fragment (its
  // LDS reads went out in the first half of the slots).  So every fragment is
  // converted over the 4 MFMAs before its first use, 5 VALU instructions per
  // 32-cycle MFMA.
  __device__ __forceinline__ void cvt_slot(Frags& F, Frags& G, int i) const {
    if constexpr (kCvt) {
      const int grp = i / 4, p = i % 4;
      if constexpr (F16 == 1) cvt_piece(grp + 1 < kMB ? F.a[0][grp + 1] : G.a[0][0], p);
      else cvt_piece(grp + 1 < NB ? F.b[0][grp + 1] : G.b[0][0], p);
    }
  }
  // The first fragment of a freshly read set, all at once (tile start).
  __device__ __forceinline__ void cvt_first(Frags& F) const {
    if constexpr (kCvt) {
#pragma unroll
      for (int p = 0; p < 4; ++p) cvt_piece(F16 == 1 ? F.a[0][0] : F.b[0][0], p);
    }
  }

  // Barrier of step kt: stage kt + 1 is complete for every wave.  Stages
  // kt + 1 .. last are this wave's outstanding loads (in issue order).
  __device__ __forceinline__ static void wait_next(int later) {
    if (later >= 2) wait_loads_barrier<2 * kLoads>();
    else if (later == 1) wait_loads_barrier<kLoads>();
    else wait_loads_barrier<0>();
  }

  // This wave's loads of one stage are split in two halves: the first half
  // of stage kt + NS goes out during phase 3 of step kt (into buffer S, free
  // after that step's barrier), the second half during phase 1 of step
  // kt + 1 (same buffer).  Both halves are spread evenly over the MFMAs.
  static constexpr int kLoadsLo = kLoads / 2;
  static constexpr int kLoadsHi = kLoads - kLoadsLo;
  // n loads over kHalfMfmas slots: load d goes after MFMA (d * kHalfMfmas) / n.
  // Index of the load after MFMA i, or -1.
  __device__ __forceinline__ static constexpr int load_at(int i, int n) {
    for (int d = 0; d < n; ++d)
      if ((d * kHalfMfmas) / n == i) return d;
    return -1;
  }

  __device__ __forceinline__ void step(const Args& args, LDS_AS char* smem, int kt, Frags& f0,
                                       Frags& f1, f32x16 (&acc)[kMB][kNB]) const {
    const int S = kt % NS, SN = S + 1 == NS ? 0 : S + 1, SP = S == 0 ? NS - 1 : S - 1;
    // phase 1: second half of stage kt + NS - 1 (buffer SP); the prologue
    // already issued it when kt == 0
    const bool live1 = kt >= 1 && kt + NS - 1 < nk;
#pragma unroll
    for (int i = 0; i < kHalfMfmas; ++i) {
      mfma_i(f0, acc, i);
      if (i < kFrags) read_frag(S, 1, f1, i);
      cvt_slot(f0, f1, i);
      if (load_at(i, kLoadsHi) >= 0)
        issue_one(args, (kt + NS - 1) * BK, smem + SP * kStage, kLoadsLo + load_at(i, kLoadsHi),
                  live1);
      __builtin_amdgcn_sched_barrier(0);
    }
    const bool next = kt + 1 < nk;
    if (next) {
      const int last = kt + NS - 1 < nk - 1 ? kt + NS - 1 : nk - 1;   // last stage issued
      wait_next(last - (kt + 1));
    }
    __builtin_amdgcn_sched_barrier(0);
    // phase 3: first half of stage kt + NS (buffer S).  Branch-free: past the
    // last step the reads fetch unused data and the loads (with an empty
    // range) only write zeros into this wave's sink block, so every step runs
    // the same instruction stream.
    const bool live3 = kt + NS < nk;
#pragma unroll
    for (int i = 0; i < kHalfMfmas; ++i) {
      mfma_i(f1, acc, i);
      if (i < kFrags) read_frag(SN, 0, f0, i);
      cvt_slot(f1, f0, i);
      if (load_at(i, kLoadsLo) >= 0)
        issue_one(args, (kt + NS) * BK, smem + S * kStage, load_at(i, kLoadsLo), live3);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- K loop.  The prologue issued stages 0 .. min(NS, nk) - 1.  Ends with
  // every load of the tile consumed; LDS reads of the last stage may still be
  // in flight (the caller's barrier covers them).
  __device__ __forceinline__ void mainloop(const Args& args, LDS_AS char* smem,
                                           f32x16 (&acc)[kMB][kNB]) const {
#pragma unroll
    for (int a = 0; a < kMB; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
    if (nk == 0) return;
    wait_next((nk < NS ? nk : NS) - 1);   // stage 0
    Frags f0, f1;
#pragma unroll
    for (int i = 0; i < kFrags; ++i) read_frag(0, 0, f0, i);
    cvt_first(f0);
    for (int kt = 0; kt < nk; ++kt) step(args, smem, kt, f0, f1, acc);
  }

  // dphi: destination row and alpha of the tile's rows into LDS (before the
  // next tile's loads are issued, so that this wait covers only them).
  __device__ __forceinline__ void stage_rows(const Args& args, LDS_AS char* prm) const {
    if (IS_DW) return;
    const int tid = threadIdx.x;
    LDS_AS int32_t* s_perm = reinterpret_cast<LDS_AS int32_t*>(prm);
    LDS_AS float* s_alpha = reinterpret_cast<LDS_AS float*>(prm + kMaxRows * 4);
#pragma unroll
    for (int r = tid; r < TBM; r += kThreads) {
      const bool ok = m0 + r < q;
      const int32_t u = ok ? args.perm[seg + m0 + r] : -1;
      s_perm[r] = (uint32_t)u < (uint32_t)args.P ? u : -1;   // perm holds pair indices < P
      s_alpha[r] = !ok ? 0.f : args.ops.dp_alpha_folded ? 1.f : args.alpha_c[seg + m0 + r];
    }
  }

  // ---- SiLU-GLU chain.  For tile row a this lane holds dphi (before alpha)
  // of compacted row j = pair u in 4 x 4 quads of columns.  With the saved
  // pre-activations a, b of pair u: s = sigmoid(a), silu = a s,
  // silu' = s (1 + a (1 - s)); gate gradient dphi * b * silu', up gradient
  // dphi * silu, rounded to bf16 into glu_out[j] = [gate | up].
  // Lanes l and l + 32 hold the two 4-column halves of each 8-column group
  // of the same row.  Memory is accessed 16 bytes per lane: for the column
  // groups g0 = 2h and g1 = 2h + 1 of block b, lane l moves group g0 and lane
  // l + 32 group g1, and the two swap the halves that belong to the other
  // (ds_bpermute) -- half as many load and store instructions, each touching
  // the same 32 rows, as 8-byte accesses.  The a and b rows are gathered from
  // the original pair layout; the next row's loads stay in flight while the
  // current row is computed.  Nothing branches but the stores: lanes without
  // a row (u < 0) or past the matrix edge (column counts are multiples of 8)
  // load column 0 of row 0 instead.
  struct GluRow {
    u32x4 a[NB][2], b[NB][2];   // [block b][group pair h]
  };

  // First column of the 8-column group this lane moves for pair (b, h).
  __device__ __forceinline__ int glu_col(int ln, int b, int h) const {
    return wn * WN + b * 32 + 16 * h + 8 * (ln >> 5);
  }

  __device__ __forceinline__ void glu_load(const Args& args, int32_t u, int ln, int ncols,
                                           GluRow& r) const {
    const int d_in = args.d_in;
    const bool row_ok = u >= 0;
    const int64_t src = row_ok ? (int64_t)u * d_in + n0 : 0;
    const uint16_t* arow = args.ops.glu_a + src;
    const uint16_t* brow = args.ops.glu_b + src;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int col = glu_col(ln, b, h);
        const int c = row_ok && col < ncols ? col : 0;
        r.a[b][h] = *reinterpret_cast<const u32x4*>(arow + c);
        r.b[b][h] = *reinterpret_cast<const u32x4*>(brow + c);
      }
  }

  // Value of the partner lane (l ^ 32).
  __device__ __forceinline__ static uint32_t swap32(uint32_t v, int ln) {
    return (uint32_t)__builtin_amdgcn_ds_bpermute((ln ^ 32) << 2, (int)v);
  }

  // Gate and up gradients of one 4-column quad (bf16, packed in pairs).
  __device__ __forceinline__ static void glu_quad(u32x2 av, u32x2 bv, const float (&d)[4],
                                                  u32x2& gate, u32x2& up) {
    bf16x4 go, uo;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t aw = av[k >> 1], bw = bv[k >> 1];
      const float x = __uint_as_float((k & 1) ? (aw & 0xFFFF0000u) : (aw << 16));
      const float y = __uint_as_float((k & 1) ? (bw & 0xFFFF0000u) : (bw << 16));
      // Sigmoid from the hardware exp2 and reciprocal (about 1 ulp each, far
      // below the bf16 rounding of the result); exp(-x) = 2^(-x log2(e)),
      // whose overflow to +inf gives s = 0, as it should.
      const float sg = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.44269504f * x));
      go[k] = (__bf16)(d[k] * y * (sg * (1.f + x * (1.f - sg))));
      uo[k] = (__bf16)(d[k] * (x * sg));
    }
    gate = __builtin_bit_cast(u32x2, go);
    up = __builtin_bit_cast(u32x2, uo);
  }

  // The same in float32, unrounded: gate and up gradients of the quad.
  __device__ __forceinline__ static void glu_quad_f32(u32x2 av, u32x2 bv, const float (&d)[4],
                                                      f32x4& gate, f32x4& up) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t aw = av[k >> 1], bw = bv[k >> 1];
      const float x = __uint_as_float((k & 1) ? (aw & 0xFFFF0000u) : (aw << 16));
      const float y = __uint_as_float((k & 1) ? (bw & 0xFFFF0000u) : (bw << 16));
      const float sg = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.44269504f * x));
      gate[k] = d[k] * y * (sg * (1.f + x * (1.f - sg)));
      up[k] = d[k] * (x * sg);
    }
  }

  __device__ __forceinline__ void glu_store(const Args& args, int32_t u, int64_t j, int ln,
                                            int ncols, const f32x16 (&acc)[kMB][kNB], int a,
                                            const GluRow& r) const {
    const int d_in = args.d_in;
    const bool hi = ln >= 32;
    if constexpr (GLU == 2) {
      // float32 output: each lane's register quad is 4 consecutive columns of
      // its own row, 16 bytes, stored as they are (no partner exchange)
      float* gate = reinterpret_cast<float*>(args.ops.glu_out) + j * (2 * (int64_t)d_in) + n0;
      float* up = gate + d_in;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          u32x2 qa[2], qb[2];
          {
            const u32x4 A = r.a[b][h], B = r.b[b][h];
            const uint32_t ra0 = swap32(hi ? A[0] : A[2], ln), ra1 = swap32(hi ? A[1] : A[3], ln);
            const uint32_t rb0 = swap32(hi ? B[0] : B[2], ln), rb1 = swap32(hi ? B[1] : B[3], ln);
            qa[0] = hi ? u32x2{ra0, ra1} : u32x2{A[0], A[1]};
            qa[1] = hi ? u32x2{A[2], A[3]} : u32x2{ra0, ra1};
            qb[0] = hi ? u32x2{rb0, rb1} : u32x2{B[0], B[1]};
            qb[1] = hi ? u32x2{B[2], B[3]} : u32x2{rb0, rb1};
          }
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int g = 2 * h + t;
            float d[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
              asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(d[k]) : "a"(acc[a][b][4 * g + k]));
            f32x4 gv, uv;
            glu_quad_f32(qa[t], qb[t], d, gv, uv);
            // columns of register quad g: 8 g + 4 (lane / 32) .. + 3 of block b
            const int col = wn * WN + b * 32 + 8 * g + 4 * (ln >> 5);
            if (u >= 0 && col < ncols) {
              *reinterpret_cast<f32x4*>(gate + col) = gv;
              *reinterpret_cast<f32x4*>(up + col) = uv;
            }
          }
        }
      return;
    }
    uint16_t* gate = reinterpret_cast<uint16_t*>(args.ops.glu_out) + j * (2 * (int64_t)d_in) + n0;
    uint16_t* up = gate + d_in;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // this lane's quads of groups g0 and g1: its own half of the 16 bytes
        // it loaded, and the partner's half of the partner's load
        u32x2 qa[2], qb[2];
        {
          const u32x4 A = r.a[b][h], B = r.b[b][h];
          const uint32_t ra0 = swap32(hi ? A[0] : A[2], ln), ra1 = swap32(hi ? A[1] : A[3], ln);
          const uint32_t rb0 = swap32(hi ? B[0] : B[2], ln), rb1 = swap32(hi ? B[1] : B[3], ln);
          qa[0] = hi ? u32x2{ra0, ra1} : u32x2{A[0], A[1]};
          qa[1] = hi ? u32x2{A[2], A[3]} : u32x2{ra0, ra1};
          qb[0] = hi ? u32x2{rb0, rb1} : u32x2{B[0], B[1]};
          qb[1] = hi ? u32x2{B[2], B[3]} : u32x2{rb0, rb1};
        }
        u32x2 go[2], uo[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int g = 2 * h + t;
          // read the accumulators straight from their AGPRs, here: a plain
          // use makes the compiler copy all 256 accumulators to VGPRs at once
          float d[4];
#pragma unroll
          for (int k = 0; k < 4; ++k)
            asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(d[k]) : "a"(acc[a][b][4 * g + k]));
          glu_quad(qa[t], qb[t], d, go[t], uo[t]);
        }
        // lane l stores group g0 (its quad, then the partner's); lane l + 32
        // group g1 (the partner's quad, then its own)
        const u32x2 gs = hi ? go[0] : go[1], us = hi ? uo[0] : uo[1];
        const u32x2 gr{swap32(gs[0], ln), swap32(gs[1], ln)};
        const u32x2 ur{swap32(us[0], ln), swap32(us[1], ln)};
        const u32x4 gv = hi ? u32x4{gr[0], gr[1], go[1][0], go[1][1]}
                            : u32x4{go[0][0], go[0][1], gr[0], gr[1]};
        const u32x4 uv = hi ? u32x4{ur[0], ur[1], uo[1][0], uo[1][1]}
                            : u32x4{uo[0][0], uo[0][1], ur[0], ur[1]};
        const int col = glu_col(ln, b, h);
        if (u >= 0 && col < ncols) {
          *reinterpret_cast<u32x4*>(gate + col) = gv;
          *reinterpret_cast<u32x4*>(up + col) = uv;
        }
      }
  }

  __device__ __forceinline__ void glu_epilogue(const Args& args, LDS_AS const char* prm,
                                               const f32x16 (&acc)[kMB][kNB]) const {
    LDS_AS const int32_t* s_perm = reinterpret_cast<LDS_AS const int32_t*>(prm);
    // Opaque copies: keep the compiler from computing the column offsets and
    // edge predicates of every quad ahead of the main loop, where they would
    // stay live across it.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    int ncols = args.d_in - n0;
    asm volatile("" : "+s"(ncols));
    int32_t u[kMB];
#pragma unroll
    for (int a = 0; a < kMB; ++a) u[a] = s_perm[wm * WTM + a * 32 + (ln & 31)];
    GluRow r[2];
    glu_load(args, u[0], ln, ncols, r[0]);
#pragma unroll
    for (int a = 0; a < kMB; ++a) {
      if (a + 1 < kMB) glu_load(args, u[a + 1], ln, ncols, r[(a + 1) & 1]);
      // at most two rows of loads live (128 VGPRs): the accumulators hold
      // every AGPR, so nothing more may be hoisted
      __builtin_amdgcn_sched_barrier(0);
      glu_store(args, u[a], seg + m0 + wm * WTM + a * 32 + (ln & 31), ln, ncols, acc, a,
                r[a & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- epilogue.  Accumulator block (a, b) holds D[m][n] for tile row
  // m = wm*128 + a*32 + lane%32 and column n = wn*128 + b*32 + 8*(r/4) +
  // 4*(lane/32) + r%4 in register r: each register quad is 4 consecutive
  // columns of the lane's own row.  Stores are paired by quads (2p, 2p+1):
  // adjacent lanes (r, r^1) swap one quad each (one DPP lane swap per
  // register), after which the first store of the pair writes the even row
  // of each lane pair and the second the odd row, and each row's 64 bytes
  // 16p .. 16p+15 come from the four lanes r, r^1, r+32, r^1+32 -- two
  // coalesced 32-byte lane pairs instead of two lanes 32 apart per 32 bytes.
  // Column counts are multiples of 4, so a quad never straddles the edge.
  __device__ __forceinline__ static float swap_adjacent(float v) {
    // quad_perm [1, 0, 3, 2]: lane l reads lane l ^ 1
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1,
                                                              0xF, 0xF, false));
  }
  __device__ __forceinline__ void epilogue(const Args& args, const GemmTable& tab,
                                           LDS_AS const char* prm,
                                           const f32x16 (&acc)[kMB][kNB]) const {
    const int d_out = args.d_out, d_in = args.d_in;
    LDS_AS const int32_t* s_perm = reinterpret_cast<LDS_AS const int32_t*>(prm);
    LDS_AS const float* s_alpha = reinterpret_cast<LDS_AS const float*>(prm + kMaxRows * 4);
    // Split dW tiles go to their chunk's partial tile (full 256x256, row-major;
    // the reduction crops it to the matrix edge).  A tall weight-gradient tile
    // spans two row tiles of that grid: waves 0-1 write the upper one, waves
    // 2-3 the lower one (columns 0..127 only, the rest lies past d_in); rows
    // past d_out are not written, so the lower tile may lie past the grid.
    float* part = nullptr;
    const int prow0 = TALL ? (wm >> 1) * kTile : 0;   // first tile row of this wave's partial
    if (IS_DW && chunks > 1) {
      const int tile = ((m0 + prow0) / kTile) * tab.tiles_n + n0 / kTile;
      part = args.ops.partials + ((partial_base(tab, e) + (int64_t)tile * chunks + chunk) << 16);
    }
    if constexpr (GLU != 0) {   // SiLU-GLU chain: no dphi, no alpha
      glu_epilogue(args, prm, acc);
      return;
    }
    // Opaque copies: keep the compiler from computing every quad's column
    // and edge predicate ahead of the main loop, where they would stay live.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    int ncols = (IS_DW && part != nullptr) ? TBN : d_in - n0;
    asm volatile("" : "+s"(ncols));
    const bool odd = (ln & 1) != 0;
    // this lane's column inside each 16-column group: 0/4 (lane half) + 8 (odd lane)
    const int cq = 4 * (ln >> 5) + (odd ? 8 : 0);
    // float16 weight gradient: 2^-(sA + sB) of the expert, applied exactly
    int unscale = 0;
    if constexpr (IS_DW && F16)
      unscale = -(f16_scale_exp(args.ops.dw_ebound[2 * e]) +
                  f16_scale_exp(args.ops.dw_ebound[2 * e + 1]));
#pragma unroll
    for (int a = 0; a < kMB; ++a) {
      // rows of this lane's two stores: the even and the odd row of its pair
      const int lrow0 = wm * WTM + a * 32 + (ln & 30);
      float* orow[2] = {nullptr, nullptr};
      float scale[2] = {1.f, 1.f};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int lrow = lrow0 + h;
        if (IS_DW) {
          if (part != nullptr) {
            if (!TALL || m0 + lrow < mrows) orow[h] = part + (lrow - prow0) * kTile;
          }
          else if (m0 + lrow < mrows) orow[h] = args.dW + ((int64_t)e * d_out + m0 + lrow) * d_in + n0;
        } else {
          const int32_t u = s_perm[lrow];
          scale[h] = s_alpha[lrow];
          if (u >= 0) orow[h] = args.dphi + (int64_t)u * d_in + n0;
        }
      }
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const int col = wn * WN + b * 32 + 16 * p + cq;
          f32x4 v0, v1;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // read straight from the accumulation registers, here: a plain
            // use makes the compiler copy all 256 accumulators at once
            float q0, q1;
            asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(q0) : "a"(acc[a][b][8 * p + i]));
            asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(q1) : "a"(acc[a][b][8 * p + 4 + i]));
            // even lanes pass quad 2p+1 of their row, odd lanes quad 2p
            const float got = swap_adjacent(odd ? q0 : q1);
            v0[i] = odd ? got : q0;   // even row of the pair
            v1[i] = odd ? q1 : got;   // odd row
          }
          if (!IS_DW) {
            v0 *= scale[0];
            v1 *= scale[1];
          }
          if constexpr (IS_DW && F16) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              v0[i] = __builtin_amdgcn_ldexpf(v0[i], unscale);
              v1[i] = __builtin_amdgcn_ldexpf(v1[i], unscale);
            }
          }
          if (col < ncols) {
            if (orow[0] != nullptr) *reinterpret_cast<f32x4*>(orow[0] + col) = v0;
            if (orow[1] != nullptr) *reinterpret_cast<f32x4*>(orow[1] + col) = v1;
          }
        }
    }
  }
};

// LDS stages for a tile whose stage is `bytes` long: as many as fit in
// 144 KiB, at most 4 (0 when not even 2 fit).
constexpr int kStageBudget = 144 * 1024;
constexpr int stages_for(int bytes) {
  return 4 * bytes <= kStageBudget ? 4 : 3 * bytes <= kStageBudget ? 3 : 2 * bytes <= kStageBudget ? 2 : 0;
}
constexpr int cmax(int a, int b) { return a > b ? a : b; }

// Stage counts of the square tiles of both products and of the tall tiles.
// Tall input-gradient tiles run where their stage fits twice.  Tall
// weight-gradient tiles run only in kernels whose dW reads a two-plane
// operand (the exact mode): there they made the GLM 20x GEMM 4.7 % faster;
// with single-pass dW tiles, which halved the tiles in flight, 12 % slower.
template <int DW_PA, int DW_PB, int DP_PA, int DP_PB>
struct Cfg {
  static constexpr int sq = kPlaneBytes;                         // square tile plane
  static constexpr int ta = 2 * kPlaneBytes, tb = kPlaneBytes / 2;   // tall tile A / B plane
  static constexpr int NS_DW = stages_for((DW_PA + DW_PB) * sq);
  static constexpr int NS_DP = stages_for((DP_PA + DP_PB) * sq);
  static constexpr int NS_DPT = stages_for(DP_PA * ta + DP_PB * tb);
  static constexpr int NS_DWT = stages_for(DW_PA * ta + DW_PB * tb);
  static constexpr bool tall_fits = NS_DPT >= 2;
  static constexpr bool tall_dw = tall_fits && DW_PA + DW_PB >= 3 && NS_DWT >= 2;
  static constexpr int stages =
      cmax(cmax(NS_DW * (DW_PA + DW_PB) * sq, NS_DP * (DP_PA + DP_PB) * sq),
           cmax(tall_fits ? NS_DPT * (DP_PA * ta + DP_PB * tb) : 0,
                tall_dw ? NS_DWT * (DW_PA * ta + DW_PB * tb) : 0));
  static constexpr int sink = stages + kPermBytes + 16;   // kWaves x 1 KiB
  static constexpr int bytes = sink + kWaves * 1024;
  static_assert(NS_DW >= 2 && NS_DP >= 2, "stages");
  static_assert(bytes <= 160 * 1024, "LDS");
};

// Zero-fill of the input-gradient rows of dropped pairs (zero_keep[u] == 0),
// memory-bound work that runs beside the matrix-core-bound tiles of the same
// launch.  A workgroup claims kZeroChunk consecutive pairs at a time from the
// zero counter; each wave reads the keep bytes of 64 of them, one per lane,
// and clears the rows whose ballot bit is set, 16 bytes per lane per store,
// marked non-temporal (nothing reads them back in this launch; as ordinary
// stores they evicted the tiles' operands from the caches and cost the
// launch about 4% more).  Returns when every chunk has been claimed.
constexpr int kZeroChunk = 256;
__device__ __forceinline__ void zero_dropped(const Args& args, LDS_AS int32_t* s_next) {
  if (args.ops.zero_rows == nullptr) return;
  const int64_t P = args.P;
  const int nchunks = (int)((P + kZeroChunk - 1) / kZeroChunk);
  const int zch = args.d_in / 4;   // float4 per row (d_in % 4 == 0)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (;;) {
    if (threadIdx.x == 0) s_next[0] = atomicAdd(args.ops.queue_heads + kZeroCounter, 1);
    lds_barrier();
    const int c = __builtin_amdgcn_readfirstlane(s_next[0]);
    lds_barrier();   // everyone has read s_next before it is rewritten
    if (c >= nchunks) return;
    const int64_t u0 = (int64_t)c * kZeroChunk + 64 * wave;
    const bool drop = u0 + lane < P && args.ops.zero_keep[u0 + lane] == 0;
    uint64_t m = __ballot(drop);
    while (m != 0) {
      const int r = __builtin_ctzll(m);
      m &= m - 1;
      f32x4* row = reinterpret_cast<f32x4*>(args.ops.zero_rows) + (u0 + r) * zch;
      for (int i = lane; i < zch; i += 64)
        __builtin_nontemporal_store(f32x4{0.f, 0.f, 0.f, 0.f}, row + i);
    }
  }
}

// Persistent: one workgroup per CU drains its XCD's queue.  Between tiles the
// next tile's first loads are issued before the finished tile's stores, so
// the store drain overlaps the next load latency.  Every workgroup exits when
// every queue's counter and the zero-fill counter have passed their ends.
template <int DW_PA, int DW_PB, int DP_PA, int DP_PB, int GLU, int DW_F16>
__global__ __launch_bounds__(kThreads, 1) void grouped_backward_kernel(Args args, GemmTable tab) {
  using C = Cfg<DW_PA, DW_PB, DP_PA, DP_PB>;
  using DwTile = Tile<true, DW_PA, DW_PB, C::NS_DW, 0, DW_F16>;
  using DpTile = Tile<false, DP_PA, DP_PB, C::NS_DP, GLU>;
  // tall edge tiles: not with the SiLU-GLU epilogue
  constexpr bool kTall = GLU == 0 && C::tall_fits;
  constexpr bool kTallDw = kTall && C::tall_dw;
  using DpTall = Tile<false, DP_PA, DP_PB, kTall ? C::NS_DPT : 2, 0, false, true>;
  using DwTall = Tile<true, DW_PA, DW_PB, kTallDw ? C::NS_DWT : 2, 0, DW_F16, true>;
  // 256 x 128 weight-gradient tiles for a last column of at most 128 columns,
  // where weight-gradient tiles are not tall (one operand plane per side, no
  // conversion in registers): no MFMA works on the empty half
  constexpr bool kHalfDw =
      !kTallDw && GLU == 0 && DW_PA == 1 && DW_PB == 1 && (DW_F16 == 0 || DW_F16 == 3);
  constexpr int kHalfStage = DW_PA * kPlaneBytes + DW_PB * kPlaneBytes / 2;
  constexpr int kNsHalf = C::stages / kHalfStage > 4 ? 4 : C::stages / kHalfStage;
  using DwHalf = Tile<true, DW_PA, DW_PB, kHalfDw ? kNsHalf : 2, 0, kHalfDw ? DW_F16 : 0, false,
                      true>;
  const bool tall_on = kTall && tab.tall != 0;
  __shared__ __attribute__((aligned(16))) char smem_raw[C::bytes];
  LDS_AS char* smem = (LDS_AS char*)(smem_raw);
  LDS_AS char* prm = smem + C::stages;
  LDS_AS int32_t* s_next = reinterpret_cast<LDS_AS int32_t*>(prm + kPermBytes);
  LDS_AS char* sink = smem + C::sink;
  const int x = blockIdx.x % kXcds;
  int qx = x;   // the queue this workgroup currently drains

  // Next valid item (idle slots skipped): from this XCD's queue, then --
  // once that is exhausted -- from the other XCDs' queues in turn, so that no
  // CU idles while another XCD still has tiles.  -1 when every queue is done.
  // A stolen tile loses the L2 locality of its group, which only matters at
  // the end of the launch.
  auto fetch = [&](bool& is_dw, TileJob& job) -> int {
    for (int hop = 0; hop < kXcds;) {
      const int nit = queue_items(tab, qx);
      if (threadIdx.x == 0) s_next[0] = atomicAdd(args.ops.queue_heads + qx, 1);
      lds_barrier();
      const int i = __builtin_amdgcn_readfirstlane(s_next[0]);
      lds_barrier();   // everyone has read s_next before it is rewritten
      if (i >= nit) {   // this queue is exhausted: move to the next XCD's
        qx = qx + 1 == kXcds ? 0 : qx + 1;
        ++hop;
        continue;
      }
      if (decode(tab, qx, i, is_dw, job, tall_on, kTallDw, kHalfDw)) return i;
    }
    return -1;
  };
  // Runs fn on the tile of job j (one of up to four tile types).
  auto with_tile = [&](bool is_dw, const TileJob& j, auto&& fn) __attribute__((always_inline)) {
    if (is_dw) {
      if constexpr (kTallDw) {
        if (j.tall) {
          fn(DwTall(args, tab, j, smem, sink));
          return;
        }
      }
      if constexpr (kHalfDw) {
        if (j.half) {
          fn(DwHalf(args, tab, j, smem, sink));
          return;
        }
      }
      fn(DwTile(args, tab, j, smem, sink));
      return;
    }
    if constexpr (kTall) {
      if (j.tall) {
        fn(DpTall(args, tab, j, smem, sink));
        return;
      }
    }
    fn(DpTile(args, tab, j, smem, sink));
  };

  f32x16 acc[kMB][kNB];
  if ((int)blockIdx.x < args.ops.zero_first) zero_dropped(args, s_next);
  bool cur_dw;
  TileJob cur;
  if (fetch(cur_dw, cur) < 0) {
    zero_dropped(args, s_next);
    return;
  }
  with_tile(cur_dw, cur, [&](const auto& t) __attribute__((always_inline)) { t.prologue(args, smem); });
  for (;;) {
    with_tile(cur_dw, cur, [&](const auto& t) __attribute__((always_inline)) {
      t.mainloop(args, smem, acc);
      t.stage_rows(args, prm);   // dphi tiles only
    });
    bool nxt_dw;
    TileJob nxt;
    const bool more = fetch(nxt_dw, nxt) >= 0;   // its barrier also frees every stage
    if (more)
      with_tile(nxt_dw, nxt, [&](const auto& t) __attribute__((always_inline)) { t.prologue(args, smem); });
    with_tile(cur_dw, cur, [&](const auto& t) __attribute__((always_inline)) {
      t.epilogue(args, tab, prm, acc);
    });
    if (!more) break;
    lds_barrier();   // the perm/alpha rows are read before the next tile restages them
    cur_dw = nxt_dw;
    cur = nxt;
  }
  zero_dropped(args, s_next);   // help with what is left of the zero-fill
}

template <int DW_PA, int DW_PB, int DP_PA, int DP_PB, int GLU = 0, int DW_F16 = 0>
hipError_t launch(const Args& args, const GemmTable& tab, hipStream_t s) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  const int blocks = (cus + kXcds - 1) / kXcds * kXcds;   // one per CU, a multiple of 8
  hipLaunchKernelGGL((grouped_backward_kernel<DW_PA, DW_PB, DP_PA, DP_PB, GLU, DW_F16>), dim3(blocks),
                     dim3(kThreads), 0, s, args, tab);
  return hipGetLastError();
}

// ------------------------------------------------------------ split-K reduction
// dW tile of a split expert = sum over its K chunks (in chunk order) of the
// fp32 partial tiles, cropped to the matrix edge.  Each workgroup reduces a
// 16 KiB slice of one tile; each thread keeps 4 independent 16-byte loads per
// chunk in flight.
constexpr int kRedThreads = 256;
constexpr int kRedVec = 4;                                        // f32x4 per thread
constexpr int kRedSlices = kTile * kTile / 4 / (kRedThreads * kRedVec);   // slices per tile

__global__ __launch_bounds__(kRedThreads) void reduce_partials_kernel(
    GemmTable tab, const float* __restrict__ partials, float* __restrict__ dW, int32_t d_out,
    int32_t d_in) {
  const int tiles = tab.dw_tiles_m * tab.tiles_n;
  int b = blockIdx.x / kRedSlices;
  const int slice = blockIdx.x % kRedSlices;
  int e = 0, S = 1;
  for (; e < tab.E; ++e) {   // the b-th tile among split experts
    S = dw_chunks(tab.seg_off[e + 1] - tab.seg_off[e], tab.kc);
    if (S > 1) {
      if (b < tiles) break;
      b -= tiles;
    }
  }
  if (e >= tab.E) return;
  const int tile = b;
  const int m0 = (tile / tab.tiles_n) * BM, n0 = (tile % tab.tiles_n) * BN;
  const f32x4* src = reinterpret_cast<const f32x4*>(
      partials + ((partial_base(tab, e) + (int64_t)tile * S) << 16));
  const int v0 = slice * (kRedThreads * kRedVec) + threadIdx.x;
  f32x4 acc[kRedVec];
#pragma unroll
  for (int i = 0; i < kRedVec; ++i) acc[i] = src[v0 + i * kRedThreads];
  for (int c = 1; c < S; ++c) {
    const f32x4* sc = src + (int64_t)c * (BM * BN / 4);
    f32x4 x[kRedVec];
#pragma unroll
    for (int i = 0; i < kRedVec; ++i) x[i] = sc[v0 + i * kRedThreads];
#pragma unroll
    for (int i = 0; i < kRedVec; ++i) acc[i] += x[i];
  }
#pragma unroll
  for (int i = 0; i < kRedVec; ++i) {
    const int v = v0 + i * kRedThreads;
    const int row = v / (BN / 4), col = (v % (BN / 4)) * 4;
    if (m0 + row < d_out && n0 + col < d_in)
      *reinterpret_cast<f32x4*>(dW + ((int64_t)e * d_out + m0 + row) * d_in + n0 + col) = acc[i];
  }
}

// ------------------------------------------------------------ operand prologue
// hi/lo bf16 planes of alpha[row] * src[row][8c .. 8c+7] (cols % 8 == 0 for
// bf16 sources; float32 sources also allow cols % 4 == 0 via a 4-wide tail).
template <bool F32>
__global__ __launch_bounds__(256) void split_kernel(const void* __restrict__ src, int64_t rows,
                                                    int32_t cols, const float* __restrict__ alpha,
                                                    uint16_t* __restrict__ hi,
                                                    uint16_t* __restrict__ lo,
                                                    int32_t* __restrict__ zero, int nzero) {
  // also clears the grouped GEMM's work-queue counters (saves a launch)
  if (blockIdx.x == 0 && (int)threadIdx.x < nzero) zero[threadIdx.x] = 0;
  const int64_t quads = rows * (cols / 4);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int qpr = cols / 4;   // 4-element groups per row
  for (int64_t oc = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; 2 * oc < quads;
       oc += stride) {
    // this thread: 4-element groups 2*oc and 2*oc+1 (the second may be on the next row
    // for float32 sources with an odd number of groups per row)
    float x[8];
    int64_t qd0 = 2 * oc;
    const bool two = qd0 + 1 < quads;
    if (F32) {
      const f32x4* s4 = reinterpret_cast<const f32x4*>(src);
      const f32x4 a = s4[qd0];
      const f32x4 b = two ? s4[qd0 + 1] : f32x4{0.f, 0.f, 0.f, 0.f};
      x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
      x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
    } else {   // cols % 8 == 0: both groups are on one row, one 16-byte load
      const u32x4 v = reinterpret_cast<const u32x4*>(src)[oc];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(v[i] << 16);
        x[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
      }
    }
    const float a0 = alpha ? alpha[qd0 / qpr] : 1.f;
    const float a1 = alpha ? alpha[(qd0 + 1) / qpr] : 1.f;
    bf16x8 h, l;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const HiLo e = alpha_split(i < 4 ? a0 : a1, x[i]);
      h[i] = e.h;
      l[i] = e.l;
    }
    const u32x4 hw = __builtin_bit_cast(u32x4, h), lw = __builtin_bit_cast(u32x4, l);
    if (two) {
      reinterpret_cast<u32x4*>(hi)[oc] = hw;
      if (lo) reinterpret_cast<u32x4*>(lo)[oc] = lw;
    } else {
      reinterpret_cast<u32x2*>(hi)[qd0] = u32x2{hw[0], hw[1]};
      if (lo) reinterpret_cast<u32x2*>(lo)[qd0] = u32x2{lw[0], lw[1]};
    }
  }
}

__global__ void zero_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

hipError_t launch_zero(int32_t* p, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_split(int src_dtype, const void* src, int64_t rows, int32_t cols,
                        const float* alpha, uint16_t* hi, uint16_t* lo, hipStream_t s,
                        int32_t* zero, int nzero) {
  const int64_t quads = rows * (cols / 4);
  if (quads <= 0) return nzero > 0 ? launch_zero(zero, nzero, s) : hipSuccess;
  int64_t blocks = (quads / 2 + 255) / 256 + 1;
  if (blocks > 256 * 16) blocks = 256 * 16;
  if (src_dtype == LRMOE_F32)
    hipLaunchKernelGGL(split_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, src, rows,
                       cols, alpha, hi, lo, zero, nzero);
  else
    hipLaunchKernelGGL(split_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, src, rows,
                       cols, alpha, hi, lo, zero, nzero);
  return hipGetLastError();
}

hipError_t launch_reduce_partials(const GemmTable& tab, const float* partials, float* dW,
                                  int32_t d_out, int32_t d_in, hipStream_t s) {
  int64_t blocks = 0;
  for (int e = 0; e < tab.E; ++e)
    if (dw_chunks(tab.seg_off[e + 1] - tab.seg_off[e], tab.kc) > 1)
      blocks += (int64_t)tab.dw_tiles_m * tab.tiles_n;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(reduce_partials_kernel, dim3((unsigned)(blocks * kRedSlices)),
                     dim3(kRedThreads), 0, s, tab, partials, dW, d_out, d_in);
  return hipGetLastError();
}

hipError_t launch_grouped_backward(const GemmTable& tab, const GemmOperands& ops,
                                   const int32_t* perm, const float* alpha_c, float* dW,
                                   float* dphi, int32_t d_out, int32_t d_in, int32_t P,
                                   hipStream_t s) {
  const Args args{ops, alpha_c, perm, dW, dphi, d_out, d_in, P};
  const int key = ops.dw_pa * 1000 + ops.dw_pb * 100 + ops.dp_pa * 10 + ops.dp_pb;
  if (ops.dw_f16) {   // float16 weight gradient, bf16 input gradient
    if (key != 1111 || ops.dw_ebound == nullptr) return hipErrorInvalidValue;
    if (ops.glu_out != nullptr) {
      if (!ops.glu_f32) return hipErrorInvalidValue;
      switch (ops.dw_f16) {
        case 1: return launch<1, 1, 1, 1, 2, 1>(args, tab, s);
        case 2: return launch<1, 1, 1, 1, 2, 2>(args, tab, s);
        case 3: return launch<1, 1, 1, 1, 2, 3>(args, tab, s);
        default: return hipErrorInvalidValue;
      }
    }
    switch (ops.dw_f16) {
      case 1: return launch<1, 1, 1, 1, 0, 1>(args, tab, s);
      case 2: return launch<1, 1, 1, 1, 0, 2>(args, tab, s);
      case 3: return launch<1, 1, 1, 1, 0, 3>(args, tab, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (ops.glu_out != nullptr) {   // SiLU-GLU chain: bf16 storage only
    if (ops.glu_f32) {            // exact weight gradient, float32 hand-off
      switch (key) {
        case 1211: return launch<1, 2, 1, 1, 2>(args, tab, s);
        case 2111: return launch<2, 1, 1, 1, 2>(args, tab, s);
        default: return hipErrorInvalidValue;
      }
    }
    switch (key) {                // single rounding, bf16 hand-off
      case 1111: return launch<1, 1, 1, 1, 1>(args, tab, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (key) {
    case 1211: return launch<1, 2, 1, 1>(args, tab, s);   // bf16, alpha folded into phi
    case 2111: return launch<2, 1, 1, 1>(args, tab, s);   // bf16, alpha folded into g
    case 1111: return launch<1, 1, 1, 1>(args, tab, s);   // bf16, single rounding
    case 2121: return launch<2, 1, 2, 1>(args, tab, s);   // float32 g_c, bf16 phi_c and W
    case 2222: return launch<2, 2, 2, 2>(args, tab, s);   // float32 storage
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lrmoe
