// Kernels 2+3: gather the sub-table rows and project them, with the E_0 epilogue.
//
// Computes the final form of section A2 of the deep-notes page on "Scaling Embeddings
// Outperforms Scaling Experts in Language Models" for a batch of rows r:
//   out[r] = ( E_0[tok[r]] + sum_s W_{n,k} E_{n,k}[idx[r, s]] ) / ((N-1)K + 1).
// Stacking the W_{n,k} side by side into W [D, D] (W[o, s*d + c] = W_{n,k}[o, c]) and the
// gathered rows into g_r = [E_{2,1}[.], E_{2,2}[.], ...] (length D) turns the double sum
// into one product W g_r, so the whole batch is a single [rows, D] x [D, D]^T contraction:
// the only dense work on the path. Both operands are contiguous along the contraction
// axis, which is the layout the matrix cores want.
//
// bf16 path (D % 256 == 0, d % 64 == 0): tiles of BM rows x BN outputs (BN = 256, or 128
// for small batches), 64-deep slices.
// A 64-deep slice never straddles two sub-tables, so for each of the BM rows the A-loader
// reads one 128-byte piece (a full L2 line) of one sub-table row straight from HBM into
// LDS (global_load_lds_dwordx4; no gathered copy of the batch is ever written). W slices
// travel the same way. Slices sit in XOR-swizzled LDS buffers (2 for 256-row tiles, 3 or 4
// for shorter ones); the loads of the next slice fly while 8 waves (2 per SIMD) multiply the
// current one with v_mfma_f32_32x32x16_bf16 (fp32 accumulation). Waits and barriers are
// explicit, so loads stay in flight across them. The epilogue adds the E_0 row, scales by
// 1/(S+1) (times the output factor of the scale amplification, section 3.2.4) in fp32 and
// rounds once to bf16, or, for the layer-normalisation amplification, stores the unrounded
// fp32 rows that the normalisation pass reads.
// Measured on MI355X (64K rows, D = 3072): the loads into LDS, not the matrix cores, bound
// this kernel. Dropping either operand's slice loads saves less than their sum, and running
// one operand's loads two slices ahead gains nothing, so the bytes each CU moves into LDS per
// slice set the pace; the tile order below is chosen for L2 reuse.
// Blocks are numbered so that the 32 blocks resident on one XCD at a time cover 4 row
// tiles x 8 output tiles, which keeps their A rows and W panels in that XCD's L2.
#include <algorithm>
#include <atomic>

#include "bf16.h"
#include "kernels.h"
#include "lds_dma.h"

namespace ngram {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));   // one 16-byte vector
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
// E_0 piece of VO consecutive bf16 outputs: 16 bytes for 8, 8 bytes for 4
template <int VO> struct EVec;
template <> struct EVec<8> { typedef u32x4_t type; };
template <> struct EVec<4> { typedef u32x2_t type; };

// One product out[m, n] = inv * (E0[tok[m], n] + sum_k A[m, k] B[n, k]) over nrows rows m and
// N outputs n, with A's row m the concatenation of the S gathered rows E[s][idx[m, s]] (K
// values in all, d per sub-table) and B [N, K] row-major with row stride ldb. The layer's
// forward has N = K = ldb = ldo = D; its backward runs dense products through the same
// kernels: a dense A is one "sub-table" read with identity indices, and E0 is null.
// Per-layer embeddings batch several layers (their own tables, W and output; the same rows
// and indices) into one launch: blockIdx.z is the layer.
struct ProjArgs {
  const void* E[kMaxLaunchTables];    // sub-table s of launch layer l: E[l * S + s]
  uint32_t Vm1[NGRAM_MAX_SUBTABLES];  // V_{n,k} - 1: indices are clamped to their table
  const int32_t* idx;                 // [nrows, S], shared by the layers
  const int32_t* tok;                 // [nrows]; outside [0, V0) -> zero row (E0 only)
  const void* E0[kMaxLaunchLayers];   // [V0, N], or null: no E_0 term, every row valid
  const void* W[kMaxLaunchLayers];    // B operand [N, ldb] (the stacked W in the layer)
  void* out[kMaxLaunchLayers];        // [nrows, ldo]: config dtype, fp32, or fp32 partials
                                      // [splits, nrows, ldo]
  int32_t layers;                     // layers in this launch (gridDim.z)
  int64_t nrows;
  int64_t ldb, ldo;                   // row strides of B and of the output, in elements
  int32_t K, N, S, d, V0;
  float inv;                          // output factor / (S + 1), or the product's factor
  int32_t tiles_m, tiles_n;
  int32_t splits;                     // contraction ranges (partial-sum output only)
  int32_t row_group, row_stride, row_off;   // output row of compact row m (see RowMap)
};

// Output row of compact row m; rows whose token is kSkipRow are not written at all.
__device__ __forceinline__ int64_t out_row(const ProjArgs& a, int64_t m) {
  return a.row_group ? (m / a.row_group) * a.row_stride + a.row_off + m % a.row_group : m;
}

// Output modes of the matrix-core kernel.
enum OutMode {
  kOutBf16 = 0,     // inv * (acc + E_0 row), rounded once to bf16 (the layer's output)
  kOutF32 = 1,      // the same value unrounded, fp32 (layer-norm input; dense products)
  kOutPartial = 2   // acc of this block's contraction range, fp32, no E_0 and no factor
};

// ------------------------------------------------------------------ bf16 matrix-core path

constexpr int kBN = 256;          // outputs per tile (128 for small batches, see run_product)
constexpr int kBK = 64;           // slice depths divide this (the routing checks d % kBK)

// LDS for a tile's hash indices (BM * S int32) and, at its end, the rows' E_0 tokens (BM
// int32): S <= 16 fits 256-row tiles, S <= 31 128-row tiles, S <= 64 64-row tiles.
template <int BM> struct IdxLds {
  static constexpr int bytes = BM >= 256 ? 17408 : BM >= 128 ? 16384 : 16640;
};

// Contraction depth of one slice (BK = 64: a full 128-byte L2 line of each row per load)
// and LDS slice buffers (NST; 160 KB of LDS per CU): 256-row tiles double-buffer, shorter
// tiles keep two slices in flight, 64-row tiles of 128 or 64 outputs (the smallest batches)
// three: 256 rows of the 30B layer in 64 x 128 tiles, 29.8 vs 33.1 us per call (four in
// flight: 31.3 us; 64 x 64 tiles: 26.8 vs 24.4 us; 128 x 128 decode tiles gain nothing from
// a third: 43.4 vs 43.2 us per step). Measured on the 64K-token batch and
// not adopted: 32-deep slices with four buffers (twice the barriers, half-line loads): 1365
// vs 1251 us; for small batches, 128-deep slices (two buffers): slower by 12-14%.
template <int BM, int BN> struct Tile {
  static constexpr int BK = 64;
  static constexpr int NST = BM >= 256 ? 2 : (BM == 64 && BN <= 128) ? 4 : 3;
  static_assert(NST * (BM + BN) * BK * 2 + IdxLds<BM>::bytes <= 163840,
                "the slice buffers and the tile's indices must fit the LDS");
};

// Wait until at most N of this wave's global loads are in flight (they complete in issue
// order), then meet the other waves. The memory clobber keeps LDS accesses on their side.
template <int N>
__device__ __forceinline__ void wait_loads_and_meet() {
  asm volatile("s_waitcnt vmcnt(%0)\n\t"
               "s_waitcnt lgkmcnt(0)\n\t"
               "s_barrier" :: "n"(N) : "memory");
}

// Wave grid of a tile: 8 waves (2 per SIMD, so one can issue while the other waits on
// memory), all loading; the NWC that multiply lie WGM along rows x NWC/WGM along outputs,
// each owning a WM x WN block of 32x32 matrix-core tiles.
// (16 waves of 64x64 outputs, 4 per SIMD in 122 VGPRs, measured the same: 1214 vs 1212 us.)
template <int BM, int BN> struct WaveGrid {
  static constexpr int NW = 8;   // waves per block
  // waves that multiply: 64 x 64 tiles (the smallest batches) have four 32 x 32 blocks, and
  // the other four waves only load (a CU's load rate grows with the waves issuing loads)
  static constexpr int NWC = BM == 64 && BN == 64 ? 4 : NW;
  static constexpr int WGM = BM >= 128 ? 4 : 2;
};

template <int BM, int OM, int BN>
__global__ __launch_bounds__((WaveGrid<BM, BN>::NW * 64), 1) void proj_mfma_kernel(const ProjArgs a) {
  constexpr int NST = Tile<BM, BN>::NST;
  constexpr int BK = Tile<BM, BN>::BK;
  constexpr int RB = BK * 2;             // bytes of one row per slice
  constexpr int CPR = RB / 16;           // 16-byte chunks per row per slice
  constexpr int RPL = 1024 / RB;         // rows per wave load (64 lanes x 16 bytes)
  constexpr int KS = BK / 16;            // 16-deep k-steps per slice
  constexpr int NW = WaveGrid<BM, BN>::NW;
  constexpr int NT = NW * 64;            // threads per block
  constexpr int WGM = WaveGrid<BM, BN>::WGM;
  constexpr int NWC = WaveGrid<BM, BN>::NWC;
  constexpr int WGN = NWC / WGM;
  constexpr int AR = BM / NW;            // A rows each wave loads
  constexpr int BR = BN / NW;            // W rows each wave loads
  constexpr int WM = BM / WGM;           // rows per wave
  constexpr int WN = BN / WGN;           // outputs per wave
  constexpr int TI = WM / 32;            // 32-row MFMA blocks per wave
  constexpr int TJ = WN / 32;            // 32-output MFMA blocks per wave
  constexpr int A_BYTES = BM * RB;       // rows of RB bytes, XOR-swizzled 16-byte chunks
  constexpr int B_BYTES = BN * RB;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int QA = A_BYTES / (NW * 1024);   // A loads per wave per slice (RPL rows each)
  constexpr int QB = B_BYTES / (NW * 1024);   // W loads per wave per slice
  constexpr int PER_SLICE = QA + QB;
  // One LDS pool: NST slice stages + the tile's hash indices during the main loop; the
  // epilogue then reuses it to turn each wave's results into row-major order.
  // bytes per staged fp32 row: 16 bytes past a multiple of 256, so the 16 rows one write
  // instruction's lane group covers fall in 16 different 16-byte bank groups
  constexpr int EP_PITCH = WN * 4 + 16;
  constexpr int IDXB = IdxLds<BM>::bytes;
  constexpr int POOL = NST * STAGE + IDXB;
  static_assert(NW * 32 * EP_PITCH <= POOL - BM * 4,
                "epilogue staging must fit the LDS pool, short of the tokens");
  __shared__ __attribute__((aligned(1024))) char lds[POOL];
  int32_t* sidx = reinterpret_cast<int32_t*>(lds + NST * STAGE);
  int32_t* stok = reinterpret_cast<int32_t*>(lds + NST * STAGE + IDXB - BM * 4);

  // -- XCD-aware tile order: block b runs on XCD b % 8; give each XCD a contiguous range
  //    of virtual tiles and walk a range GM row tiles at a time, outputs slowest, so the
  //    32 blocks resident on an XCD share 4 tiles of gathered rows and 8 panels of W in
  //    its L2 (the best of the 2..32 row-tile groups measured).
  //    The contraction ranges of one tile (partial-sum output) take consecutive numbers.
  const int nb = a.tiles_m * a.tiles_n * (OM == kOutPartial ? a.splits : 1);
  const int b = blockIdx.x;
  const int xcd = b & 7, local = b >> 3;
  const int per = nb >> 3, rem = nb & 7;
  const int vb = xcd * per + (xcd < rem ? xcd : rem) + local;
  const int split = OM == kOutPartial ? vb % a.splits : 0;
  const int v = OM == kOutPartial ? vb / a.splits : vb;
  constexpr int GM = 4;
  const int group = v / (GM * a.tiles_n);
  const int first_m = group * GM;
  const int gm = min(GM, a.tiles_m - first_m);
  const int in_group = v - group * GM * a.tiles_n;
  const int tm = first_m + in_group % gm;
  const int tn = in_group / gm;
  const int64_t m0 = int64_t(tm) * BM;
  const int n0 = tn * BN;

  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const bool mult = NWC == NW || w < NWC;   // this wave multiplies (else it only loads)
  const int wm = mult ? w / WGN : 0, wn = mult ? w % WGN : 0;

  // -- hash indices of the tile's rows (rows past the batch repeat the last row), and the
  //    rows' E_0 tokens for the epilogue (-1 past the batch; 0 without E_0)
  for (int e = t; e < BM * a.S; e += NT) {
    const int r = e / a.S, s = e - r * a.S;
    const int64_t m = m0 + r < a.nrows ? m0 + r : a.nrows - 1;
    sidx[e] = a.idx[m * a.S + s];
  }
  if (OM != kOutPartial && t < BM) {
    const int64_t m = m0 + t;
    stok[t] = m < a.nrows ? (a.E0[blockIdx.z] != nullptr ? a.tok[m] : 0) : -1;
  }
  __syncthreads();

  // -- loads: lane p fills LDS chunk (row p/CPR, chunk p%CPR) of an RPL-row group with
  //    logical 16-byte chunk c = (p%CPR) ^ swz(row), CPR lanes per row piece. LDS has 64
  //    banks of 4 bytes: a 16-byte read serves 16 lanes per cycle, and a fragment read's 16
  //    lanes are 16 consecutive rows, one logical chunk. With 128-byte rows two rows span
  //    the 256 bytes of banks, so swz(r) = (r/2) mod 8 puts the 16 rows in 16 different
  //    16-byte bank groups (r mod 8 left rows r and r+8 colliding: 1.9% slower). 64-byte
  //    rows: (r/2) mod 4.
  auto swz = [](int r) __attribute__((always_inline)) {
    return CPR == 8 ? (r >> 1) & 7 : (r / (8 / CPR)) % CPR;
  };
  const int prow = lane / CPR;
  // physical chunk of load q's row (A rows of this wave, then W rows)
  auto pchunk_a = [&](int q) __attribute__((always_inline)) {
    return (lane % CPR) ^ swz(w * AR + q * RPL + prow);
  };
  auto pchunk_b = [&](int q) __attribute__((always_inline)) {
    return (lane % CPR) ^ swz(w * BR + q * RPL + prow);
  };
  const uint32_t lds0 = lds_address(lds);
  const int layer = blockIdx.z;
  const uint16_t* const* E = reinterpret_cast<const uint16_t* const*>(a.E) + layer * a.S;
  const uint16_t* W = static_cast<const uint16_t*>(a.W[layer]);
  const uint16_t* bp = W + int64_t(n0 + w * BR + prow) * a.ldb;
  const uint16_t* ap[QA];
  const int KT_ALL = a.K / BK;   // slices of the whole contraction
  // this block's slice range (all of it unless the contraction is split)
  const int kt_lo = OM == kOutPartial ? int(int64_t(split) * KT_ALL / a.splits) : 0;
  const int kt_hi = OM == kOutPartial ? int(int64_t(split + 1) * KT_ALL / a.splits) : KT_ALL;
  const int kps = a.d / BK;      // slices per sub-table
  int s_cur = -1;

  // The slice being fetched: its LDS stage, its offset within the current sub-table.
  uint32_t f_sb = 0;
  int f_koff = 0, f_kt = 0;
  auto prep = [&](int kt) __attribute__((always_inline)) {
    if (kt == kt_lo || kt == (s_cur + 1) * kps) {   // first slice of the range or of a table
      s_cur = kt / kps;
#pragma unroll
      for (int q = 0; q < QA; ++q) {
        const int r = w * AR + q * RPL + prow;
        const uint32_t id = min(uint32_t(sidx[r * a.S + s_cur]), a.Vm1[s_cur]);
        ap[q] = E[s_cur] + int64_t(id) * a.d + pchunk_a(q) * 8;
      }
    }
    f_sb = lds0 + uint32_t((kt - kt_lo) % NST) * STAGE;
    f_koff = (kt - s_cur * kps) * BK;
    f_kt = kt;
  };
  // load q of this wave's PER_SLICE loads of the slice (A rows first, then W rows)
  auto dma = [&](int q) __attribute__((always_inline)) {
    if (q < QA)
      dma16(ap[q] + f_koff, f_sb + w * AR * RB + q * 1024);
    else
      dma16(bp + int64_t((q - QA) * RPL) * a.ldb + pchunk_b(q - QA) * 8 + f_kt * BK,
            f_sb + A_BYTES + w * BR * RB + (q - QA) * 1024);
  };
  auto issue = [&](int kt) __attribute__((always_inline)) {
    prep(kt);
#pragma unroll
    for (int q = 0; q < PER_SLICE; ++q) dma(q);
  };

  f32x16_t acc[TJ][TI];
#pragma unroll
  for (int j = 0; j < TJ; ++j)
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.f;

  // fragment lane (fr, fk): 8 consecutive k (logical chunk 2*kk + fk) of row fr
  const int fr = lane & 31, fk = lane >> 5;
  const int arow0 = (wm * WM + fr) * RB;           // byte offset of the lane's first A row
  const int brow0 = A_BYTES + (wn * WN + fr) * RB;
  int pcs[KS];                                     // physical chunk byte offset per k-step
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) pcs[kk] = ((2 * kk + fk) ^ swz(fr)) * 16;

  bf16x8_t wf[2][TJ], xf[2][TI];
  auto frags = [&](const char* sp, int kk, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < TJ; ++j)
      wf[buf][j] = *reinterpret_cast<const bf16x8_t*>(sp + brow0 + j * 32 * RB + pcs[kk]);
#pragma unroll
    for (int i = 0; i < TI; ++i)
      xf[buf][i] = *reinterpret_cast<const bf16x8_t*>(sp + arow0 + i * 32 * RB + pcs[kk]);
  };
  // One 16-deep k-step: TI x TJ matrix-core ops. W block as the first operand: each lane's
  // results are 4 consecutive outputs of one row, which makes the epilogue's E_0 reads and
  // stores 8 bytes wide. The next slice's loads are spread between the ops (DPP per k-step):
  // issued all at once after the barrier, the 8 waves' loads overflow the address unit's
  // queue and hold every wave at issue, away from its matrix-core work. 256-row tiles (two
  // stages, so the loads must land within the slice) place them in the first three of the
  // four k-steps, which measured ~2% faster than all four; shorter tiles use all four.
  constexpr int NM = TI * TJ;
  constexpr int LOAD_STEPS = NST == 2 && KS == 4 ? 3 : KS;
  constexpr int DPP = (PER_SLICE + LOAD_STEPS - 1) / LOAD_STEPS;
  constexpr int EVERY = NM / DPP > 0 ? NM / DPP : 1;
  // every load of the slice gets a slot (NM / EVERY slots per k-step, at most DPP used)
  static_assert((NM / EVERY < DPP ? NM / EVERY : DPP) * LOAD_STEPS >= PER_SLICE,
                "the load slots of a slice must cover its loads");
  // When a k-step has at least as many matrix-core ops as fragment reads (256 x 256 tiles: 8
  // ops, 6 reads), the next k-step's fragments are read one after each op, into the other
  // fragment buffer, in the order that k-step's ops use them; otherwise (shorter tiles) a
  // k-step's reads go out together, two k-steps ahead. 64K-token batch: 1154 vs 1176 us and
  // 1177 vs 1208 us in two same-GPU A/Bs, outputs bitwise equal (the same reads and ops in
  // another order). With one wave per SIMD (4 waves of 128 x 128) it gained nothing: 1250 us.
  constexpr bool kInterleave = NM >= TI + TJ;
  // r-th fragment read of k-step kk: wf[0], xf[0 .. TI-1], then wf[1 .. TJ-1]
  auto frag1 = [&](const char* sp, int kk, int buf, int r) __attribute__((always_inline)) {
    if (r == 0)
      wf[buf][0] = *reinterpret_cast<const bf16x8_t*>(sp + brow0 + pcs[kk]);
    else if (r <= TI)
      xf[buf][r - 1] =
          *reinterpret_cast<const bf16x8_t*>(sp + arow0 + (r - 1) * 32 * RB + pcs[kk]);
    else
      wf[buf][r - TI] =
          *reinterpret_cast<const bf16x8_t*>(sp + brow0 + (r - TI) * 32 * RB + pcs[kk]);
  };
  auto mma = [&](int buf, bool loads, int part, const char* sp) __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < NM; ++x) {
      const int j = x / TI, i = x % TI;
      acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[buf][j], xf[buf][i], acc[j][i],
                                                          0, 0, 0);
      if constexpr (kInterleave) {
        __builtin_amdgcn_sched_barrier(0);
        if (part + 1 < KS && x < TI + TJ) {
          frag1(sp, part + 1, buf ^ 1, x);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      const int q = part * DPP + (x + 1) / EVERY - 1;
      if (loads && (x + 1) % EVERY == 0 && (x + 1) / EVERY <= DPP && q < PER_SLICE) {
        __builtin_amdgcn_sched_barrier(0);
        dma(q);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  const int NK = kt_hi - kt_lo;  // slices of this block
  for (int p = 0; p < NST - 1 && p < NK; ++p) issue(kt_lo + p);
  for (int k = 0; k < NK; ++k) {
    // The next loads' addresses first: they read only the tile's indices (fixed since the
    // tile start), so their LDS round trip at a sub-table's first slice overlaps the wait
    // below instead of delaying the first matrix-core op (64K-token batch: 1138 vs 1154 us
    // and 1197 vs 1210 us in two same-GPU A/Bs, outputs bitwise equal).
    const bool loads = k + NST - 1 < NK;
    if (loads) prep(kt_lo + k + NST - 1);
    // own loads of slice k done (the later slices already issued stay in flight), then all
    // waves meet: slice k is complete in LDS and every wave is past slice k-1, whose buffer
    // the load of slice k+NST-1 reuses.
    const int ahead = NST - 2 < NK - 1 - k ? NST - 2 : NK - 1 - k;
    if (NST >= 5 && ahead >= 3) wait_loads_and_meet<(NST >= 5 ? 3 : 0) * PER_SLICE>();
    else if (NST >= 4 && ahead >= 2) wait_loads_and_meet<(NST >= 4 ? 2 : 0) * PER_SLICE>();
    else if (NST >= 3 && ahead >= 1) wait_loads_and_meet<(NST >= 3 ? 1 : 0) * PER_SLICE>();
    else wait_loads_and_meet<0>();
    const char* sp = lds + (k % NST) * STAGE;
    if (!mult) {
      if (loads) {
#pragma unroll
        for (int q = 0; q < PER_SLICE; ++q) dma(q);
      }
    } else if constexpr (kInterleave) {
      // the first k-step's fragments in the order its ops use them, so the first op waits
      // for two reads rather than five (1131-1132 vs 1137-1146 us, bitwise equal)
#pragma unroll
      for (int r = 0; r < TI + TJ; ++r) frag1(sp, 0, 0, r);
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) mma(kk & 1, loads, kk, sp);
    } else {
      frags(sp, 0, 0);
      if (KS > 1) frags(sp, 1, 1);
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        mma(kk & 1, loads, kk, sp);
        if (kk + 2 < KS) frags(sp, kk + 2, kk & 1);
      }
    }
  }

  // -- epilogue: acc[j][i][4g + q] is output n = n0 + wn*WN + 32j + 8g + 4fk + q of row
  //    m = m0 + wm*WM + 32i + fr. Each wave stages 32 rows at a time (fp32) in its own
  //    part of the LDS pool, then reads them back row-major, VO consecutive outputs per
  //    lane (WN/VO lanes per row), so E_0 is read and the output written in whole lines.
  //    bf16 rows take 8 outputs per lane (16-byte E_0 loads and stores: half the memory
  //    instructions of 4 per lane; 1204 -> 1163 us on the 64K-token batch). fp32 rows and
  //    partial sums take 4 (16-byte stores already; 8 measured no faster with E_0 and 1%
  //    slower without). E_0 add and the 1/(S+1) scale in fp32, one rounding to bf16.
  const uint16_t* __restrict__ E0 = static_cast<const uint16_t*>(a.E0[layer]);
  uint16_t* __restrict__ out = static_cast<uint16_t*>(a.out[layer]);
  char* ep = lds + w * (32 * EP_PITCH);
  constexpr int VO = OM == kOutBf16 ? 8 : 4;   // outputs per lane in the read-back
  constexpr int LPR = WN / VO;          // lanes per output row
  constexpr int RPI = 64 / LPR;         // rows per wave instruction
  constexpr int NIT = 32 / RPI;
  static_assert(64 % LPR == 0 && RPI <= 32, "a wave instruction covers whole rows");
  typedef typename EVec<VO>::type ev_t;
  // Byte offset, in a staged row, of outputs n .. n+3 (n % 4 == 0). With 8 per lane, the
  // first 4 of every group of 8 sit in the row's first half and the other 4 in its second,
  // so the read-back's 16 lanes of one LDS cycle read 256 contiguous bytes (no conflicts)
  // and each staging write stays one 16-byte piece.
  auto spos = [](int n) __attribute__((always_inline)) {
    return VO == 8 ? ((n >> 2) & 1) * (WN * 2) + (n >> 3) * 16 : n * 4;
  };
  const int er = lane / LPR, ec = lane % LPR;
  // the E_0 pieces of all of the wave's output rows are requested before any is used
  // (tokens from LDS, all read first; loads not behind a branch each), so the tile waits for
  // one round trip to memory instead of two (the token, then its row) per 32-row group:
  // 12-20 us less per 64K-token launch; issued before the barrier below, they fly while the
  // waves meet (1094-1101 vs 1102-1107 us, bitwise equal)
  ev_t ev_all[OM != kOutPartial ? TI : 1][NIT];
  if constexpr (OM != kOutPartial) {
    if (mult) {   // load-only waves write no outputs
      const int n = n0 + wn * WN + ec * VO;
      int32_t tka[TI][NIT];
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int it = 0; it < NIT; ++it) tka[i][it] = stok[wm * WM + i * 32 + it * RPI + er];
      if (E0 != nullptr) {
        // rows with an invalid token read row 0 (their outputs are zeros or not written)
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int it = 0; it < NIT; ++it) {
            const int32_t tk = uint32_t(tka[i][it]) < uint32_t(a.V0) ? tka[i][it] : 0;
            ev_all[i][it] = *reinterpret_cast<const ev_t*>(E0 + int64_t(tk) * a.N + n);
          }
      } else {
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int it = 0; it < NIT; ++it) ev_all[i][it] = ev_t{};
      }
    }
  }
  // Every wave is done with the slice buffers before any stages its results there. No slice
  // load is in flight (the last slice waited for all of them), so the waves meet after their
  // LDS reads only; a __syncthreads would also wait for the E_0 requests above.
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (!mult) return;
#pragma unroll
  for (int i = 0; i < TI; ++i) {
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4_t v = {acc[j][i][4 * g + 0], acc[j][i][4 * g + 1], acc[j][i][4 * g + 2],
                     acc[j][i][4 * g + 3]};
        *reinterpret_cast<f32x4_t*>(ep + fr * EP_PITCH + spos(j * 32 + g * 8 + fk * 4)) = v;
      }
    // the wave reads back what its own lanes wrote: wait for the writes, keep the order
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // all loads of the 32 rows first (tok, then E_0), then the stores: a load placed after
    // a store would wait for it, since the compiler cannot rule out aliasing
    const int64_t mrow = m0 + wm * WM + i * 32 + er;
    const int n = n0 + wn * WN + ec * VO;
    if constexpr (OM == kOutPartial) {
      float* pp = static_cast<float*>(a.out[layer]) + int64_t(split) * a.nrows * a.ldo;
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int64_t m = mrow + it * RPI;
        const f32x4_t y = *reinterpret_cast<const f32x4_t*>(ep + (it * RPI + er) * EP_PITCH +
                                                             spos(ec * 4));
        if (m < a.nrows) *reinterpret_cast<f32x4_t*>(pp + m * a.ldo + n) = y;
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      continue;
    }
    // without E_0 (dense products) every row is valid and nothing is added
    const bool has_e0 = E0 != nullptr;
    int32_t tk[NIT];
    ev_t ev[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      tk[it] = stok[wm * WM + i * 32 + it * RPI + er];
      ev[it] = ev_all[i][it];
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int64_t m = mrow + it * RPI;
      const char* row = ep + (it * RPI + er) * EP_PITCH;
      if (m < a.nrows && tk[it] != kSkipRow) {
        const int64_t om = out_row(a, m);
        const bool ok = !has_e0 || uint32_t(tk[it]) < uint32_t(a.V0);
        if constexpr (OM == kOutF32) {
          const f32x4_t y = *reinterpret_cast<const f32x4_t*>(row + spos(ec * 4));
          const f32x4_t res = ok ? f32x4_t{(y[0] + bf16_to_f32(ev[it].x & 0xffffu)) * a.inv,
                                           (y[1] + bf16_to_f32(ev[it].x >> 16)) * a.inv,
                                           (y[2] + bf16_to_f32(ev[it].y & 0xffffu)) * a.inv,
                                           (y[3] + bf16_to_f32(ev[it].y >> 16)) * a.inv}
                                 : f32x4_t{0.f, 0.f, 0.f, 0.f};
          *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(out) + om * a.ldo + n) = res;
        } else {
          const f32x4_t ya = *reinterpret_cast<const f32x4_t*>(row + spos(ec * 8));
          const f32x4_t yb = *reinterpret_cast<const f32x4_t*>(row + spos(ec * 8 + 4));
          u32x4_t res = {0u, 0u, 0u, 0u};
          if (ok) {
#pragma unroll
            for (int h = 0; h < 4; ++h) {
              const f32x4_t& y = h < 2 ? ya : yb;
              const uint32_t e = ev[it][h];
              const float lo = (y[(h & 1) * 2] + bf16_to_f32(e & 0xffffu)) * a.inv;
              const float hi = (y[(h & 1) * 2 + 1] + bf16_to_f32(e >> 16)) * a.inv;
              res[h] = f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
            }
          }
          __builtin_nontemporal_store(res, reinterpret_cast<u32x4_t*>(out + om * a.ldo + n));
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // reads done before the next writes
  }
}

// ------------------------------------------------------------------ generic path
// Any dtype and shape (used for fp32 and for bf16 shapes the tiles above do not cover):
// 64 x 64 output tiles, 16-deep slices gathered element by element into LDS, fp32 FMA.

template <typename T> __device__ __forceinline__ float ld(const T* p);
template <> __device__ __forceinline__ float ld<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld<uint16_t>(const uint16_t* p) {
  return bf16_to_f32(*p);
}
template <typename T> __device__ __forceinline__ void st(T* p, float v);
template <> __device__ __forceinline__ void st<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void st<uint16_t>(uint16_t* p, float v) {
  *p = uint16_t(f32_to_bf16_rne(v));
}

template <typename T, typename TO>
__global__ __launch_bounds__(256) void proj_generic_kernel(const ProjArgs a) {
  __shared__ float As[16][64 + 4];
  __shared__ float Bs[16][64 + 4];
  __shared__ const T* Etab[NGRAM_MAX_SUBTABLES];
  __shared__ uint32_t Vtab[NGRAM_MAX_SUBTABLES];
  const int t = threadIdx.x, tx = t & 15, ty = t >> 4;
  const int layer = blockIdx.z;
  if (t < a.S) {
    Etab[t] = static_cast<const T*>(a.E[layer * a.S + t]);
    Vtab[t] = a.Vm1[t];
  }
  const int64_t m0 = int64_t(blockIdx.x) * 64;
  const int n0 = blockIdx.y * 64;
  const T* __restrict__ W = static_cast<const T*>(a.W[layer]);
  float acc[4][4] = {};
  __syncthreads();
  for (int k0 = 0; k0 < a.K; k0 += 16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int lin = t + 256 * e, r = lin >> 4, kk = lin & 15;
      const int k = k0 + kk;
      const int64_t m = m0 + r;
      float v = 0.f;
      if (m < a.nrows && k < a.K) {
        const int s = k / a.d, c = k - s * a.d;
        const uint32_t id = min(uint32_t(a.idx[m * a.S + s]), Vtab[s]);
        v = ld<T>(Etab[s] + int64_t(id) * a.d + c);
      }
      As[kk][r] = v;
      const int n = n0 + r;
      Bs[kk][r] = (n < a.N && k < a.K) ? ld<T>(W + int64_t(n) * a.ldb + k) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += As[kk][ty + 16 * i] * Bs[kk][tx + 16 * j];
    __syncthreads();
  }
  const T* __restrict__ E0 = static_cast<const T*>(a.E0[layer]);
  TO* __restrict__ out = static_cast<TO*>(a.out[layer]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty + 16 * i;
    if (m >= a.nrows) continue;
    const bool has_e0 = E0 != nullptr;          // without E_0 every row is valid
    const int32_t tk = has_e0 ? a.tok[m] : 0;
    if (tk == kSkipRow) continue;
    const int64_t om = out_row(a, m);
    const bool ok = !has_e0 || uint32_t(tk) < uint32_t(a.V0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx + 16 * j;
      if (n >= a.N) continue;
      const float e0 = has_e0 && ok ? ld<T>(E0 + int64_t(tk) * a.N + n) : 0.f;
      const float y = ok ? (acc[i][j] + e0) * a.inv : 0.f;
      st<TO>(out + om * a.ldo + n, y);
    }
  }
}

// N = 1: no sub-tables, e = E_0(t) (then any output factor or normalisation).
// Plain rows: 16-byte vectors copied, one per thread.
__global__ __launch_bounds__(256) void e0_lookup_kernel(const ProjArgs a, int32_t row_bytes) {
  const int64_t cpr = row_bytes / 16;
  const int64_t item = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (item >= a.nrows * cpr) return;
  const int64_t r = item / cpr, c = item - r * cpr;
  const int32_t tk = a.tok[r];
  if (tk == kSkipRow) return;
  const int layer = blockIdx.z;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (uint32_t(tk) < uint32_t(a.V0))
    v = reinterpret_cast<const uint4*>(static_cast<const char*>(a.E0[layer]) +
                                       int64_t(tk) * row_bytes)[c];
  reinterpret_cast<uint4*>(static_cast<char*>(a.out[layer]) + out_row(a, r) * row_bytes)[c] = v;
}

// Scaled (or fp32-output) rows: one element per thread, fp32 product, one rounding.
template <typename T, typename TO>
__global__ __launch_bounds__(256) void e0_scaled_kernel(const ProjArgs a) {
  const int64_t item = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (item >= a.nrows * a.N) return;
  const int64_t r = item / a.N;
  const int32_t tk = a.tok[r];
  if (tk == kSkipRow) return;
  const int layer = blockIdx.z;
  float v = 0.f;
  if (uint32_t(tk) < uint32_t(a.V0))
    v = ld<T>(static_cast<const T*>(a.E0[layer]) + int64_t(tk) * a.N + (item - r * a.N)) *
        a.inv;
  st<TO>(static_cast<TO*>(a.out[layer]) + out_row(a, r) * a.N + (item - r * a.N), v);
}

// out[m, n] += f * sum_s part[s, m, n]: the split partial sums added in split order (the
// same order every run), 4 outputs per thread.
__global__ __launch_bounds__(256) void accum_partials_kernel(const float* __restrict__ part,
                                                             int32_t splits, int64_t M,
                                                             int64_t ldo, int32_t N, float f,
                                                             float* __restrict__ out) {
  const int64_t q = int64_t(blockIdx.x) * 256 + threadIdx.x;   // group of 4 outputs
  const int64_t per_row = N / 4;
  if (q >= M * per_row) return;
  const int64_t m = q / per_row;
  const int64_t off = m * ldo + (q - m * per_row) * 4;
  f32x4_t y = *reinterpret_cast<const f32x4_t*>(part + off);
  for (int s = 1; s < splits; ++s)
    y += *reinterpret_cast<const f32x4_t*>(part + int64_t(s) * M * ldo + off);
  f32x4_t* o = reinterpret_cast<f32x4_t*>(out + off);
  *o = *o + y * f;
}

template <int BM, int OM, int BN = kBN>
hipError_t run_mfma(ProjArgs a, int64_t nrows, int osz, hipStream_t st) {
  // at most 2^20 row tiles per launch keeps the tile numbering in 32-bit ints (partial sums
  // are laid out per launch, so they take one launch)
  const int64_t chunk = int64_t(BM) << 20;
  if ((OM == kOutPartial || a.row_group != 0) && nrows > chunk) return hipErrorInvalidValue;
  const int32_t* idx = a.idx;
  const int32_t* tok = a.tok;
  char* out[kMaxLaunchLayers];
  for (int l = 0; l < a.layers; ++l) out[l] = static_cast<char*>(a.out[l]);
  for (int64_t r0 = 0; r0 < nrows; r0 += chunk) {
    const int64_t n = nrows - r0 < chunk ? nrows - r0 : chunk;
    a.idx = idx + r0 * a.S;
    a.tok = tok ? tok + r0 : nullptr;
    for (int l = 0; l < a.layers; ++l) a.out[l] = out[l] + r0 * a.ldo * osz;
    a.nrows = n;
    a.tiles_m = int32_t((n + BM - 1) / BM);
    a.tiles_n = a.N / BN;
    const int64_t blocks = int64_t(a.tiles_m) * a.tiles_n * (OM == kOutPartial ? a.splits : 1);
    hipLaunchKernelGGL((proj_mfma_kernel<BM, OM, BN>), dim3(unsigned(blocks), 1, unsigned(a.layers)),
                       dim3(WaveGrid<BM, BN>::NW * 64), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Tile shape of the matrix-core kernel for the product `a` over nrows rows with output mode
// om, or bm = 0: the generic path (or, for partial sums, no path).
struct Route {
  int bm, bn;
};
// Compute units of the current device (the number of blocks one round of tiles occupies).
int device_cus() {
  static std::atomic<int> cached{0};
  int n = cached.load(std::memory_order_relaxed);
  if (n > 0) return n;
  int dev = 0;
  n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    n = 256;
  cached.store(n, std::memory_order_relaxed);
  return n;
}

Route mfma_route(const ProjArgs& a, int32_t dtype, int om, int64_t nrows) {
  if (!(dtype == NGRAM_BF16 && a.N % kBN == 0 && a.d % kBK == 0 && a.K % kBK == 0))
    return {0, 0};
  // A tile keeps its rows' hash indices (and E_0 tokens) in LDS.
  const int per_row = a.S + (om != kOutPartial ? 1 : 0);   // int32 per row
  const bool f256 = 256 * per_row * 4 <= IdxLds<256>::bytes;
  const bool f128 = 128 * per_row * 4 <= IdxLds<128>::bytes;
  const bool f64 = 64 * per_row * 4 <= IdxLds<64>::bytes;
  if (om == kOutPartial) {
    // split contractions (the backward's dW): 256-row tiles once the ranges give 512 blocks
    const int64_t tiles_n = a.N / kBN;
    const bool big = ((nrows + 255) / 256) * tiles_n * a.splits >= 512;
    const bool mid = ((nrows + 127) / 128) * tiles_n * a.splits >= 256;
    const int bm = big && f256 ? 256 : (big || mid) && f128 ? 128 : f64 ? 64 : f128 ? 128
                 : f256 ? 256 : 0;
    return {bm, kBN};
  }
  // The loads into LDS bound these kernels, and each CU takes its blocks one after another,
  // so pick the tile whose busiest CU loads the fewest bytes: rounds of blocks over the CUs
  // times (BM + BN) rows of the contraction per block. Larger tiles win ties. (Each output's
  // sum order does not depend on the tile, so the choice never changes a bit.) The 30B
  // layer's shapes: 64K rows -> 256 x 256 (12 rounds); 1280 decode rows -> 128 x 128 (240
  // blocks, one round); 256 draft-phase rows -> 64 x 64 (192 blocks of 0.79 MB, where 96
  // blocks of 64 x 128 loaded 1.18 MB each: 24.4 vs 30.1 us per call, since the four
  // load-only waves keep a CU's load rate that of eight); 16K rows of D = 1024 -> 256 x 256
  // (one round of 256 blocks: 1 MB per CU, where two rounds of 128 x 256 took 1.5 MB).
  static constexpr int kCand[6][2] = {{256, 256}, {128, 256}, {64, 256}, {128, 128}, {64, 128},
                                      {64, 64}};
  const int64_t cus = device_cus();
  Route best{0, 0};
  int64_t best_cost = 0;
  for (const auto& c : kCand) {
    const bool fits = c[0] == 256 ? f256 : c[0] == 128 ? f128 : f64;
    if (!fits || a.N % c[1] != 0) continue;
    const int64_t blocks = ((nrows + c[0] - 1) / c[0]) * (a.N / c[1]) * a.layers;
    const int64_t cost = ((blocks + cus - 1) / cus) * (c[0] + c[1]);
    if (best.bm == 0 || cost < best_cost) {
      best = {c[0], c[1]};
      best_cost = cost;
    }
  }
  return best;
}

template <int OM>
hipError_t dispatch(Route r, const ProjArgs& a, int64_t nrows, int osz, hipStream_t st) {
  if (r.bm == 256) return run_mfma<256, OM>(a, nrows, osz, st);
  if (r.bm == 128 && r.bn == kBN) return run_mfma<128, OM>(a, nrows, osz, st);
  if (r.bm == 64 && r.bn == kBN) return run_mfma<64, OM>(a, nrows, osz, st);
  if constexpr (OM != kOutPartial) {
    if (r.bm == 128 && r.bn == 128) return run_mfma<128, OM, 128>(a, nrows, osz, st);
    if (r.bm == 64 && r.bn == 128) return run_mfma<64, OM, 128>(a, nrows, osz, st);
    if (r.bm == 64 && r.bn == 64) return run_mfma<64, OM, 64>(a, nrows, osz, st);
  }
  return hipErrorInvalidValue;
}

// Runs the product `a` describes (E/idx/S/d, K, N, ldb, ldo, E0/tok, inv) over nrows rows.
// om: kOutBf16 (config dtype), kOutF32, or kOutPartial (a.splits ranges, matrix cores only).
hipError_t run_product(ProjArgs a, int32_t dtype, int om, int64_t nrows, hipStream_t st) {
  const int osz = om == kOutBf16 ? (dtype == NGRAM_F32 ? 4 : 2) : 4;
  const Route r = mfma_route(a, dtype, om, nrows);
  if (r.bm != 0) {
    if (om == kOutPartial) return dispatch<kOutPartial>(r, a, nrows, osz, st);
    if (om == kOutF32) return dispatch<kOutF32>(r, a, nrows, osz, st);
    return dispatch<kOutBf16>(r, a, nrows, osz, st);
  }
  // no tile keeps this many indices, or not a matrix-core shape: the generic path below
  if (om == kOutPartial) return hipErrorInvalidValue;   // callers use kOutF32 here
  const unsigned gy = unsigned((a.N + 63) / 64);
  const int32_t* idx = a.idx;
  const int32_t* tok = a.tok;
  if (a.row_group != 0 && nrows > (int64_t(1) << 30)) return hipErrorInvalidValue;
  for (int64_t r0 = 0; r0 < nrows; r0 += (int64_t(1) << 30)) {
    ProjArgs b = a;
    const int64_t n = nrows - r0 < (int64_t(1) << 30) ? nrows - r0 : (int64_t(1) << 30);
    b.idx = idx + r0 * a.S;
    b.tok = tok ? tok + r0 : nullptr;
    for (int l = 0; l < a.layers; ++l) b.out[l] = static_cast<char*>(a.out[l]) + r0 * a.ldo * osz;
    b.nrows = n;
    const dim3 grid(unsigned((n + 63) / 64), gy, unsigned(a.layers));
    if (dtype == NGRAM_F32)
      hipLaunchKernelGGL((proj_generic_kernel<float, float>), grid, dim3(256), 0, st, b);
    else if (om == kOutF32)
      hipLaunchKernelGGL((proj_generic_kernel<uint16_t, float>), grid, dim3(256), 0, st, b);
    else
      hipLaunchKernelGGL((proj_generic_kernel<uint16_t, uint16_t>), grid, dim3(256), 0, st, b);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// A dense product A [M, K] x B [N, K]^T as ProjArgs: A is one "sub-table" of M rows of K
// values read through identity indices, no E_0.
ProjArgs dense_args(const void* A, int64_t M, const void* B, int32_t N, int32_t K,
                    const int32_t* ident, void* out, int64_t ldo, float inv) {
  ProjArgs a{};
  a.E[0] = A;
  a.Vm1[0] = uint32_t(M - 1);
  a.idx = ident;
  a.tok = nullptr;
  a.E0[0] = nullptr;
  a.W[0] = B;
  a.out[0] = out;
  a.layers = 1;
  a.nrows = M;
  a.ldb = K;
  a.ldo = ldo;
  a.K = K;
  a.N = N;
  a.S = 1;
  a.d = K;
  a.V0 = 0;
  a.inv = inv;
  a.splits = 1;
  return a;
}

}  // namespace

hipError_t launch_project_layers(const LayerDesc& L, const LayerParams* layers, int32_t nlayers,
                                 const int32_t* idx, const int32_t* tok, int64_t nrows,
                                 bool f32out, const RowMap& map, hipStream_t st) {
  if (nrows <= 0 || nlayers <= 0) return hipSuccess;
  if (L.form == NGRAM_FORM_BASIC && L.S > 0) {
    for (int l = 0; l < nlayers; ++l) {
      const hipError_t e = launch_basic(L, layers[l].E0, layers[l].E, idx, tok, nrows,
                                        layers[l].out, f32out, map, st);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  ProjArgs a{};
  for (int s = 0; s < L.S; ++s) a.Vm1[s] = L.V[s] - 1u;
  a.idx = idx;
  a.tok = tok;
  a.nrows = nrows;
  a.K = L.D;
  a.N = L.D;
  a.ldb = L.D;
  a.ldo = L.D;
  a.S = L.S;
  a.d = L.d;
  a.V0 = L.V0;
  a.inv = L.scale / float(L.S + 1);
  a.splits = 1;
  a.row_group = map.group;
  a.row_stride = map.stride;
  a.row_off = map.off;
  const int osz = f32out ? 4 : L.esz;   // bytes per output element
  // layers per launch: as many as the kernel arguments hold
  const int per = std::min<int>(kMaxLaunchLayers, L.S > 0 ? kMaxLaunchTables / L.S
                                                           : kMaxLaunchLayers);
  for (int l0 = 0; l0 < nlayers; l0 += per) {
    a.layers = std::min(per, nlayers - l0);
    for (int l = 0; l < a.layers; ++l) {
      const LayerParams& p = layers[l0 + l];
      for (int s = 0; s < L.S; ++s) a.E[l * L.S + s] = p.E[s];
      a.E0[l] = p.E0;
      a.W[l] = p.W;
      a.out[l] = p.out;
    }
    hipError_t e = hipSuccess;
    if (L.S > 0) {
      e = run_product(a, L.dtype, f32out ? kOutF32 : kOutBf16, nrows, st);
    } else if (!f32out && L.scale == 1.0f) {
      const int32_t row_bytes = L.D * L.esz;
      const int64_t items = nrows * (row_bytes / 16);
      hipLaunchKernelGGL(e0_lookup_kernel, dim3(unsigned((items + 255) / 256), 1,
                                                unsigned(a.layers)),
                         dim3(256), 0, st, a, row_bytes);
      e = hipGetLastError();
    } else {
      // at most 2^30 rows x D elements per launch keeps the grid in range
      const int64_t rows_per = std::max<int64_t>(1, (int64_t(1) << 38) / L.D);
      if (map.group != 0 && nrows > rows_per) return hipErrorInvalidValue;
      for (int64_t r0 = 0; r0 < nrows && e == hipSuccess; r0 += rows_per) {
        ProjArgs b = a;
        b.nrows = std::min(rows_per, nrows - r0);
        b.tok = tok + r0;
        for (int l = 0; l < a.layers; ++l)
          b.out[l] = static_cast<char*>(a.out[l]) + r0 * L.D * osz;
        const dim3 grid(unsigned((b.nrows * L.D + 255) / 256), 1, unsigned(a.layers));
        if (L.dtype == NGRAM_F32)
          hipLaunchKernelGGL((e0_scaled_kernel<float, float>), grid, dim3(256), 0, st, b);
        else if (f32out)
          hipLaunchKernelGGL((e0_scaled_kernel<uint16_t, float>), grid, dim3(256), 0, st, b);
        else
          hipLaunchKernelGGL((e0_scaled_kernel<uint16_t, uint16_t>), grid, dim3(256), 0, st, b);
        e = hipGetLastError();
      }
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_project(const LayerDesc& L, const void* E0, const void* const* E,
                          const void* W, const int32_t* idx, const int32_t* tok,
                          int64_t nrows, void* out, bool f32out, const RowMap& map,
                          hipStream_t st) {
  const LayerParams p{E0, E, W, out};
  return launch_project_layers(L, &p, 1, idx, tok, nrows, f32out, map, st);
}

hipError_t launch_dense_product(const LayerDesc& L, const void* A, int64_t M, const void* B,
                                int32_t N, int32_t K, const int32_t* ident, float* out,
                                int64_t ldo, float inv, bool accumulate, float* part,
                                int32_t splits, hipStream_t st) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (!accumulate)
    return run_product(dense_args(A, M, B, N, K, ident, out, ldo, inv), L.dtype, kOutF32, M, st);
  // accumulate: partial sums into `part`, then out += inv * (their sum in split order)
  const bool mfma = L.dtype == NGRAM_BF16 && N % kBN == 0 && K % kBK == 0;
  hipError_t e;
  float f = inv;
  if (mfma) {
    ProjArgs a = dense_args(A, M, B, N, K, ident, part, ldo, 1.0f);
    a.splits = splits < 1 ? 1 : splits;
    e = run_product(a, L.dtype, kOutPartial, M, st);
  } else {
    splits = 1;
    e = run_product(dense_args(A, M, B, N, K, ident, part, ldo, inv), L.dtype, kOutF32, M, st);
    f = 1.0f;
  }
  if (e != hipSuccess) return e;
  const int64_t groups = M * (N / 4);
  hipLaunchKernelGGL(accum_partials_kernel, dim3(unsigned((groups + 255) / 256)), dim3(256), 0,
                     st, part, mfma ? splits : 1, M, ldo, N, f, out);
  return hipGetLastError();
}

}  // namespace ngram
