// Backward of the layer (training): gradients of
//   e_i = c ( E_0(t_i) + sum_s W_s E_s(h_{i,s}) ),  c = factor / ((N-1)K + 1),
// the final form of section A2 of the deep-notes page on "Scaling Embeddings Outperforms
// Scaling Experts in Language Models" (the pages train the layer but give no backward; these
// are its plain derivatives). For the upstream gradient dout [T, D]:
//   dW   += c dout^T G               (G [T, D] the gathered rows; the stacked W's layout)
//   dE_s[r] += c sum_{i: h_{i,s} = r} (dout W)[i, s*d : (s+1)*d]
//   dE_0[t] += c sum_{i: t_i = t} dout_i
// Positions whose token is outside [0, V0) produced zero rows in the forward and contribute
// nothing here.
//
// Products run on the projection's kernels (launch_dense_product): dG = c dout W through
// the transposed W, dW through dout^T and G^T padded to a multiple of 64 tokens (the
// contraction), split into ranges whose fp32 partial sums are added in a fixed order.
// The scatter-adds are deterministic, with no atomics: (key, position) pairs are sorted
// with a stable LSD radix sort (8-bit digits; key = token, or sub-table s and row r), then
// each run of equal keys is summed in position order by one owner: runs inside a chunk of
// kChunk sorted entries directly, runs that cross chunks by the chunk where they start,
// which adds the later chunks' partial sums in order.
#include <algorithm>

#include "bf16.h"
#include "kernels.h"

namespace ngram {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <typename T> __device__ __forceinline__ float ldf(const T* p);
template <> __device__ __forceinline__ float ldf<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ldf<uint16_t>(const uint16_t* p) {
  return bf16_to_f32(*p);
}

constexpr int kTile = 64;           // transpose tile edge
constexpr int kChunkWide = 64;      // E_0's chunk of sorted entries (kChunk: sub-tables)
constexpr int kSortThreads = 256;
constexpr int kSortRounds = kSortTile / kSortThreads;   // keys per thread per sort tile

__global__ __launch_bounds__(256) void iota_kernel(int32_t* p, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) p[i] = int32_t(i);
}

// XT[c, r] = X[r, c] for r < rows (and 0 for rows <= r < ldt): X [rows, cols] row-major,
// XT [cols, ldt]. When tok is not null, rows r whose tok[r] is outside [0, V0) read as 0.
template <typename T>
__global__ __launch_bounds__(256) void transpose_pad_kernel(const T* __restrict__ X,
                                                            int64_t rows, int32_t cols,
                                                            const int32_t* __restrict__ tok,
                                                            int32_t V0, T* __restrict__ XT,
                                                            int64_t ldt) {
  __shared__ T tile[kTile][kTile + 2];
  const int64_t r0 = int64_t(blockIdx.x) * kTile;
  const int c0 = blockIdx.y * kTile;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < kTile; i += 4) {
    const int64_t r = r0 + i;
    const int c = c0 + tx;
    T v = T(0);
    if (r < rows && c < cols && (tok == nullptr || uint32_t(tok[r]) < uint32_t(V0)))
      v = X[r * cols + c];
    tile[i][tx] = v;
  }
  __syncthreads();
  for (int j = ty; j < kTile; j += 4) {
    const int c = c0 + j;
    const int64_t r = r0 + tx;
    if (c < cols && r < ldt) XT[int64_t(c) * ldt + r] = tile[tx][j];
  }
}

// 16-bit elements, 16-byte vectors: the same transposes with each thread moving 8 elements
// per access (64 x 64 tiles; the LDS pitch of 72 elements keeps the column reads spread
// over the banks). `src_row(r)` gives the tile's first column in source row r (null past
// the last row) and whether the row is kept (else it reads as zeros). A thread asks for both
// of its rows' index data first, then loads both rows, then drops the rows not kept: one or
// two memory round trips instead of up to three per row.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kPitch = kTile + 8;

struct SrcRow {
  const uint16_t* p;   // the tile's first column in the source row; null past the last row
  bool keep;           // false: the row reads as zeros
};

template <typename RowFn>
__device__ __forceinline__ void transpose_tile16(uint16_t (*tile)[kPitch], RowFn src_row,
                                                 int c0, uint16_t* XT, int64_t ldt, int cols,
                                                 int64_t r0) {
  const int t = threadIdx.x, q = t % 8;
  SrcRow sr[2];                                  // 512 vectors of 8 elements per tile
#pragma unroll
  for (int k = 0; k < 2; ++k) sr[k] = src_row(t / 8 + 32 * k);
  u32x4_t v[2];
#pragma unroll
  for (int k = 0; k < 2; ++k)
    v[k] = sr[k].p != nullptr ? *reinterpret_cast<const u32x4_t*>(sr[k].p + q * 8)
                              : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
  for (int k = 0; k < 2; ++k)
    *reinterpret_cast<u32x4_t*>(&tile[t / 8 + 32 * k][q * 8]) =
        sr[k].keep ? v[k] : u32x4_t{0u, 0u, 0u, 0u};
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = t / 8 + 32 * k, q = t % 8;    // output row c0 + c, tokens r0 + 8q ..
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = uint32_t(tile[q * 8 + 2 * j][c]) | (uint32_t(tile[q * 8 + 2 * j + 1][c]) << 16);
    if (c0 + c < cols && r0 + q * 8 < ldt)
      *reinterpret_cast<u32x4_t*>(XT + int64_t(c0 + c) * ldt + r0 + q * 8) =
          u32x4_t{w[0], w[1], w[2], w[3]};
  }
}

// dout^T for bf16 (cols % 64 == 0, ldt % 64 == 0)
__global__ __launch_bounds__(256) void transpose_pad16_kernel(const uint16_t* __restrict__ X,
                                                              int64_t rows, int32_t cols,
                                                              const int32_t* __restrict__ tok,
                                                              int32_t V0,
                                                              uint16_t* __restrict__ XT,
                                                              int64_t ldt) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kTile][kPitch];
  const int64_t r0 = int64_t(blockIdx.x) * kTile;
  const int c0 = blockIdx.y * kTile;
  auto src_row = [&](int r) -> SrcRow {
    const int64_t rr = r0 + r;
    if (rr >= rows) return SrcRow{nullptr, false};
    // the row's address does not depend on its token: both loads fly together
    return SrcRow{X + rr * cols + c0, tok == nullptr || uint32_t(tok[rr]) < uint32_t(V0)};
  };
  transpose_tile16(tile, src_row, c0, XT, ldt, cols, r0);
}

struct GatherTArgs {
  const void* E[NGRAM_MAX_SUBTABLES];
  uint32_t Vm1[NGRAM_MAX_SUBTABLES];
  const int32_t* idx;   // [rows, S]
  const int32_t* tok;   // [rows]
  void* GT;             // [D, ldt]
  int64_t rows, ldt;
  int32_t S, d, D, V0;
};

// GT[s*d + c, i] = E_s[idx[i, s], c]: the gathered rows, transposed (tokens along the
// contraction); 0 for padding positions and for positions with an invalid token.
template <typename T>
__global__ __launch_bounds__(256) void gather_transpose_kernel(const GatherTArgs a) {
  __shared__ T tile[kTile][kTile + 2];
  const int64_t r0 = int64_t(blockIdx.x) * kTile;
  const int c0 = blockIdx.y * kTile;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < kTile; i += 4) {
    const int64_t r = r0 + i;
    const int c = c0 + tx;
    T v = T(0);
    if (r < a.rows && c < a.D && uint32_t(a.tok[r]) < uint32_t(a.V0)) {
      const int s = c / a.d, cc = c - s * a.d;
      const uint32_t id = min(uint32_t(a.idx[r * a.S + s]), a.Vm1[s]);
      v = static_cast<const T*>(a.E[s])[int64_t(id) * a.d + cc];
    }
    tile[i][tx] = v;
  }
  __syncthreads();
  T* GT = static_cast<T*>(a.GT);
  for (int j = ty; j < kTile; j += 4) {
    const int c = c0 + j;
    const int64_t r = r0 + tx;
    if (c < a.D && r < a.ldt) GT[int64_t(c) * a.ldt + r] = tile[tx][j];
  }
}

// G^T for bf16 when every 64-column tile lies in one sub-table (d % 64 == 0)
__global__ __launch_bounds__(256) void gather_transpose16_kernel(const GatherTArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kTile][kPitch];
  const int64_t r0 = int64_t(blockIdx.x) * kTile;
  const int c0 = blockIdx.y * kTile;
  const int s = c0 / a.d;
  const uint16_t* E = static_cast<const uint16_t*>(a.E[s]);
  auto src_row = [&](int r) -> SrcRow {
    const int64_t rr = r0 + r;
    if (rr >= a.rows) return SrcRow{nullptr, false};
    // token and index together (the index is clamped into the table, so the row load is in
    // bounds whatever the token)
    const int32_t tk = a.tok[rr];
    const uint32_t id = min(uint32_t(a.idx[rr * a.S + s]), a.Vm1[s]);
    return SrcRow{E + int64_t(id) * a.d + (c0 - s * a.d), uint32_t(tk) < uint32_t(a.V0)};
  };
  transpose_tile16(tile, src_row, c0, static_cast<uint16_t*>(a.GT), a.ldt, a.D, r0);
}

// Sort inputs. E_0: key = token, value = position. Sub-tables: pair p = i*S + s has key
// (s << row_bits) | idx[i, s] and value i (row_bits: enough for the largest table's rows, so
// the keys take as few sort passes as they can). Invalid positions get the key `sentinel`
// (sorted last).
__global__ __launch_bounds__(256) void keys_tokens_kernel(const int32_t* __restrict__ tok,
                                                          int64_t n, int32_t V0,
                                                          uint64_t sentinel,
                                                          uint64_t* __restrict__ keys,
                                                          uint32_t* __restrict__ vals) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  const int32_t t = tok[i];
  keys[i] = uint32_t(t) < uint32_t(V0) ? uint64_t(t) : sentinel;
  vals[i] = uint32_t(i);
}

// (the indices come from the hash kernel, so they lie in [0, V_s))
__global__ __launch_bounds__(256) void keys_subtables_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ tok, int64_t rows, int32_t S,
    int32_t V0, int32_t row_bits, uint64_t sentinel, uint64_t* __restrict__ keys,
    uint32_t* __restrict__ vals) {
  const int64_t p = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (p >= rows * S) return;
  const int64_t i = p / S;
  const int s = int(p - i * S);
  keys[p] = uint32_t(tok[i]) < uint32_t(V0) ? (uint64_t(s) << row_bits) | uint32_t(idx[p])
                                            : sentinel;
  vals[p] = uint32_t(i);
}

// ---- stable LSD radix sort, 8-bit digits -------------------------------------------
// hist[digit * nblocks + b] = count of `digit` in tile b.
__global__ __launch_bounds__(kSortThreads) void radix_hist_kernel(const uint64_t* keys,
                                                                  int64_t n, int shift,
                                                                  uint32_t* hist) {
  __shared__ uint32_t h[256];
  const int t = threadIdx.x;
  h[t] = 0;
  __syncthreads();
  const int64_t base = int64_t(blockIdx.x) * kSortTile;
  for (int k = 0; k < kSortRounds; ++k) {
    const int64_t i = base + int64_t(k) * kSortThreads + t;
    if (i < n) atomicAdd(&h[(keys[i] >> shift) & 255u], 1u);
  }
  __syncthreads();
  hist[int64_t(t) * gridDim.x + blockIdx.x] = h[t];
}

// In-place exclusive prefix sum of the m digit-major counts hist[digit * nblocks + b], in
// two launches over tiles of kScanTile counts: the tile totals, then each tile scanned with
// the sum of the tiles before it (read by every block: there are few tiles).
constexpr int kScanTile = 1024;

__global__ __launch_bounds__(256) void scan_totals_kernel(const uint32_t* v, int64_t m,
                                                          uint32_t* totals) {
  __shared__ uint32_t part[256];
  const int t = threadIdx.x;
  const int64_t base = int64_t(blockIdx.x) * kScanTile;
  uint32_t s = 0;
#pragma unroll
  for (int k = 0; k < kScanTile / 256; ++k) {
    const int64_t i = base + k * 256 + t;
    if (i < m) s += v[i];
  }
  part[t] = s;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (t < off) part[t] += part[t + off];
    __syncthreads();
  }
  if (t == 0) totals[blockIdx.x] = part[0];
}

__global__ __launch_bounds__(256) void scan_apply_kernel(uint32_t* v, int64_t m,
                                                         const uint32_t* totals) {
  __shared__ uint32_t part[256];
  const int t = threadIdx.x;
  // sum of the earlier tiles
  uint32_t before = 0;
  for (int64_t b = t; b < blockIdx.x; b += 256) before += totals[b];
  part[t] = before;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (t < off) part[t] += part[t + off];
    __syncthreads();
  }
  const uint32_t carry = part[0];
  __syncthreads();
  // this tile: thread t holds 4 consecutive counts
  constexpr int PER = kScanTile / 256;
  const int64_t base = int64_t(blockIdx.x) * kScanTile + int64_t(t) * PER;
  uint32_t x[PER], s = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    x[k] = base + k < m ? v[base + k] : 0u;
    s += x[k];
  }
  part[t] = s;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {                // inclusive scan of thread sums
    const uint32_t y = t >= off ? part[t - off] : 0u;
    __syncthreads();
    part[t] += y;
    __syncthreads();
  }
  uint32_t run = carry + part[t] - s;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    if (base + k < m) v[base + k] = run;
    run += x[k];
  }
}

// Scatter of tile b in index order: keys of equal digit keep their order (stable). Each
// round takes 256 consecutive keys; a key's rank among equal digits in its wave comes from
// 8 ballots, the waves before it and the earlier rounds from counters in LDS.
__global__ __launch_bounds__(kSortThreads) void radix_scatter_kernel(
    const uint64_t* __restrict__ kin, const uint32_t* __restrict__ vin, int64_t n, int shift,
    const uint32_t* __restrict__ offs, uint64_t* __restrict__ kout,
    uint32_t* __restrict__ vout) {
  __shared__ uint32_t base[256];       // global position of this tile's first key per digit
  __shared__ uint32_t wcount[4][256];  // keys per digit in each wave of the current round
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  base[t] = offs[int64_t(t) * gridDim.x + blockIdx.x];
  for (int q = 0; q < 4; ++q) wcount[q][t] = 0;
  __syncthreads();
  const uint64_t lt = (uint64_t(1) << lane) - 1;
  const int64_t tile0 = int64_t(blockIdx.x) * kSortTile;
  for (int k = 0; k < kSortRounds; ++k) {
    const int64_t i = tile0 + int64_t(k) * kSortThreads + t;
    const bool valid = i < n;
    const uint64_t key = valid ? kin[i] : 0;
    const uint32_t dig = uint32_t(key >> shift) & 255u;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint64_t m = __ballot(valid && ((dig >> b) & 1u));
      peers &= ((dig >> b) & 1u) ? m : ~m;
    }
    const uint32_t rank = __popcll(peers & lt);
    if (valid && rank == 0) wcount[wv][dig] = __popcll(peers);
    __syncthreads();
    if (valid) {
      uint32_t pos = base[dig] + rank;
      for (int q = 0; q < wv; ++q) pos += wcount[q][dig];
      kout[pos] = key;
      vout[pos] = vin[i];
    }
    __syncthreads();
    base[t] += wcount[0][t] + wcount[1][t] + wcount[2][t] + wcount[3][t];
    for (int q = 0; q < 4; ++q) wcount[q][t] = 0;
    __syncthreads();
  }
}

// ---- segmented sums of sorted (key, position) runs --------------------------------------
struct SegArgs {
  float* dst[NGRAM_MAX_SUBTABLES];   // gradient table of each key class (E_0: dst[0])
  const uint64_t* keys;              // sorted
  const uint32_t* vals;              // positions, in the keys' order
  const void* src;                   // rows summed: [rows, ld_src] (fp32 or config dtype)
  float* head;                       // [nchunks, width]: sum of the run a chunk starts in
  float* tail;                       // [nchunks, width]: sum of the run a chunk ends in
  uint32_t* owners;                  // [1 + nchunks]: count, then chunks that own a run
                                     // continuing past their end (any order)
  int64_t n, nchunks, ld_src;
  uint64_t sentinel;
  int32_t width;                     // gradient row width (D for E_0, d for sub-tables)
  int32_t chunk;                     // sorted entries per chunk
  int32_t by_table;                  // 1: key = (s << row_bits) | r, source columns s*col_step...
  int32_t row_bits;
  int32_t col_step;                  // source columns per key class (0: all read column 0)
  float factor;                      // applied to source rows (c for dout, 1 for dG)
};

__device__ __forceinline__ float* dst_row(const SegArgs& a, uint64_t key) {
  if (a.by_table)
    return a.dst[key >> a.row_bits] + int64_t(key & ((uint64_t(1) << a.row_bits) - 1)) * a.width;
  return a.dst[0] + int64_t(key) * a.width;
}

// 4 consecutive source values as fp32 (16 bytes of fp32, 8 bytes of bf16).
template <typename T> __device__ __forceinline__ f32x4_t ld4(const T* p);
template <> __device__ __forceinline__ f32x4_t ld4<float>(const float* p) {
  return *reinterpret_cast<const f32x4_t*>(p);
}
template <> __device__ __forceinline__ f32x4_t ld4<uint16_t>(const uint16_t* p) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t h = *reinterpret_cast<const u32x2_t*>(p);
  return f32x4_t{bf16_to_f32(h.x & 0xffffu), bf16_to_f32(h.x >> 16), bf16_to_f32(h.y & 0xffffu),
                 bf16_to_f32(h.y >> 16)};
}

// The runs are summed in vectors of 4 columns: lane v of a block of THREADS handles vectors
// v, v + THREADS, ... (NV of them) of a gradient row, so a sub-table row (256 values) is
// one wave and an E_0 row (3072) one 256-thread block. Blocks cover column groups of
// THREADS * NV * 4 values (grid.y) when rows are wider.
template <int THREADS, int NV>
struct Cols {
  static constexpr int kGroup = THREADS * NV * 4;
  static __device__ __forceinline__ int col(int v) {
    return int(blockIdx.y) * kGroup + (int(threadIdx.x) + v * THREADS) * 4;
  }
};

// Level 1: block (chunk, column group) walks its CH entries in order. A run lying
// wholly inside the chunk is added to its gradient row here (its only owner); the run the
// chunk starts in, if it began earlier, goes to head[chunk]; a run that begins here and
// continues past the chunk goes to tail[chunk] and the chunk joins the level-2 list. The
// chunk's keys and positions are staged in LDS; the source rows of B entries, and the
// gradient rows of the runs they end, are loaded before any is used.
template <typename T, int THREADS, int NV, int CH>
__global__ __launch_bounds__(THREADS) void segsum_level1_kernel(const SegArgs a) {
  constexpr int B = NV >= 4 ? 2 : (NV >= 2 ? 4 : 8);
  using C = Cols<THREADS, NV>;
  __shared__ uint64_t skey[CH + 2];         // keys[lo - 1 .. hi] (ends valid if present)
  __shared__ uint32_t sval[CH];
  const int64_t chunk = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t lo = chunk * CH, hi = std::min<int64_t>(a.n, lo + CH);
  const int cnt = int(hi - lo);
  const bool has_prev = lo > 0, has_next = hi < a.n;
  for (int i = t; i < cnt; i += THREADS) {
    skey[i + 1] = a.keys[lo + i];
    sval[i] = a.vals[lo + i];
  }
  if (t == 0) skey[0] = has_prev ? a.keys[lo - 1] : 0;
  if (t == 0) skey[cnt + 1] = has_next ? a.keys[hi] : 0;
  __syncthreads();
  const bool cont_in = has_prev && skey[0] == skey[1];
  f32x4_t acc[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) acc[v] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  bool first = true;
  for (int b0 = 0; b0 < cnt; b0 += B) {
    f32x4_t rows[B][NV], dsts[B][NV];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int j = b0 + u;
      const bool live = j < cnt && skey[j + 1] != a.sentinel;
      const uint64_t key = live ? skey[j + 1] : 0;
      const int s = a.by_table ? int(key >> a.row_bits) : 0;
      const T* row = static_cast<const T*>(a.src) + int64_t(live ? sval[j] : 0) * a.ld_src +
                     s * a.col_step;
      const bool last = j + 1 == cnt;
      const bool ends = live && (last ? !(has_next && skey[cnt + 1] == key) : skey[j + 2] != key);
      const bool owned = ends && !(cont_in && key == skey[1]);   // added here, directly
      const float* d = owned ? dst_row(a, key) : nullptr;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int c = C::col(v);
        rows[u][v] = live && c < a.width ? ld4<T>(row + c) : f32x4_t{0.f, 0.f, 0.f, 0.f};
        dsts[u][v] = owned && c < a.width ? *reinterpret_cast<const f32x4_t*>(d + c)
                                          : f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int j = b0 + u;
      if (j >= cnt) break;
      const uint64_t key = skey[j + 1];
      if (key == a.sentinel) return;               // invalid positions sort last
#pragma unroll
      for (int v = 0; v < NV; ++v) acc[v] += rows[u][v] * a.factor;
      const bool last = j + 1 == cnt;
      if (!last && skey[j + 2] == key) continue;   // the run goes on in this chunk
      const bool cont_out = last && has_next && skey[cnt + 1] == key;
      float* dst = first && cont_in ? a.head + chunk * a.width
                   : cont_out       ? a.tail + chunk * a.width
                                    : dst_row(a, key);
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int c = C::col(v);
        if (c < a.width)
          *reinterpret_cast<f32x4_t*>(dst + c) =
              (first && cont_in) || cont_out ? acc[v] : dsts[u][v] + acc[v];
        acc[v] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
      if (cont_out && !(first && cont_in) && blockIdx.y == 0 && t == 0)
        a.owners[1 + atomicAdd(a.owners, 1u)] = uint32_t(chunk);
      first = false;
    }
  }
}

// Level 2: each chunk listed by level 1 (its last run starts in it and continues) adds its
// tail and the head sums of the following chunks that the run covers, in order. The run's
// end is found first, so the sum's loads do not wait on each other: each lane of a wave
// checks whether the run reaches one of the next 64 chunks (the chunk's first entry holds
// the run's key; keys are sorted, so the run covers every chunk before it), and only a
// longer run takes a binary search past them.
// Blocks stride over the list; its order does not matter (each run has one owner).
template <int THREADS, int NV>
__global__ __launch_bounds__(THREADS) void segsum_level2_kernel(const SegArgs a) {
  using C = Cols<THREADS, NV>;
  const uint32_t n_owners = a.owners[0];
  const int lane = threadIdx.x & 63;
  for (uint32_t o = blockIdx.x; o < n_owners; o += gridDim.x) {
    const int64_t chunk = a.owners[1 + o];
    const int64_t hi = std::min<int64_t>(a.n, chunk * a.chunk + a.chunk);
    const uint64_t key = a.keys[hi - 1];
    const int64_t pc = chunk + 1 + lane;           // chunk whose first entry this lane checks
    const bool reaches = pc < a.nchunks && a.keys[pc * a.chunk] == key;
    const uint64_t stop = __ballot(!reaches);      // lane 0 reaches (the run continues)
    int64_t last_chunk;                            // chunks chunk+1 .. last_chunk hold a head
    if (stop != 0) {
      last_chunk = chunk + __builtin_ctzll(stop);
    } else {
      // A 64-way search for the first index past the run in [l, r] (keys[l - 1] holds the
      // run's key; keys[r] is past it, or r = n). Each round lane i checks the last entry of
      // the i-th of 64 equal segments of [l, r); the first segment whose last entry is past
      // the run holds the answer, and if none is, the run fills [l, r).
      int64_t l = std::min<int64_t>(a.n, (chunk + 64) * a.chunk + 1), r = a.n;
      while (l < r) {
        const int64_t step = (r - l + 63) / 64;
        const int64_t p = std::min<int64_t>(r, l + (lane + 1) * step) - 1;
        const uint64_t past = __ballot(l + lane * step < r && a.keys[p] != key);
        if (past == 0) {
          l = r;
        } else {
          const int i = __builtin_ctzll(past);
          r = std::min<int64_t>(r, l + (i + 1) * step) - 1;   // that segment's last entry
          l += i * step;                                     // that segment's first entry
        }
      }
      last_chunk = (l - 1) / a.chunk;
    }
    // the tail, then the heads in chunk order; each lane's columns are fixed, so the loads
    // of one column range do not sit behind a branch and go out several at a time
    f32x4_t acc[NV];
    const float* tl = a.tail + chunk * a.width;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int c = C::col(v);
      acc[v] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (c < a.width) {
        f32x4_t sum = *reinterpret_cast<const f32x4_t*>(tl + c);
#pragma unroll 16
        for (int64_t ch = chunk + 1; ch <= last_chunk; ++ch)
          sum += *reinterpret_cast<const f32x4_t*>(a.head + ch * a.width + c);
        acc[v] = sum;
      }
    }
    float* dst = dst_row(a, key);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int c = C::col(v);
      if (c < a.width)
        *reinterpret_cast<f32x4_t*>(dst + c) = *reinterpret_cast<const f32x4_t*>(dst + c) + acc[v];
    }
  }
}

int key_bits(uint64_t max_key) {
  int b = 1;
  while (b < 64 && (max_key >> b) != 0) ++b;
  return b;
}

// Sorts n (key, value) pairs with keys below 2^bits, ping-ponging between the two buffers;
// on return k0/v0 name the buffers that hold the result.
hipError_t radix_sort_pp(uint64_t*& k0, uint32_t*& v0, uint64_t*& k1, uint32_t*& v1,
                         uint32_t* hist, int64_t n, int bits, hipStream_t st) {
  const int64_t nblocks = (n + kSortTile - 1) / kSortTile;
  for (int shift = 0; shift < bits; shift += 8) {
    hipLaunchKernelGGL(radix_hist_kernel, dim3(unsigned(nblocks)), dim3(kSortThreads), 0, st, k0,
                       n, shift, hist);
    const int64_t m = 256 * nblocks, ntiles = (m + kScanTile - 1) / kScanTile;
    hipLaunchKernelGGL(scan_totals_kernel, dim3(unsigned(ntiles)), dim3(256), 0, st, hist, m,
                       hist + m);
    hipLaunchKernelGGL(scan_apply_kernel, dim3(unsigned(ntiles)), dim3(256), 0, st, hist, m,
                       hist + m);
    hipLaunchKernelGGL(radix_scatter_kernel, dim3(unsigned(nblocks)), dim3(kSortThreads), 0, st,
                       k0, v0, n, shift, hist, k1, v1);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    std::swap(k0, k1);
    std::swap(v0, v1);
  }
  return hipSuccess;
}

// The same with the result in the first buffers (an odd number of passes copies it back).
hipError_t radix_sort(uint64_t* k0, uint32_t* v0, uint64_t* k1, uint32_t* v1, uint32_t* hist,
                      int64_t n, int bits, hipStream_t st) {
  uint64_t* ka = k0;
  uint32_t* va = v0;
  hipError_t e = radix_sort_pp(ka, va, k1, v1, hist, n, bits, st);
  if (e == hipSuccess && ka != k0) {
    e = hipMemcpyAsync(k0, ka, size_t(n) * 8, hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess) e = hipMemcpyAsync(v0, va, size_t(n) * 4, hipMemcpyDeviceToDevice, st);
  }
  return e;
}

__global__ void clear_count_kernel(uint32_t* c) { *c = 0u; }

template <typename T, int THREADS, int NV>
hipError_t segsum_launch(const SegArgs& a, hipStream_t st) {
  const unsigned gy = unsigned((a.width + Cols<THREADS, NV>::kGroup - 1) / Cols<THREADS, NV>::kGroup);
  if (a.chunk == kChunkWide)
    hipLaunchKernelGGL((segsum_level1_kernel<T, THREADS, NV, kChunkWide>),
                       dim3(unsigned(a.nchunks), gy), dim3(THREADS), 0, st, a);
  else
    hipLaunchKernelGGL((segsum_level1_kernel<T, THREADS, NV, kChunk>),
                       dim3(unsigned(a.nchunks), gy), dim3(THREADS), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((segsum_level2_kernel<THREADS, NV>),
                     dim3(unsigned(std::min<int64_t>(a.nchunks, 1024)), gy), dim3(THREADS), 0, st,
                     a);
  return hipGetLastError();
}

template <typename T>
hipError_t segsum_typed(const SegArgs& a, hipStream_t st) {
  // one 4-value vector per lane: a wave per row of up to 256 values, else 256-thread blocks
  // over column groups of 1024 values (more blocks, longer load batches)
  if (a.width <= 256) return segsum_launch<T, 64, 1>(a, st);
  return segsum_launch<T, 256, 1>(a, st);
}

// Chunks of kChunk entries for the sub-tables (many short runs), kChunkWide for E_0, whose
// hottest tokens form runs of thousands: fewer partial sums for their owner to add, while
// enough chunks remain to fill the GPU in level 1 (measured best of 32, 64 and 256).
hipError_t segsum(SegArgs a, bool src_f32, hipStream_t st) {
  a.chunk = a.by_table ? kChunk : kChunkWide;
  a.nchunks = (a.n + a.chunk - 1) / a.chunk;
  hipLaunchKernelGGL(clear_count_kernel, dim3(1), dim3(1), 0, st, a.owners);
  return src_f32 ? segsum_typed<float>(a, st) : segsum_typed<uint16_t>(a, st);
}

int32_t ceil_log2(int64_t x) {
  int32_t b = 0;
  while ((int64_t(1) << b) < x) ++b;
  return b;
}

}  // namespace

hipError_t launch_radix_sort(uint64_t* k0, uint32_t* v0, uint64_t* k1, uint32_t* v1,
                             uint32_t* hist, int64_t n, int bits, hipStream_t st) {
  return radix_sort(k0, v0, k1, v1, hist, n, bits, st);
}

hipError_t launch_backward(const LayerDesc& L, const BackwardArgs& b, hipStream_t st) {
  const int64_t T = b.rows;
  const int64_t Tp = (T + 63) / 64 * 64;
  const int64_t D = L.D;
  const float c = L.scale / float(L.S + 1);
  // the basic form has no projection: dE_s sums c dout rows directly, and there is no dW
  const bool basic = L.form == NGRAM_FORM_BASIC;
  const bool need_dg = L.S > 0 && b.dE != nullptr;
  const bool need_dw = L.S > 0 && b.dW != nullptr && !basic;
  hipError_t e;
  const int64_t nid = std::max<int64_t>(T, D);
  hipLaunchKernelGGL(iota_kernel, dim3(unsigned((nid + 255) / 256)), dim3(256), 0, st, b.ident,
                     nid);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const bool f32 = L.dtype == NGRAM_F32;
  if (need_dg && !basic) {
    // W^T, then dG = c dout (W^T)^T = c dout W
    const dim3 g((unsigned((D + kTile - 1) / kTile)), unsigned((D + kTile - 1) / kTile));
    if (f32)
      hipLaunchKernelGGL(transpose_pad_kernel<float>, g, dim3(256), 0, st,
                         static_cast<const float*>(b.W), D, int32_t(D), nullptr, 0,
                         static_cast<float*>(b.WT), D);
    else
      hipLaunchKernelGGL(transpose_pad_kernel<uint16_t>, g, dim3(256), 0, st,
                         static_cast<const uint16_t*>(b.W), D, int32_t(D), nullptr, 0,
                         static_cast<uint16_t*>(b.WT), D);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    e = launch_dense_product(L, b.dout, T, b.WT, int32_t(D), int32_t(D), b.ident, b.dG, D, c,
                             false, nullptr, 1, st);
    if (e != hipSuccess) return e;
  }
  if (need_dw) {
    // dout^T (invalid positions zeroed) and G^T, both [D, Tp]; then dW += c dout^T G
    const dim3 g(unsigned(Tp / kTile), unsigned((D + kTile - 1) / kTile));
    GatherTArgs ga{};
    for (int s = 0; s < L.S; ++s) {
      ga.E[s] = b.E[s];
      ga.Vm1[s] = L.V[s] - 1u;
    }
    ga.idx = b.idx;
    ga.tok = b.tokens;
    ga.GT = b.GT;
    ga.rows = T;
    ga.ldt = Tp;
    ga.S = L.S;
    ga.d = L.d;
    ga.D = L.D;
    ga.V0 = L.V0;
    if (f32) {
      hipLaunchKernelGGL(transpose_pad_kernel<float>, g, dim3(256), 0, st,
                         static_cast<const float*>(b.dout), T, int32_t(D), b.tokens, L.V0,
                         static_cast<float*>(b.doutT), Tp);
      hipLaunchKernelGGL(gather_transpose_kernel<float>, g, dim3(256), 0, st, ga);
    } else {
      if (D % kTile == 0)
        hipLaunchKernelGGL(transpose_pad16_kernel, g, dim3(256), 0, st,
                           static_cast<const uint16_t*>(b.dout), T, int32_t(D), b.tokens, L.V0,
                           static_cast<uint16_t*>(b.doutT), Tp);
      else
        hipLaunchKernelGGL(transpose_pad_kernel<uint16_t>, g, dim3(256), 0, st,
                           static_cast<const uint16_t*>(b.dout), T, int32_t(D), b.tokens, L.V0,
                           static_cast<uint16_t*>(b.doutT), Tp);
      if (L.d % kTile == 0)
        hipLaunchKernelGGL(gather_transpose16_kernel, g, dim3(256), 0, st, ga);
      else
        hipLaunchKernelGGL(gather_transpose_kernel<uint16_t>, g, dim3(256), 0, st, ga);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    e = launch_dense_product(L, b.doutT, D, b.GT, int32_t(D), int32_t(Tp), b.ident, b.dW, D, c,
                             true, b.part, backward_splits(L, T), st);
    if (e != hipSuccess) return e;
  }
  if (need_dg) {
    // dE_s: sort (s, row) keys of all T*S pairs, sum the dG blocks of each run
    const int64_t n = T * L.S;
    // key = (s << row_bits) | row: 24 + 4 bits for the 30B layer, 4 sort passes (not 5)
    uint32_t vmax = 1;
    for (int s = 0; s < L.S; ++s) vmax = std::max(vmax, L.V[s]);
    const int32_t row_bits = std::max<int32_t>(1, ceil_log2(int64_t(vmax)));
    const uint64_t sentinel = uint64_t(1) << (row_bits + ceil_log2(L.S));
    hipLaunchKernelGGL(keys_subtables_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, st,
                       b.idx, b.tokens, T, L.S, L.V0, row_bits, sentinel, b.keys0, b.vals0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    uint64_t *ks = b.keys0, *kt = b.keys1;
    uint32_t *vs = b.vals0, *vt = b.vals1;
    e = radix_sort_pp(ks, vs, kt, vt, b.hist, n, key_bits(sentinel), st);
    if (e != hipSuccess) return e;
    SegArgs a{};
    for (int s = 0; s < L.S; ++s) a.dst[s] = b.dE[s];
    a.keys = ks;
    a.vals = vs;
    a.src = basic ? b.dout : static_cast<const void*>(b.dG);
    a.head = b.head;
    a.tail = b.tail;
    a.owners = b.owners;
    a.n = n;
    a.ld_src = D;
    a.sentinel = sentinel;
    a.width = L.d;
    a.by_table = 1;
    a.row_bits = row_bits;
    a.col_step = basic ? 0 : L.d;
    a.factor = basic ? c : 1.0f;
    if ((e = segsum(a, basic ? f32 : true, st)) != hipSuccess) return e;
  }
  if (b.dE0 != nullptr) {
    // dE_0: sort tokens, sum c * dout rows of each run
    const uint64_t sentinel = uint64_t(1) << ceil_log2(int64_t(L.V0) + 1);
    hipLaunchKernelGGL(keys_tokens_kernel, dim3(unsigned((T + 255) / 256)), dim3(256), 0, st,
                       b.tokens, T, L.V0, sentinel, b.keys0, b.vals0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    uint64_t *ks = b.keys0, *kt = b.keys1;
    uint32_t *vs = b.vals0, *vt = b.vals1;
    e = radix_sort_pp(ks, vs, kt, vt, b.hist, T, key_bits(sentinel), st);
    if (e != hipSuccess) return e;
    SegArgs a{};
    a.dst[0] = b.dE0;
    a.keys = ks;
    a.vals = vs;
    a.src = b.dout;
    a.head = b.head;
    a.tail = b.tail;
    a.owners = b.owners;
    a.n = T;
    a.ld_src = D;
    a.sentinel = sentinel;
    a.width = L.D;
    a.by_table = 0;
    a.factor = c;
    if ((e = segsum(a, f32, st)) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ngram
