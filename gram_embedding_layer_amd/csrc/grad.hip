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

#include "kernels.h"

namespace ngram {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

template <typename T> __device__ __forceinline__ float ldf(const T* p);
template <> __device__ __forceinline__ float ldf<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ldf<uint16_t>(const uint16_t* p) {
  return bf16_to_f32(*p);
}

constexpr int kTile = 64;           // transpose tile edge
constexpr int kSortThreads = 256;
constexpr int kSortRounds = kSortTile / kSortThreads;   // keys per thread per sort tile
constexpr int kScanThreads = 1024;
constexpr int kColsPerThread = 4;   // columns per thread in the reductions
constexpr int kColGroup = 256 * kColsPerThread;

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

// Sort inputs. E_0: key = token, value = position. Sub-tables: pair p = i*S + s has key
// (s << 31) | idx[i, s] and value i. Invalid positions get the key `sentinel` (sorted last).
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
    int32_t V0, uint64_t sentinel, uint64_t* __restrict__ keys, uint32_t* __restrict__ vals) {
  const int64_t p = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (p >= rows * S) return;
  const int64_t i = p / S;
  const int s = int(p - i * S);
  keys[p] = uint32_t(tok[i]) < uint32_t(V0) ? (uint64_t(s) << 31) | uint32_t(idx[p])
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

// In-place exclusive prefix sum of n counts, one block.
__global__ __launch_bounds__(kScanThreads) void exclusive_scan_kernel(uint32_t* v, int64_t n) {
  __shared__ uint32_t part[kScanThreads];
  const int t = threadIdx.x;
  const int64_t per = (n + kScanThreads - 1) / kScanThreads;
  const int64_t lo = std::min<int64_t>(n, t * per), hi = std::min<int64_t>(n, lo + per);
  uint32_t sum = 0;
  for (int64_t i = lo; i < hi; ++i) sum += v[i];
  part[t] = sum;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {     // Hillis-Steele over the sums
    const uint32_t x = t >= off ? part[t - off] : 0u;
    __syncthreads();
    part[t] += x;
    __syncthreads();
  }
  uint32_t run = part[t] - sum;                            // exclusive prefix of this thread
  for (int64_t i = lo; i < hi; ++i) {
    const uint32_t x = v[i];
    v[i] = run;
    run += x;
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
  int64_t n, nchunks, ld_src;
  uint64_t sentinel;
  int32_t width;                     // gradient row width (D for E_0, d for sub-tables)
  int32_t by_table;                  // 1: key = (s << 31) | r, source columns s*width...
  float factor;                      // applied to source rows (c for dout, 1 for dG)
};

template <typename T>
__device__ __forceinline__ void run_add(const SegArgs& a, int64_t j, int col0, f32x4_t& acc) {
  const uint64_t key = a.keys[j];
  const int s = a.by_table ? int(key >> 31) : 0;
  const T* row = static_cast<const T*>(a.src) + int64_t(a.vals[j]) * a.ld_src + s * a.width;
#pragma unroll
  for (int k = 0; k < kColsPerThread; ++k) {
    const int c = col0 + k * 256;
    if (c < a.width) acc[k] += ldf<T>(row + c) * a.factor;
  }
}

__device__ __forceinline__ float* dst_row(const SegArgs& a, uint64_t key) {
  if (a.by_table) return a.dst[key >> 31] + int64_t(key & 0x7fffffffu) * a.width;
  return a.dst[0] + int64_t(key) * a.width;
}

__device__ __forceinline__ void add_row(float* row, int col0, int width, const f32x4_t& v) {
#pragma unroll
  for (int k = 0; k < kColsPerThread; ++k) {
    const int c = col0 + k * 256;
    if (c < width) row[c] += v[k];
  }
}

__device__ __forceinline__ void put_row(float* row, int col0, int width, const f32x4_t& v) {
#pragma unroll
  for (int k = 0; k < kColsPerThread; ++k) {
    const int c = col0 + k * 256;
    if (c < width) row[c] = v[k];
  }
}

// Level 1: block (chunk, column group) walks its kChunk entries in order. A run lying
// wholly inside the chunk is added to its gradient row here (its only owner); the run the
// chunk starts in, if it began earlier, goes to head[chunk]; a run that begins here and
// continues past the chunk goes to tail[chunk] for level 2.
template <typename T>
__global__ __launch_bounds__(256) void segsum_level1_kernel(const SegArgs a) {
  const int64_t chunk = blockIdx.x;
  const int col0 = blockIdx.y * kColGroup + threadIdx.x;
  const int64_t lo = chunk * kChunk, hi = std::min<int64_t>(a.n, lo + kChunk);
  const bool cont_in = lo > 0 && a.keys[lo - 1] == a.keys[lo];
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  bool first = true;
  for (int64_t j = lo; j < hi; ++j) {
    const uint64_t key = a.keys[j];
    if (key == a.sentinel) break;                  // invalid positions sort last
    run_add<T>(a, j, col0, acc);
    const bool run_ends_here = j + 1 >= hi || a.keys[j + 1] != key;
    if (!run_ends_here) continue;
    const bool cont_out = j + 1 == hi && hi < a.n && a.keys[hi] == key;
    if (first && cont_in) {
      put_row(a.head + chunk * a.width, col0, a.width, acc);
    } else if (cont_out) {
      put_row(a.tail + chunk * a.width, col0, a.width, acc);
    } else {
      add_row(dst_row(a, key), col0, a.width, acc);
    }
    first = false;
    acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
}

// Level 2: a chunk whose last run starts in it and continues adds its tail and the head
// sums of the following chunks that the run covers, in order.
__global__ __launch_bounds__(256) void segsum_level2_kernel(const SegArgs a) {
  const int64_t chunk = blockIdx.x;
  const int col0 = blockIdx.y * kColGroup + threadIdx.x;
  const int64_t lo = chunk * kChunk, hi = std::min<int64_t>(a.n, lo + kChunk);
  if (hi >= a.n) return;
  const uint64_t key = a.keys[hi - 1];
  if (key == a.sentinel || a.keys[hi] != key) return;      // the last run ends here
  if (lo > 0 && a.keys[lo - 1] == key) return;             // ... or began in an earlier chunk
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  const float* tl = a.tail + chunk * a.width;
#pragma unroll
  for (int k = 0; k < kColsPerThread; ++k)
    if (col0 + k * 256 < a.width) acc[k] = tl[col0 + k * 256];
  for (int64_t c = chunk + 1; c < a.nchunks && a.keys[c * kChunk] == key; ++c) {
    const float* hd = a.head + c * a.width;
#pragma unroll
    for (int k = 0; k < kColsPerThread; ++k)
      if (col0 + k * 256 < a.width) acc[k] += hd[col0 + k * 256];
  }
  add_row(dst_row(a, key), col0, a.width, acc);
}

int key_bits(uint64_t max_key) {
  int b = 1;
  while (b < 64 && (max_key >> b) != 0) ++b;
  return b;
}

// Sorts n (key, value) pairs in place (result in k0/v0); keys below 2^bits.
hipError_t radix_sort(uint64_t* k0, uint32_t* v0, uint64_t* k1, uint32_t* v1, uint32_t* hist,
                      int64_t n, int bits, hipStream_t st) {
  const int64_t nblocks = (n + kSortTile - 1) / kSortTile;
  for (int shift = 0; shift < bits; shift += 8) {
    hipLaunchKernelGGL(radix_hist_kernel, dim3(unsigned(nblocks)), dim3(kSortThreads), 0, st, k0,
                       n, shift, hist);
    hipLaunchKernelGGL(exclusive_scan_kernel, dim3(1), dim3(kScanThreads), 0, st, hist,
                       256 * nblocks);
    hipLaunchKernelGGL(radix_scatter_kernel, dim3(unsigned(nblocks)), dim3(kSortThreads), 0, st,
                       k0, v0, n, shift, hist, k1, v1);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    std::swap(k0, k1);
    std::swap(v0, v1);
  }
  // an odd number of passes leaves the result in the second buffer: copy it back
  if (((bits + 7) / 8) % 2 == 1) {
    hipError_t e = hipMemcpyAsync(k1, k0, size_t(n) * 8, hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess)
      e = hipMemcpyAsync(v1, v0, size_t(n) * 4, hipMemcpyDeviceToDevice, st);
    return e;
  }
  return hipSuccess;
}

hipError_t segsum(SegArgs a, bool src_f32, hipStream_t st) {
  a.nchunks = (a.n + kChunk - 1) / kChunk;
  const dim3 grid(unsigned(a.nchunks), unsigned((a.width + kColGroup - 1) / kColGroup));
  if (src_f32)
    hipLaunchKernelGGL(segsum_level1_kernel<float>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(segsum_level1_kernel<uint16_t>, grid, dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(segsum_level2_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

int32_t ceil_log2(int64_t x) {
  int32_t b = 0;
  while ((int64_t(1) << b) < x) ++b;
  return b;
}

}  // namespace

hipError_t launch_backward(const LayerDesc& L, const BackwardArgs& b, hipStream_t st) {
  const int64_t T = b.rows;
  const int64_t Tp = (T + 63) / 64 * 64;
  const int64_t D = L.D;
  const float c = L.scale / float(L.S + 1);
  const bool need_dg = L.S > 0 && b.dE != nullptr;
  const bool need_dw = L.S > 0 && b.dW != nullptr;
  hipError_t e;
  const int64_t nid = std::max<int64_t>(T, D);
  hipLaunchKernelGGL(iota_kernel, dim3(unsigned((nid + 255) / 256)), dim3(256), 0, st, b.ident,
                     nid);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const bool f32 = L.dtype == NGRAM_F32;
  if (need_dg) {
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
      hipLaunchKernelGGL(transpose_pad_kernel<uint16_t>, g, dim3(256), 0, st,
                         static_cast<const uint16_t*>(b.dout), T, int32_t(D), b.tokens, L.V0,
                         static_cast<uint16_t*>(b.doutT), Tp);
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
    const uint64_t sentinel = uint64_t(1) << (31 + ceil_log2(L.S));
    hipLaunchKernelGGL(keys_subtables_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, st,
                       b.idx, b.tokens, T, L.S, L.V0, sentinel, b.keys0, b.vals0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    e = radix_sort(b.keys0, b.vals0, b.keys1, b.vals1, b.hist, n, key_bits(sentinel), st);
    if (e != hipSuccess) return e;
    SegArgs a{};
    for (int s = 0; s < L.S; ++s) a.dst[s] = b.dE[s];
    a.keys = b.keys0;
    a.vals = b.vals0;
    a.src = b.dG;
    a.head = b.head;
    a.tail = b.tail;
    a.n = n;
    a.ld_src = D;
    a.sentinel = sentinel;
    a.width = L.d;
    a.by_table = 1;
    a.factor = 1.0f;
    if ((e = segsum(a, true, st)) != hipSuccess) return e;
  }
  if (b.dE0 != nullptr) {
    // dE_0: sort tokens, sum c * dout rows of each run
    const uint64_t sentinel = uint64_t(1) << ceil_log2(int64_t(L.V0) + 1);
    hipLaunchKernelGGL(keys_tokens_kernel, dim3(unsigned((T + 255) / 256)), dim3(256), 0, st,
                       b.tokens, T, L.V0, sentinel, b.keys0, b.vals0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    e = radix_sort(b.keys0, b.vals0, b.keys1, b.vals1, b.hist, T, key_bits(sentinel), st);
    if (e != hipSuccess) return e;
    SegArgs a{};
    a.dst[0] = b.dE0;
    a.keys = b.keys0;
    a.vals = b.vals0;
    a.src = b.dout;
    a.head = b.head;
    a.tail = b.tail;
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
