// Kernel 1 (rolling hash) and the N-gram cache kernels of the decode path.
//
// The hash is the polynomial rolling hash of section A2 of the deep-notes page on "Scaling
// Embeddings Outperforms Scaling Experts in Language Models":
//   H_{n,k}(t_{i-n+1..i}) = (sum_{j<n} t_{i-j} V0^j) mod V_{n,k}.
// The raw polynomial needs up to n*31 bits (more than 64 for n >= 3 at V0 = 2^17), so it is
// evaluated by Horner's rule from the oldest id to the newest, reducing modulo V_{n,k} after
// every step: x <- (x*V0 + t) mod V. With x < V < 2^31 and t < 2^32 every intermediate is
// below 2^63, and the step's residue is taken exactly by Barrett reduction (below).
#include "decode_step.h"

namespace ngram {
namespace {

constexpr int kThreads = 256;

// Thread i of a prefill-shaped launch: checks entry i of cu_seqlens (0 = c_0 <= c_1 <= ...
// <= c_nseq = ntok), then, for a position i < ntok, its id, and fills c[j] = t_{i-j} for
// j < nord (pad id 0 before the start of the position's sequence). False past the batch.
template <int NMAX>
__device__ __forceinline__ bool position_context(const int32_t* __restrict__ tokens,
                                                 const int32_t* __restrict__ cu, int32_t nseq,
                                                 int64_t ntok, int64_t V0, int nord, int64_t i,
                                                 int32_t* __restrict__ flags,
                                                 uint32_t (&c)[NMAX]) {
  if (flags != nullptr && i <= nseq) {
    const int64_t ci = cu[i];
    const bool bad = (i == 0 && ci != 0) || (i == nseq && ci != ntok) ||
                     (i < nseq && ci > cu[i + 1]);
    if (bad) atomicOr(flags, NGRAM_FLAG_BAD_SEQLENS);
  }
  if (i >= ntok) return false;
  // sequence of position i: the last b with cu[b] <= i
  int lo = 0, hi = nseq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= i) lo = mid; else hi = mid - 1;
  }
  int64_t start = cu[lo];
  start = start < 0 ? 0 : (start > i ? i : start);   // never read outside [0, i]
  const int32_t t = tokens[i];
  if (flags != nullptr && uint32_t(t) >= uint32_t(V0)) atomicOr(flags, NGRAM_FLAG_BAD_TOKEN);
#pragma unroll
  for (int j = 0; j < NMAX; ++j)
    c[j] = (j < nord && i - j >= start) ? uint32_t(tokens[i - j]) : 0u;
  return true;
}

// Whether batch entry b's slot already appears at an earlier entry (slots of one call must be
// distinct; a repeated slot would have two entries read and append to one ring at once).
// Every thread of the block calls it (it meets the others at barriers): the block reads
// slots[0, bmax) tile by tile into `tile` (nthreads ints) and the `nparts` threads of an
// entry share the comparisons with the entries below b (thread `part` takes every nparts-th).
// bmax: one past the block's last entry. Inactive threads pass b = 0.
__device__ __forceinline__ bool slot_seen_before(const int32_t* __restrict__ slots, int32_t bmax,
                                                 int32_t b, int32_t slot, int part, int nparts,
                                                 int32_t* tile, int nthreads) {
  bool seen = false;
  for (int32_t t0 = 0; t0 < bmax; t0 += nthreads) {
    __syncthreads();                                   // the previous tile is read
    const int32_t q = t0 + int32_t(threadIdx.x);
    tile[threadIdx.x] = q < bmax ? slots[q] : -1;
    __syncthreads();
    for (int k = part; k < nthreads && t0 + k < b; k += nparts) seen |= tile[k] == slot;
  }
  return seen;
}

// One thread per (position, sub-table): thread g hashes sub-table g % S of position g / S, so
// a position's S hashes run side by side (a thread per position left one wave per SIMD
// working through ~36 dependent 64-bit Horner steps) and the index writes are contiguous.
// The position's first thread checks cu_seqlens and the id.
template <int NMAX>
__global__ __launch_bounds__(kThreads) void hash_prefill_kernel(
    const LayerDesc L, const int32_t* __restrict__ tokens, const int32_t* __restrict__ cu,
    int32_t nseq, int64_t ntok, int32_t* __restrict__ idx, int32_t* __restrict__ flags) {
  const int64_t g = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t i = g / L.S;
  const int s = int(g - i * L.S);
  uint32_t c[NMAX];
  if (!position_context<NMAX>(tokens, cu, nseq, ntok, L.V0, L.N, i, s == 0 ? flags : nullptr,
                              c))
    return;
  const int n = 2 + s / L.K;               // order of sub-table s = (n-2)K + (k-1)
  const uint64_t V = L.V[s], m = L.Vinv[s];
  uint64_t x = 0;
#pragma unroll
  for (int j = NMAX - 1; j >= 0; --j)
    if (j < n) x = horner_step(x, uint64_t(L.V0), c[j], V, m);
  idx[g] = int32_t(x);
}

// One decode step: every thread hashes one (batch entry, row, sub-table) of the window
// from the N-gram cache and the step's new ids, so a row's S hashes run side by side rather
// than one after another (a thread per row left each SIMD one wave doing ~36 dependent
// 64-bit Horner steps: 9 us per 256 x 5-row step of the 30B layer). Batch entry b uses cache
// slot slots[b] (or b); its rows j in [row_begin, row_begin + width) become compact rows
// b * width + (j - row_begin). A block holds whole batch entries (kDecThreads / (width * S)
// of them), so when the step also commits, all reads of an entry's ring precede the barrier
// and the commit's writes (by the entry's first thread) follow. Rows past n_new[b] (and
// every row of an entry whose slot is out of range) get the token `unused_tok`: -1 (the
// projection writes a zero row) or kSkipRow (the row is not written).
constexpr int kDecThreads = 512;   // >= width * S for every accepted width (<= 8) and S (<= 64)

template <int NMAX>
__global__ __launch_bounds__(kDecThreads) void hash_decode_kernel(const LayerDesc L,
                                                                  const DecodeArgs a) {
  const int ns = L.S > 0 ? L.S : 1;                // threads per row
  const int tpe = a.width * ns;                    // threads per batch entry
  const int epb = kDecThreads / tpe;               // batch entries per block
  const int b = blockIdx.x * epb + int(threadIdx.x) / tpe;
  const int within = int(threadIdx.x) % tpe;
  const int jj = within / ns, s = within % ns;
  const int j = a.row_begin + jj;
  const bool active = int(threadIdx.x) < epb * tpe && b < a.nbatch;
  const bool lead = within == 0;                   // the entry's flags and commit
  // with a slot map: an entry whose slot an earlier entry already uses is ignored (no rows
  // written, no commit), so no ring is read and appended to by two entries at once
  bool dup = false;
  if (a.slots != nullptr) {
    __shared__ int32_t tile[kDecThreads];
    __shared__ int32_t seen[kDecThreads];          // per entry of the block (epb <= 512)
    const int le = int(threadIdx.x) / tpe;
    if (int(threadIdx.x) < epb) seen[threadIdx.x] = 0;
    const int32_t bmax = min(a.nbatch, int32_t(blockIdx.x + 1) * epb);
    const bool hit = slot_seen_before(a.slots, bmax, active ? b : 0, active ? a.slots[b] : -1,
                                      within, tpe, tile, kDecThreads);
    if (active && hit) seen[le] = 1;
    __syncthreads();
    dup = active && seen[le] != 0;
  }
  DecodeEntry<NMAX> e{};
  int acc = 0;
  if (active) {
    // the row's context (ids up to j) and, for the entry's commit, every new id
    e = load_entry<NMAX>(L, a, b, lead ? NGRAM_MAX_DECODE_TOKENS - 1 : j);
    if (a.n_commit != nullptr && lead) acc = a.n_commit[b];
    if (lead && a.flags != nullptr) {
      if (!e.slot_ok) atomicOr(a.flags, NGRAM_FLAG_BAD_SLOT);
      else if (dup) atomicOr(a.flags, NGRAM_FLAG_DUP_SLOT);
      if (e.bad_count) atomicOr(a.flags, NGRAM_FLAG_BAD_COUNT);
    }
    if (dup) e.slot_ok = false;
    const int64_t r = int64_t(b) * a.width + jj;
    uint32_t id;
    if (!entry_row(e, j, &id)) {
      if (s == 0) a.tok[r] = a.unused_tok;
      if (s < L.S) a.idx[r * L.S + s] = 0;
    } else {
      if (s == 0) {
        if (a.flags != nullptr && id >= uint32_t(L.V0)) atomicOr(a.flags, NGRAM_FLAG_BAD_TOKEN);
        a.tok[r] = int32_t(id);
      }
      if (s < L.S) a.idx[r * L.S + s] = entry_index<NMAX>(L, e, j, s);
    }
  }
  if (a.n_commit == nullptr) return;
  __syncthreads();
  if (!active || !lead || !e.slot_ok) return;
  // commit the first n_commit[b] (<= n_new[b]) new ids
  if (commit_entry<NMAX>(L, a, e, acc) && a.flags != nullptr)
    atomicOr(a.flags, NGRAM_FLAG_BAD_COUNT);
}

// Batch entry b (sequence b of the packed tokens) fills cache slot slots[b] (or b).
__global__ __launch_bounds__(kThreads) void cache_init_kernel(
    int32_t nm1, int32_t* __restrict__ ring, int64_t* __restrict__ len,
    const int32_t* __restrict__ slots, int32_t nslots, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ cu, int32_t nbatch, int64_t ntok, int32_t* __restrict__ flags) {
  const int b = blockIdx.x * kThreads + threadIdx.x;
  const int slot = b < nbatch ? (slots != nullptr ? slots[b] : b) : -1;
  if (slots != nullptr) {                          // a slot used by an earlier entry: ignored
    __shared__ int32_t tile[kThreads];
    const int32_t bmax = min(nbatch, int32_t(blockIdx.x + 1) * kThreads);
    if (slot_seen_before(slots, bmax, b < nbatch ? b : 0, slot, 0, 1, tile, kThreads) &&
        b < nbatch && slot >= 0 && slot < nslots) {
      if (flags != nullptr) atomicOr(flags, NGRAM_FLAG_DUP_SLOT);
      return;
    }
  }
  if (b >= nbatch) return;
  if (slot < 0 || slot >= nslots) {
    if (flags != nullptr) atomicOr(flags, NGRAM_FLAG_BAD_SLOT);
    return;
  }
  int64_t lo = cu[b], hi = cu[b + 1];
  if (lo < 0 || hi < lo || hi > ntok) {
    if (flags != nullptr) atomicOr(flags, NGRAM_FLAG_BAD_SEQLENS);
    lo = lo < 0 ? 0 : (lo > ntok ? ntok : lo);
    hi = hi < lo ? lo : (hi > ntok ? ntok : hi);
  }
  const int64_t n = hi - lo;
  len[slot] = n;
  if (nm1 <= 0) return;
  int32_t* rb = ring + int64_t(slot) * nm1;
  for (int s = 0; s < nm1; ++s) rb[s] = 0;
  for (int64_t q = (n > nm1 ? n - nm1 : 0); q < n; ++q) rb[q % nm1] = tokens[lo + q];
}

__global__ __launch_bounds__(kThreads) void cache_commit_kernel(
    int32_t nm1, int32_t* __restrict__ ring, int64_t* __restrict__ len,
    const int32_t* __restrict__ slots, int32_t nslots, const int32_t* __restrict__ newtok,
    const int32_t* __restrict__ n_accept, int32_t nbatch, int32_t tmax,
    int32_t* __restrict__ flags) {
  const int b = blockIdx.x * kThreads + threadIdx.x;
  const int slot = b < nbatch ? (slots != nullptr ? slots[b] : b) : -1;
  if (slots != nullptr) {                          // a slot used by an earlier entry: ignored
    __shared__ int32_t tile[kThreads];
    const int32_t bmax = min(nbatch, int32_t(blockIdx.x + 1) * kThreads);
    if (slot_seen_before(slots, bmax, b < nbatch ? b : 0, slot, 0, 1, tile, kThreads) &&
        b < nbatch && slot >= 0 && slot < nslots) {
      if (flags != nullptr) atomicOr(flags, NGRAM_FLAG_DUP_SLOT);
      return;
    }
  }
  if (b >= nbatch) return;
  if (slot < 0 || slot >= nslots) {
    if (flags != nullptr) atomicOr(flags, NGRAM_FLAG_BAD_SLOT);
    return;
  }
  int a = n_accept[b];
  if (a < 0 || a > tmax) {
    if (flags != nullptr) atomicOr(flags, NGRAM_FLAG_BAD_COUNT);
    a = a < 0 ? 0 : tmax;
  }
  int64_t committed = len[slot];
  if (committed < 0) committed = 0;
  if (nm1 > 0) {
    int32_t* rb = ring + int64_t(slot) * nm1;
    const int32_t* nt = newtok + int64_t(b) * tmax;
    for (int q = (a > nm1 ? a - nm1 : 0); q < a; ++q) rb[(committed + q) % nm1] = nt[q];
  }
  len[slot] = committed + a;
}

__global__ void clear_flags_kernel(int32_t* flags) { flags[0] = 0; }

// ------------------------------------------------------------------ hash statistics
// Collisions and table hit counts of one order n (section 3.2.2 and Fig. 3 of the same
// page), exact integers throughout. Rows in use: one bit per table row for each table size,
// set by every position whose n-gram lands on it (a plain load first, so the repeats of
// frequent n-grams do not queue atomics on one word), then the set bits are counted.
// Distinct n-grams: the exact n-gram values (V0^n <= 2^63) are sorted and the boundaries
// counted.

__global__ __launch_bounds__(kThreads) void zero_words_kernel(uint32_t* __restrict__ w,
                                                              int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (i < n) w[i] = 0u;
}

__global__ void zero_counts_kernel(int64_t* __restrict__ rows, int32_t nvocab,
                                   int64_t* __restrict__ distinct) {
  for (int v = threadIdx.x; v < nvocab; v += blockDim.x) rows[v] = 0;
  if (threadIdx.x == 0 && distinct != nullptr) *distinct = 0;
}

template <int NMAX>
__global__ __launch_bounds__(kThreads) void hash_slots_kernel(
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ cu, int32_t nseq,
    int64_t ntok, int64_t V0, int32_t n, const SlotArgs a, uint32_t* __restrict__ bits,
    int32_t* __restrict__ flags) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  uint32_t c[NMAX];
  if (!position_context<NMAX>(tokens, cu, nseq, ntok, V0, n, i, flags, c)) return;
  for (int v = 0; v < a.nv; ++v) {
    const uint64_t V = a.V[v], m = a.Vinv[v];
    uint64_t x = 0;
#pragma unroll
    for (int j = NMAX - 1; j >= 0; --j)
      if (j < n) x = horner_step(x, uint64_t(V0), c[j], V, m);
    uint32_t* word = bits + a.word_off[v] + (x >> 5);
    const uint32_t mask = 1u << (x & 31u);
    if ((*word & mask) == 0u) atomicOr(word, mask);
  }
}

// Exact n-gram values (Horner's rule without reduction; exact when V0^n <= 2^63) and the
// positions, for the sort.
template <int NMAX>
__global__ __launch_bounds__(kThreads) void ngram_values_kernel(
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ cu, int32_t nseq,
    int64_t ntok, int64_t V0, int32_t n, uint64_t* __restrict__ keys,
    uint32_t* __restrict__ vals) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  uint32_t c[NMAX];
  if (!position_context<NMAX>(tokens, cu, nseq, ntok, V0, n, i, nullptr, c)) return;
  uint64_t x = 0;
#pragma unroll
  for (int j = NMAX - 1; j >= 0; --j)
    if (j < n) x = x * uint64_t(V0) + c[j];
  keys[i] = x;
  vals[i] = uint32_t(i);
}

// Block sum of one value per thread (kThreads threads), returned to thread 0.
__device__ __forceinline__ uint64_t block_sum(uint64_t v) {
  __shared__ uint64_t part[kThreads / 64];
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  uint64_t t = 0;
  if (threadIdx.x == 0)
    for (int w = 0; w < kThreads / 64; ++w) t += part[w];
  return t;
}

// Sorted values: 1 for each first occurrence.
__global__ __launch_bounds__(kThreads) void count_distinct_kernel(
    const uint64_t* __restrict__ keys, int64_t n, int64_t* __restrict__ distinct) {
  uint64_t c = 0;
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * kThreads)
    c += (i == 0 || keys[i] != keys[i - 1]) ? 1u : 0u;
  const uint64_t t = block_sum(c);
  if (threadIdx.x == 0 && t != 0)
    atomicAdd(reinterpret_cast<unsigned long long*>(distinct), (unsigned long long)t);
}

// Set bits of each table size's bitmap (blockIdx.y: size v of the launch).
__global__ __launch_bounds__(kThreads) void count_rows_kernel(const uint32_t* __restrict__ bits,
                                                              const SlotArgs a,
                                                              int64_t* __restrict__ rows) {
  const int v = blockIdx.y;
  const int64_t lo = a.word_off[v], hi = a.word_off[v + 1];
  uint64_t c = 0;
  for (int64_t w = lo + int64_t(blockIdx.x) * kThreads + threadIdx.x; w < hi;
       w += int64_t(gridDim.x) * kThreads)
    c += __popc(bits[w]);
  const uint64_t t = block_sum(c);
  if (threadIdx.x == 0 && t != 0)
    atomicAdd(reinterpret_cast<unsigned long long*>(rows + v), (unsigned long long)t);
}

template <int NMAX>
hipError_t hash_stats_n(const StatsArgs& s, hipStream_t st) {
  const int64_t work = s.ntok > int64_t(s.nseq) + 1 ? s.ntok : int64_t(s.nseq) + 1;
  const unsigned blocks = unsigned((work + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(zero_counts_kernel, dim3(1), dim3(kThreads), 0, st, s.rows, s.nvocab,
                     s.distinct);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // table sizes in groups of kStatsGroup per launch
  for (int32_t v0 = 0; v0 < s.nvocab; v0 += kStatsGroup) {
    SlotArgs a{};
    a.nv = s.nvocab - v0 < kStatsGroup ? s.nvocab - v0 : kStatsGroup;
    uint64_t words = 0;
    for (int v = 0; v < a.nv; ++v) {
      a.V[v] = uint64_t(s.vocab[v0 + v]);
      a.Vinv[v] = ~uint64_t(0) / a.V[v];
      a.word_off[v] = words;
      words += (a.V[v] + 31) / 32;
    }
    a.word_off[a.nv] = words;
    hipLaunchKernelGGL(zero_words_kernel, dim3(unsigned((words + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, st, s.bits, int64_t(words));
    hipLaunchKernelGGL(hash_slots_kernel<NMAX>, dim3(blocks), dim3(kThreads), 0, st, s.tokens,
                       s.cu, s.nseq, s.ntok, s.V0, s.n, a, s.bits, v0 == 0 ? s.flags : nullptr);
    hipLaunchKernelGGL(count_rows_kernel, dim3(256, unsigned(a.nv)), dim3(kThreads), 0, st,
                       s.bits, a, s.rows + v0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (s.distinct == nullptr || s.ntok == 0) return hipSuccess;
  hipLaunchKernelGGL(ngram_values_kernel<NMAX>, dim3(blocks), dim3(kThreads), 0, st, s.tokens,
                     s.cu, s.nseq, s.ntok, s.V0, s.n, s.keys0, s.vals0);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  e = launch_radix_sort(s.keys0, s.vals0, s.keys1, s.vals1, s.hist, s.ntok, s.key_bits, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(count_distinct_kernel, dim3(1024), dim3(kThreads), 0, st, s.keys0, s.ntok,
                     s.distinct);
  return hipGetLastError();
}

template <int NMAX>
hipError_t hash_prefill_n(const LayerDesc& L, const int32_t* tokens, const int32_t* cu,
                          int32_t nseq, int64_t ntok, int32_t* idx, int32_t* flags,
                          hipStream_t st) {
  const int64_t work = (ntok > int64_t(nseq) + 1 ? ntok : int64_t(nseq) + 1) * L.S;
  const unsigned blocks = unsigned((work + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(hash_prefill_kernel<NMAX>, dim3(blocks), dim3(kThreads), 0, st, L, tokens,
                     cu, nseq, ntok, idx, flags);
  return hipGetLastError();
}

template <int NMAX>
hipError_t hash_decode_n(const LayerDesc& L, const DecodeArgs& a, hipStream_t st) {
  const int tpe = a.width * (L.S > 0 ? L.S : 1);
  if (tpe > kDecThreads) return hipErrorInvalidValue;   // width <= 8 and S <= 64 keep it in
  const int epb = kDecThreads / tpe;
  const unsigned blocks = unsigned((a.nbatch + epb - 1) / epb);
  hipLaunchKernelGGL(hash_decode_kernel<NMAX>, dim3(blocks), dim3(kDecThreads), 0, st, L, a);
  return hipGetLastError();
}

}  // namespace

// The context length N is a template bound so the id window lives in registers.
hipError_t launch_hash_prefill(const LayerDesc& L, const int32_t* tokens, const int32_t* cu,
                               int32_t nseq, int64_t ntok, int32_t* idx, int32_t* flags,
                               hipStream_t st) {
  if (L.N <= 2) return hash_prefill_n<2>(L, tokens, cu, nseq, ntok, idx, flags, st);
  if (L.N <= 4) return hash_prefill_n<4>(L, tokens, cu, nseq, ntok, idx, flags, st);
  if (L.N <= 8) return hash_prefill_n<8>(L, tokens, cu, nseq, ntok, idx, flags, st);
  return hash_prefill_n<NGRAM_MAX_ORDER>(L, tokens, cu, nseq, ntok, idx, flags, st);
}

hipError_t launch_hash_stats(const StatsArgs& s, hipStream_t st) {
  if (s.n <= 2) return hash_stats_n<2>(s, st);
  if (s.n <= 4) return hash_stats_n<4>(s, st);
  if (s.n <= 8) return hash_stats_n<8>(s, st);
  return hash_stats_n<NGRAM_MAX_ORDER>(s, st);
}

hipError_t launch_hash_decode(const LayerDesc& L, const DecodeArgs& a, hipStream_t st) {
  if (a.nbatch <= 0 || a.width <= 0) return hipSuccess;
  if (L.N <= 2) return hash_decode_n<2>(L, a, st);
  if (L.N <= 4) return hash_decode_n<4>(L, a, st);
  if (L.N <= 8) return hash_decode_n<8>(L, a, st);
  return hash_decode_n<NGRAM_MAX_ORDER>(L, a, st);
}

hipError_t launch_cache_init(const LayerDesc& L, int32_t* ring, int64_t* len,
                             const int32_t* slots, int32_t nslots, const int32_t* tokens,
                             const int32_t* cu, int32_t nbatch, int64_t ntok, int32_t* flags,
                             hipStream_t st) {
  const unsigned blocks = unsigned((nbatch + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(cache_init_kernel, dim3(blocks), dim3(kThreads), 0, st, L.N - 1, ring, len,
                     slots, nslots, tokens, cu, nbatch, ntok, flags);
  return hipGetLastError();
}

hipError_t launch_cache_commit(const LayerDesc& L, int32_t* ring, int64_t* len,
                               const int32_t* slots, int32_t nslots, const int32_t* newtok,
                               const int32_t* n_accept, int32_t nbatch, int32_t tmax,
                               int32_t* flags, hipStream_t st) {
  const unsigned blocks = unsigned((nbatch + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(cache_commit_kernel, dim3(blocks), dim3(kThreads), 0, st, L.N - 1, ring,
                     len, slots, nslots, newtok, n_accept, nbatch, tmax, flags);
  return hipGetLastError();
}

hipError_t launch_clear_flags(int32_t* flags, hipStream_t st) {
  hipLaunchKernelGGL(clear_flags_kernel, dim3(1), dim3(1), 0, st, flags);
  return hipGetLastError();
}

}  // namespace ngram
