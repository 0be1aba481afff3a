// Device code of the decode step's hash kernel and the exact Horner step it shares with the
// prefill hash (the rolling hash of section A2 of the deep-notes page on "Scaling Embeddings
// Outperforms Scaling Experts in Language Models"): what one batch entry of a decode step
// reads from and appends to the N-gram cache (section 4.2: the last N-1 committed ids of
// every sequence kept on the device).
#pragma once

#include "kernels.h"

namespace ngram {

// One Horner step, exactly: (x*V0 + t) mod V for x < V < 2^31, V0 < 2^31, t < 2^32, so
// y = x*V0 + t < 2^63. With m = floor((2^64 - 1) / V), q = floor(y*m / 2^64) satisfies
// floor(y/V) - 1 <= q <= floor(y/V) (y*m/2^64 > y/V - y/2^64 - y/(V 2^64) > y/V - 1), so
// r = y - q*V lies in [0, 2V) and one conditional subtraction leaves y mod V.
__device__ __forceinline__ uint64_t horner_step(uint64_t x, uint64_t V0, uint32_t t, uint64_t V,
                                                uint64_t m) {
  const uint64_t y = x * V0 + t;
  const uint64_t q = __umul64hi(y, m);
  uint64_t r = y - q * V;
  if (r >= V) r -= V;
  return r;
}

// Batch entry b of a decode step as its rows read it: the cache slot (slots[b], or b), the
// step's new-id count n_new[b] clamped into [0, tmax] (`bad_count` when it was outside),
// the committed length, the ring row (the last N-1 committed ids; N <= NMAX) and the new
// ids at positions <= jmax. Every load is issued before any is used.
template <int NMAX>
struct DecodeEntry {
  int32_t slot, nn;
  bool slot_ok, bad_count;
  int64_t committed;
  int32_t cm;            // committed mod (N-1): ring slot of the next committed id
  uint32_t ringv[NMAX > 1 ? NMAX - 1 : 1];
  uint32_t newv[NGRAM_MAX_DECODE_TOKENS];
};

template <int NMAX>
__device__ __forceinline__ DecodeEntry<NMAX> load_entry(const LayerDesc& L, const DecodeArgs& a,
                                                       int b, int jmax) {
  DecodeEntry<NMAX> e;
  const int nm1 = L.N - 1;
  e.slot = a.slots != nullptr ? a.slots[b] : b;
  e.slot_ok = e.slot >= 0 && e.slot < a.nslots;
  const int32_t nn = a.n_new[b];
#pragma unroll
  for (int q = 0; q < (NMAX > 1 ? NMAX - 1 : 1); ++q)
    e.ringv[q] = e.slot_ok && q < nm1 ? uint32_t(a.ring[int64_t(e.slot) * nm1 + q]) : 0u;
  e.committed = e.slot_ok ? a.len[e.slot] : 0;
  const int32_t* nt = a.newtok + int64_t(b) * a.tmax;
#pragma unroll
  for (int q = 0; q < NGRAM_MAX_DECODE_TOKENS; ++q)
    e.newv[q] = q < a.tmax && q <= jmax ? uint32_t(nt[q]) : 0u;
  e.bad_count = nn < 0 || nn > a.tmax;
  e.nn = nn < 0 ? 0 : (nn > a.tmax ? a.tmax : nn);
  if (e.committed < 0) e.committed = 0;
  // the only 64-bit division of the entry (a software routine on the GPU)
  e.cm = nm1 > 0 ? int32_t(e.committed % nm1) : 0;
  return e;
}

// Whether row j of the entry is computed this step (a new id in a valid slot); *id its id.
template <int NMAX>
__device__ __forceinline__ bool entry_row(const DecodeEntry<NMAX>& e, int j, uint32_t* id) {
  uint32_t t = 0;
#pragma unroll
  for (int q = 0; q < NGRAM_MAX_DECODE_TOKENS; ++q)
    if (q == j) t = e.newv[q];
  *id = t;
  return j < e.nn && e.slot_ok;
}

// Context of a computed row j: c[i] = t_{j-i} for i < N (the older ids from the ring, pad id
// 0 before the sequence start), 0 for i >= N.
template <int NMAX>
__device__ __forceinline__ void entry_context(const LayerDesc& L, const DecodeEntry<NMAX>& e,
                                              int j, uint32_t (&c)[NMAX]) {
  const int nm1 = L.N - 1;
#pragma unroll
  for (int i = 0; i < NMAX; ++i) {
    uint32_t v = 0;
    if (i < L.N) {
      if (j - i >= 0) {
#pragma unroll
        for (int q = 0; q < NGRAM_MAX_DECODE_TOKENS; ++q)   // a new id of this step
          if (q == j - i) v = e.newv[q];
      } else if (e.committed + (j - i) >= 0) {             // a committed position p:
        int u = e.cm + (j - i);                             // p mod (N-1), as -(N-1) <= j-i < 0
        if (u < 0) u += nm1;
#pragma unroll
        for (int q = 0; q < (NMAX > 1 ? NMAX - 1 : 1); ++q)
          if (q == u) v = e.ringv[q];
      }
    }
    c[i] = v;
  }
}

// H_{n,k} for sub-table s (n = 2 + s / K) of a row with context c: its last n ids reduced
// by Horner's rule from the oldest id to the newest.
template <int NMAX>
__device__ __forceinline__ int32_t context_hash(const LayerDesc& L, const uint32_t (&c)[NMAX],
                                                int s) {
  const int n = 2 + s / L.K;
  const uint64_t V = L.V[s], m = L.Vinv[s];
  uint64_t x = 0;
#pragma unroll
  for (int i = NMAX - 1; i >= 0; --i)
    if (i < n) x = horner_step(x, uint64_t(L.V0), c[i], V, m);
  return int32_t(x);
}

// H_{n,k} of a computed row j for sub-table s.
template <int NMAX>
__device__ __forceinline__ int32_t entry_index(const LayerDesc& L, const DecodeEntry<NMAX>& e,
                                               int j, int s) {
  uint32_t c[NMAX];
  entry_context<NMAX>(L, e, j, c);
  return context_hash<NMAX>(L, c, s);
}

// Append the entry's first `acc` new ids (clamped into [0, nn]) to its slot: the ring keeps
// the last N-1, len advances. The entry must have been loaded with every new id (jmax >=
// tmax - 1) and a valid slot. Returns whether acc was out of range.
template <int NMAX>
__device__ __forceinline__ bool commit_entry(const LayerDesc& L, const DecodeArgs& a,
                                             const DecodeEntry<NMAX>& e, int acc) {
  const bool bad = acc < 0 || acc > e.nn;
  if (bad) acc = acc < 0 ? 0 : e.nn;
  const int nm1 = L.N - 1;
  if (nm1 > 0) {
    int32_t* rb = a.ring + int64_t(e.slot) * nm1;
#pragma unroll
    for (int q = 0; q < NGRAM_MAX_DECODE_TOKENS; ++q)
      if (q < acc && q >= acc - nm1) rb[(e.cm + q) % nm1] = int32_t(e.newv[q]);
  }
  a.len[e.slot] = e.committed + acc;
  return bad;
}

}  // namespace ngram
