// Internal launch interface between the C-ABI entry points and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "layer_desc.h"

namespace ngram {

// kernel 1: rolling-hash indices of packed prefill positions
hipError_t launch_hash_prefill(const LayerDesc& L, const int32_t* tokens, const int32_t* cu,
                               int32_t nseq, int64_t ntok, int32_t* idx, int32_t* flags,
                               hipStream_t st);

// Token of a row that must not be written (rows outside a decode window's n_new).
constexpr int32_t kSkipRow = -2;

// kernel 4 (front half): context from the N-gram cache + new ids -> tok, idx for the rows
// [row_begin, row_begin + width) of every batch entry (compact: b * width + j - row_begin);
// then, if n_commit is not null, the step's commit into the cache
struct DecodeArgs {
  int32_t* ring;            // [nslots, N-1]
  int64_t* len;             // [nslots]
  const int32_t* slots;     // [nbatch] cache slot of each batch entry, or null (slot b)
  int32_t nslots;
  const int32_t* newtok;    // [nbatch, tmax]
  const int32_t* n_new;     // [nbatch]
  const int32_t* n_commit;  // [nbatch] or null
  int32_t nbatch, tmax, row_begin, width;
  int32_t unused_tok;       // token of rows past n_new: -1 (zero row) or kSkipRow
  int32_t* tok;             // [nbatch * width]
  int32_t* idx;             // [nbatch * width, S]
  int32_t* flags;
};
hipError_t launch_hash_decode(const LayerDesc& L, const DecodeArgs& a, hipStream_t st);

// kernel 4 (cache upkeep); slots as above
hipError_t launch_cache_init(const LayerDesc& L, int32_t* ring, int64_t* len,
                             const int32_t* slots, int32_t nslots, const int32_t* tokens,
                             const int32_t* cu, int32_t nbatch, int64_t ntok, int32_t* flags,
                             hipStream_t st);
hipError_t launch_cache_commit(const LayerDesc& L, int32_t* ring, int64_t* len,
                               const int32_t* slots, int32_t nslots, const int32_t* newtok,
                               const int32_t* n_accept, int32_t nbatch, int32_t tmax,
                               int32_t* flags, hipStream_t st);

// hash statistics of order n over packed sequences (collisions, table hit counts): rows[v]
// = distinct rows (n-gram value mod vocab[v]) in use; distinct (if not null) = distinct
// n-grams, from exact values (V0^n <= 2^63, key_bits their width) sorted in keys/vals
struct SlotArgs {
  uint64_t V[kStatsGroup];
  uint64_t Vinv[kStatsGroup];          // floor((2^64 - 1) / V): Barrett multipliers
  uint64_t word_off[kStatsGroup + 1];  // bitmap of size v: words [word_off[v], word_off[v+1])
  int32_t nv;
};
struct StatsArgs {
  const int32_t* tokens;
  const int32_t* cu;
  int32_t nseq;
  int64_t ntok;
  int64_t V0;
  int32_t n;
  const int64_t* vocab;   // host [nvocab]
  int32_t nvocab;
  int64_t* rows;          // device [nvocab]
  int64_t* distinct;      // device [1] or null
  uint32_t* bits;         // bitmaps of kStatsGroup sizes at a time
  uint64_t* keys0;
  uint64_t* keys1;
  uint32_t* vals0;
  uint32_t* vals1;
  uint32_t* hist;
  int32_t key_bits;
  int32_t* flags;
};
hipError_t launch_hash_stats(const StatsArgs& s, hipStream_t st);

// stable LSD radix sort of n (key, value) pairs by the low `bits` key bits, 8 per pass;
// result in k0/v0, k1/v1 scratch, hist [m + ceil(m / 1024)] with m = 256 * ceil(n / 4096)
hipError_t launch_radix_sort(uint64_t* k0, uint32_t* v0, uint64_t* k1, uint32_t* v1,
                             uint32_t* hist, int64_t n, int bits, hipStream_t st);

// Where the final output rows go: compact row m is written to row
// (m / group) * stride + off + m % group of `out` (group 0: row m). Rows whose token is
// kSkipRow are not written.
struct RowMap {
  int32_t group = 0, stride = 0, off = 0;
};
hipError_t launch_clear_flags(int32_t* flags, hipStream_t st);

// kernel 2: stand-alone gather of sub-table rows into G [nrows, D]
hipError_t launch_gather(const LayerDesc& L, const void* const* E, const int32_t* idx,
                         int64_t nrows, void* G, hipStream_t st);

// kernel 2 into LDS: the gather the projection performs (global_load_lds_dwordx4), each
// gathered row reduced where it lands to sums[r] = sum_k w_k (2k + 1) mod 2^32 over its
// 32-bit words
hipError_t launch_gather_lds(const LayerDesc& L, const void* const* E, const int32_t* idx,
                             int64_t nrows, uint32_t* sums, hipStream_t st);

// kernels 2+3: fused gather + projection + E_0 epilogue (times the output factor); with
// f32out, `out` is fp32 [nrows, D] and holds the unrounded rows
hipError_t launch_project(const LayerDesc& L, const void* E0, const void* const* E,
                          const void* W, const int32_t* idx, const int32_t* tok,
                          int64_t nrows, void* out, bool f32out, const RowMap& map,
                          hipStream_t st);

// Per-layer embeddings: the tables and output of one layer. Layers share the config, the
// rows and the hash indices; the projections of up to kMaxLaunchLayers layers (at most
// kMaxLaunchTables sub-table pointers in all) run in one launch.
struct LayerParams {
  const void* E0;
  const void* const* E;   // host array of S device pointers
  const void* W;
  void* out;
};
constexpr int kMaxLaunchLayers = 8;
constexpr int kMaxLaunchTables = 128;
hipError_t launch_project_layers(const LayerDesc& L, const LayerParams* layers, int32_t nlayers,
                                 const int32_t* idx, const int32_t* tok, int64_t nrows,
                                 bool f32out, const RowMap& map, hipStream_t st);

// the basic form (Eq. 1): out = (E_0 row + the S full-width table rows) / (S + 1), times the
// output factor; f32out and map as for launch_project (which calls it in that form)
hipError_t launch_basic(const LayerDesc& L, const void* E0, const void* const* E,
                        const int32_t* idx, const int32_t* tok, int64_t nrows, void* out,
                        bool f32out, const RowMap& map, hipStream_t st);

// dense product for the backward: out = inv * A B^T (fp32, overwritten) or, with
// accumulate, out += inv * A B^T through `splits` fp32 partial sums in `part`
// ([splits, M, ldo]) added in split order. A [M, K] and B [N, K] row-major in the config
// dtype; ident: int32 [M] = 0..M-1.
hipError_t launch_dense_product(const LayerDesc& L, const void* A, int64_t M, const void* B,
                                int32_t N, int32_t K, const int32_t* ident, float* out,
                                int64_t ldo, float inv, bool accumulate, float* part,
                                int32_t splits, hipStream_t st);

// backward (training): gradients accumulated into fp32 buffers; the workspace pieces
// follow BwLayout
struct BackwardArgs {
  const void* const* E;   // sub-tables (host array of S device pointers)
  const void* W;          // [D, D] stacked
  const int32_t* tokens;  // [rows]
  const int32_t* idx;     // [rows, S] (hash indices, computed first)
  const void* dout;       // [rows, D] upstream gradient, config dtype
  float* dE0;             // [V0, D] or null
  float* const* dE;       // host array of S device pointers [V_s, d], or null
  float* dW;              // [D, D] or null
  int64_t rows;
  int32_t* ident;         // workspace pieces
  void* WT;
  void* doutT;
  void* GT;
  float* dG;
  float* part;
  uint64_t* keys0;
  uint64_t* keys1;
  uint32_t* vals0;
  uint32_t* vals1;
  uint32_t* hist;
  float* head;
  float* tail;
  uint32_t* owners;
};
hipError_t launch_backward(const LayerDesc& L, const BackwardArgs& b, hipStream_t st);

// amplification by layer normalisation: pre fp32 [nrows, D] -> out [nrows, D] (config dtype);
// weight / bias: [D] in the config dtype or null
hipError_t launch_layernorm(const LayerDesc& L, const float* pre, const int32_t* tok,
                            const void* weight, const void* bias, int64_t nrows, void* out,
                            const RowMap& map, hipStream_t st);

}  // namespace ngram
