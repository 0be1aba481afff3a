// Internal launch interface between the C-ABI entry points and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "layer_desc.h"

namespace ngram {

// kernel 1: rolling-hash indices of packed prefill positions
hipError_t launch_hash_prefill(const LayerDesc& L, const int32_t* tokens, const int32_t* cu,
                               int32_t nseq, int64_t ntok, int32_t* idx, int32_t* flags,
                               hipStream_t st);

// kernel 4 (front half): context from the N-gram cache + new ids -> tok, idx; then, if
// n_commit is not null, the step's commit into the cache
hipError_t launch_hash_decode(const LayerDesc& L, int32_t* ring, int64_t* len,
                              const int32_t* newtok, const int32_t* n_new,
                              const int32_t* n_commit, int32_t nseq, int32_t tmax, int32_t* tok,
                              int32_t* idx, int32_t* flags, hipStream_t st);

// kernel 4 (cache upkeep)
hipError_t launch_cache_init(const LayerDesc& L, int32_t* ring, int64_t* len,
                             const int32_t* tokens, const int32_t* cu, int32_t nseq,
                             int64_t ntok, int32_t* flags, hipStream_t st);
hipError_t launch_cache_commit(const LayerDesc& L, int32_t* ring, int64_t* len,
                               const int32_t* newtok, const int32_t* n_accept,
                               const int32_t* n_new, int32_t nseq, int32_t tmax,
                               int32_t* flags, hipStream_t st);
hipError_t launch_clear_flags(int32_t* flags, hipStream_t st);

// kernel 2: stand-alone gather of sub-table rows into G [nrows, D]
hipError_t launch_gather(const LayerDesc& L, const void* const* E, const int32_t* idx,
                         int64_t nrows, void* G, hipStream_t st);

// kernels 2+3: fused gather + projection + E_0 epilogue (times the output factor); with
// f32out, `out` is fp32 [nrows, D] and holds the unrounded rows
hipError_t launch_project(const LayerDesc& L, const void* E0, const void* const* E,
                          const void* W, const int32_t* idx, const int32_t* tok,
                          int64_t nrows, void* out, bool f32out, hipStream_t st);

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
                            hipStream_t st);

}  // namespace ngram
