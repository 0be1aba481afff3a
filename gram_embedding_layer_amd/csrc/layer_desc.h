// Host-checked description of one N-gram embedding layer, passed by value to kernels.
// HIP-free so the host validation can be built and tested with a plain C++ compiler.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "ngram_embed.h"

namespace ngram {

struct LayerDesc {
  int32_t N;       // largest order
  int32_t K;       // sub-tables per order
  int32_t S;       // (N-1)K
  int32_t D;       // hidden size
  int32_t d;       // sub-table width: D/S in the final form, D in the basic form (0 when S == 0)
  int32_t form;    // NGRAM_FORM_FINAL / NGRAM_FORM_BASIC
  int32_t dtype;   // NGRAM_F32 / NGRAM_BF16
  int32_t esz;     // bytes per element
  int32_t V0;      // base vocabulary
  uint32_t V[NGRAM_MAX_SUBTABLES];  // V_{n,k} in sub-table order
  uint64_t Vinv[NGRAM_MAX_SUBTABLES];  // floor((2^64 - 1) / V_{n,k}): Barrett multiplier
  int32_t amp;     // NGRAM_AMP_NONE / SCALE / LAYERNORM
  float scale;     // output factor: amp_scale with NGRAM_AMP_SCALE, else 1
  float ln_eps;    // layer-normalisation epsilon (NGRAM_AMP_LAYERNORM)
};

// Largest D the layer normalisation accepts (a row in the registers of one block).
constexpr int32_t kMaxNormD = 8192;

// Checks the config (section A2 shapes, the 64-bit Horner bound) and fills `out`.
// Returns NGRAM_OK or a negative status.
int describe(const ngram_embed_config* cfg, LayerDesc* out);

// Workspace layout for `rows` output rows; false when rows < 0.
struct WsLayout {
  size_t tok_off, idx_off, pre_off, total;  // pre_off: fp32 [rows, D] (layer norm only)
};
bool ws_layout(const LayerDesc& L, int64_t rows, WsLayout* out);

// Backward (training) workspace: the hash indices, identity indices, W^T, dout^T and G^T
// (tokens padded to a multiple of 64), dG = c dout W (fp32), the split partial sums of dW,
// the radix-sort buffers and the partial sums of the segmented reduction.
constexpr int kSortTile = 4096;   // keys per radix-sort block
constexpr int kChunk = 32;        // sorted entries per segmented-reduction chunk
struct BwLayout {
  size_t idx_off, ident_off, wt_off, doutt_off, gt_off, dg_off, part_off;
  size_t keys0_off, keys1_off, vals0_off, vals1_off, hist_off, head_off, tail_off, owners_off;
  size_t total;
};
// contraction ranges of dW (c dout^T G, contracted over the rows)
int32_t backward_splits(const LayerDesc& L, int64_t rows);
bool bw_layout(const LayerDesc& L, int64_t rows, BwLayout* out);

// Hash statistics (collisions and table hit counts of one order n) over ntok positions:
// bitmaps of the table sizes (one group of kStatsGroup sizes at a time), and, when the exact
// n-gram values fit (V0^n <= 2^63: `exact`, `key_bits` their width), the sort buffers.
constexpr int kStatsGroup = 32;
struct StatsLayout {
  size_t bits_off, keys0_off, keys1_off, vals0_off, vals1_off, hist_off, total;
  bool exact;
  int32_t key_bits;
};
// NGRAM_OK, or NGRAM_EINVAL for out-of-range arguments (vocab: host [nvocab]).
int stats_layout(int64_t V0, int32_t n, int64_t ntok, const int64_t* vocab, int32_t nvocab,
                 StatsLayout* out);

inline bool aligned(const void* p, size_t a) {
  return p != nullptr && (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

}  // namespace ngram
