// Host-side validation of the layer config and workspace layout (no HIP calls).
#include <cmath>

#include "layer_desc.h"

namespace ngram {

int describe(const ngram_embed_config* cfg, LayerDesc* out) {
  if (cfg == nullptr || out == nullptr) return NGRAM_EINVAL;
  if (cfg->N < 1 || cfg->N > NGRAM_MAX_ORDER || cfg->K < 1) return NGRAM_EINVAL;
  const int64_t S = int64_t(cfg->N - 1) * cfg->K;
  if (S > NGRAM_MAX_SUBTABLES) return NGRAM_EINVAL;
  if (cfg->dtype != NGRAM_F32 && cfg->dtype != NGRAM_BF16) return NGRAM_EDTYPE;
  const int esz = cfg->dtype == NGRAM_F32 ? 4 : 2;
  if (cfg->D < 1 || cfg->V0 < 1 || cfg->V0 >= (int64_t(1) << 31)) return NGRAM_EINVAL;
  if ((int64_t(cfg->D) * esz) % 16 != 0) return NGRAM_EINVAL;
  LayerDesc L{};
  L.N = cfg->N;
  L.K = cfg->K;
  L.S = int32_t(S);
  L.D = cfg->D;
  L.dtype = cfg->dtype;
  L.esz = esz;
  L.V0 = int32_t(cfg->V0);
  // The final form, or the basic form of Eq. 1 (one full-width table per order).
  if (cfg->form != NGRAM_FORM_FINAL && cfg->form != NGRAM_FORM_BASIC) return NGRAM_EINVAL;
  if (cfg->form == NGRAM_FORM_BASIC && cfg->K != 1) return NGRAM_EINVAL;
  L.form = cfg->form;
  if (S > 0) {
    // Sub-table width D/((N-1)K) (section A2), or D in the basic form; rows must be whole
    // 16-byte vectors.
    if (L.form == NGRAM_FORM_FINAL && cfg->D % S != 0) return NGRAM_EINVAL;
    L.d = L.form == NGRAM_FORM_BASIC ? cfg->D : int32_t(cfg->D / S);
    if ((int64_t(L.d) * esz) % 16 != 0) return NGRAM_EINVAL;
    if (cfg->V == nullptr) return NGRAM_EINVAL;
    uint64_t vmax = 0;
    for (int s = 0; s < S; ++s) {
      const int64_t v = cfg->V[s];
      if (v < 1 || v >= (int64_t(1) << 31)) return NGRAM_EINVAL;
      L.V[s] = uint32_t(v);
      L.Vinv[s] = ~uint64_t(0) / uint64_t(v);
      if (uint64_t(v) > vmax) vmax = uint64_t(v);
    }
    // Horner step x*V0 + t with x < V, t < V0 stays below V*V0 <= 2^63 - 1.
    if (vmax > ((uint64_t(1) << 63) - 1) / uint64_t(cfg->V0)) return NGRAM_EOVERFLOW;
  }
  // Embedding amplification (section 3.2.4): a finite output factor, or a layer
  // normalisation with a positive epsilon over rows that fit one block's LDS.
  L.amp = cfg->amp;
  L.scale = 1.0f;
  L.ln_eps = 0.0f;
  if (cfg->amp == NGRAM_AMP_SCALE) {
    if (!std::isfinite(cfg->amp_scale)) return NGRAM_EINVAL;
    // the sentinel selects the pages' factor sqrt(D) (section 3.2.4)
    L.scale = cfg->amp_scale == NGRAM_AMP_SCALE_SQRT_D ? std::sqrt(float(cfg->D))
                                                       : cfg->amp_scale;
  } else if (cfg->amp == NGRAM_AMP_LAYERNORM) {
    if (!std::isfinite(cfg->ln_eps) || !(cfg->ln_eps > 0.0f)) return NGRAM_EINVAL;
    if (cfg->D > kMaxNormD) return NGRAM_EINVAL;
    L.ln_eps = cfg->ln_eps;
  } else if (cfg->amp != NGRAM_AMP_NONE) {
    return NGRAM_EINVAL;
  }
  *out = L;
  return NGRAM_OK;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool ws_layout(const LayerDesc& L, int64_t rows, WsLayout* out) {
  if (rows < 0) return false;
  WsLayout w;
  w.tok_off = 256;
  w.idx_off = w.tok_off + align256(size_t(rows) * 4);
  w.pre_off = w.idx_off + align256(size_t(rows) * size_t(L.S) * 4);
  w.total = w.pre_off +
            (L.amp == NGRAM_AMP_LAYERNORM ? align256(size_t(rows) * size_t(L.D) * 4) : 0);
  *out = w;
  return true;
}

int32_t backward_splits(const LayerDesc& L, int64_t rows) {
  // the matrix-core path only (bf16, whole 256-wide output tiles): about four waves of
  // blocks over the 256 CUs, at most 8 ranges and at least 4 slices per range
  if (L.dtype != NGRAM_BF16 || L.D % 256 != 0 || rows <= 0) return 1;
  const int64_t tiles = int64_t(L.D / 256) * (L.D / 256);
  const int64_t slices = (rows + 63) / 64;
  int64_t sp = (1024 + tiles / 2) / tiles;
  const int64_t cap = slices / 4 < 8 ? slices / 4 : 8;
  if (sp > cap) sp = cap;
  return sp < 1 ? 1 : int32_t(sp);
}

bool bw_layout(const LayerDesc& L, int64_t rows, BwLayout* out) {
  if (rows < 0) return false;
  const size_t T = size_t(rows), D = size_t(L.D), S = size_t(L.S), esz = size_t(L.esz);
  const size_t Tp = (T + 63) / 64 * 64;
  const size_t nsort = T * (S > 1 ? S : 1);
  const size_t nblocks = (nsort + kSortTile - 1) / kSortTile;
  const size_t seg_s = (T * S + kChunk - 1) / kChunk * size_t(L.d);
  const size_t seg_0 = (T + kChunk - 1) / kChunk * D;
  const size_t seg = seg_s > seg_0 ? seg_s : seg_0;
  const bool tables = S > 0 && L.form == NGRAM_FORM_FINAL;   // the products' operands
  BwLayout w;
  size_t o = 256;                                    // error flags
  auto take = [&](size_t bytes) { const size_t at = o; o += align256(bytes); return at; };
  w.idx_off = take(T * S * 4);
  w.ident_off = take((T > D ? T : D) * 4);
  w.wt_off = take(tables ? D * D * esz : 0);
  w.doutt_off = take(tables ? D * Tp * esz : 0);
  w.gt_off = take(tables ? D * Tp * esz : 0);
  w.dg_off = take(tables ? T * D * 4 : 0);
  w.part_off = take(tables ? size_t(backward_splits(L, rows)) * D * D * 4 : 0);
  w.keys0_off = take(nsort * 8);
  w.keys1_off = take(nsort * 8);
  w.vals0_off = take(nsort * 4);
  w.vals1_off = take(nsort * 4);
  // radix histograms [256 * nblocks] and the scan's tile totals after them
  const size_t m = 256 * (nblocks > 0 ? nblocks : 1);
  w.hist_off = take((m + (m + 1023) / 1024) * 4);
  w.head_off = take(seg * 4);
  w.tail_off = take(seg * 4);
  const size_t nchunks = (nsort + kChunk - 1) / kChunk;
  w.owners_off = take((1 + nchunks) * 4);
  w.total = o;
  *out = w;
  return true;
}

int stats_layout(int64_t V0, int32_t n, int64_t ntok, const int64_t* vocab, int32_t nvocab,
                 StatsLayout* out) {
  if (V0 < 1 || V0 >= (int64_t(1) << 31) || n < 1 || n > NGRAM_MAX_ORDER || ntok < 0 ||
      nvocab < 0 || (nvocab > 0 && vocab == nullptr) || out == nullptr)
    return NGRAM_EINVAL;
  // one group of table sizes at a time: the largest group's bitmaps
  size_t words = 0;
  for (int32_t g = 0; g < nvocab; g += kStatsGroup) {
    size_t w = 0;
    for (int32_t v = g; v < nvocab && v < g + kStatsGroup; ++v) {
      if (vocab[v] < 1 || vocab[v] >= (int64_t(1) << 31)) return NGRAM_EINVAL;
      w += size_t((vocab[v] + 31) / 32);
    }
    if (w > words) words = w;
  }
  // exact values: the largest is V0^n - 1, so V0^n <= 2^63 keeps them in 63 bits
  StatsLayout L{};
  uint64_t p = 1;
  L.exact = true;
  for (int j = 0; j < n && L.exact; ++j) {
    if (p > (uint64_t(1) << 63) / uint64_t(V0)) L.exact = false;
    else p *= uint64_t(V0);
  }
  L.key_bits = 0;
  if (L.exact)
    while (L.key_bits < 64 && (uint64_t(1) << L.key_bits) < p) ++L.key_bits;
  const size_t T = L.exact ? size_t(ntok) : 0;
  size_t o = 256;                                    // error flags
  auto take = [&](size_t bytes) { const size_t at = o; o += align256(bytes); return at; };
  L.bits_off = take(words * 4);
  L.keys0_off = take(T * 8);
  L.keys1_off = take(T * 8);
  L.vals0_off = take(T * 4);
  L.vals1_off = take(T * 4);
  const size_t m = 256 * ((T + kSortTile - 1) / kSortTile > 0 ? (T + kSortTile - 1) / kSortTile : 1);
  L.hist_off = take(L.exact ? (m + (m + 1023) / 1024) * 4 : 0);
  L.total = o;
  *out = L;
  return NGRAM_OK;
}

}  // namespace ngram
