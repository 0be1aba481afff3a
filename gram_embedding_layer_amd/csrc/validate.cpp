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
  if (S > 0) {
    // Sub-table width D/((N-1)K) (section A2); rows must be whole 16-byte vectors.
    if (cfg->D % S != 0) return NGRAM_EINVAL;
    L.d = int32_t(cfg->D / S);
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
    L.scale = cfg->amp_scale;
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

}  // namespace ngram
