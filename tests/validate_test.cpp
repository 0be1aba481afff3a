// Host unit test of the HIP-free config validation (built with g++ under sanitizers).
#include <cstdio>
#include <cstdlib>

#include "layer_desc.h"

static int failures = 0;
#define EXPECT(cond)                                              \
  do {                                                            \
    if (!(cond)) {                                                \
      std::printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #cond);  \
      ++failures;                                                 \
    }                                                             \
  } while (0)

int main() {
  using ngram::LayerDesc;
  int64_t V[64];
  for (int i = 0; i < 64; ++i) V[i] = 1009 + 2 * i;
  ngram_embed_config c{3, 2, 64, NGRAM_BF16, 1000, V};
  LayerDesc L{};
  EXPECT(ngram::describe(&c, &L) == NGRAM_OK);
  EXPECT(L.S == 4 && L.d == 16 && L.esz == 2 && L.V0 == 1000 && L.V[3] == 1015u);

  // N = 1: no sub-tables, V may be NULL
  ngram_embed_config c1{1, 4, 64, NGRAM_F32, 50, nullptr};
  EXPECT(ngram::describe(&c1, &L) == NGRAM_OK && L.S == 0 && L.d == 0);

  ngram_embed_config bad = c;
  bad.D = 60;                      // 60 % 4 != 0
  EXPECT(ngram::describe(&bad, &L) == NGRAM_EINVAL);
  bad = c;
  bad.D = 4 * 12;                  // d = 12 bf16 = 24 bytes: not whole 16-byte vectors
  EXPECT(ngram::describe(&bad, &L) == NGRAM_EINVAL);
  bad = c;
  bad.dtype = 3;
  EXPECT(ngram::describe(&bad, &L) == NGRAM_EDTYPE);
  bad = c;
  bad.V = nullptr;
  EXPECT(ngram::describe(&bad, &L) == NGRAM_EINVAL);
  bad = c;
  bad.N = 17;
  EXPECT(ngram::describe(&bad, &L) == NGRAM_EINVAL);
  bad = c;
  bad.K = 33;                      // (N-1)K = 66 > 64
  EXPECT(ngram::describe(&bad, &L) == NGRAM_EINVAL);
  EXPECT(ngram::describe(nullptr, &L) == NGRAM_EINVAL);

  // largest accepted sizes: V0 and V just below 2^31 keep V * V0 < 2^62
  int64_t Vbig[4] = {(int64_t(1) << 31) - 1, 3, 5, 7};
  ngram_embed_config big{3, 2, 64, NGRAM_F32, (int64_t(1) << 31) - 1, Vbig};
  EXPECT(ngram::describe(&big, &L) == NGRAM_OK && L.V[0] == 2147483647u);

  ngram::WsLayout w;
  EXPECT(ngram::describe(&c, &L) == NGRAM_OK);
  EXPECT(ngram::ws_layout(L, 1000, &w) && w.tok_off == 256 && w.idx_off == 256 + 4096 &&
         w.total == w.idx_off + 16128);
  EXPECT(!ngram::ws_layout(L, -1, &w));

  // embedding amplification: a zero-filled config is the plain layer (factor 1)
  EXPECT(ngram::describe(&c, &L) == NGRAM_OK && L.amp == NGRAM_AMP_NONE && L.scale == 1.0f);
  ngram_embed_config amp = c;
  amp.amp = NGRAM_AMP_SCALE;
  amp.amp_scale = 8.0f;
  EXPECT(ngram::describe(&amp, &L) == NGRAM_OK && L.scale == 8.0f);
  // the sentinel selects sqrt(D), computed on the library's side (D = 64: exactly 8)
  amp.amp_scale = NGRAM_AMP_SCALE_SQRT_D;
  EXPECT(ngram::describe(&amp, &L) == NGRAM_OK && L.scale == 8.0f);
  amp.D = 3072;
  amp.K = 4;                       // S = 8: d = 384
  EXPECT(ngram::describe(&amp, &L) == NGRAM_OK && L.scale == __builtin_sqrtf(3072.0f) &&
         L.scale > 55.42f && L.scale < 55.43f);
  amp.D = 64;
  amp.K = 2;
  amp.amp_scale = -2.5f;           // any other finite factor is used as given
  EXPECT(ngram::describe(&amp, &L) == NGRAM_OK && L.scale == -2.5f);
  amp.amp_scale = __builtin_nanf("");
  EXPECT(ngram::describe(&amp, &L) == NGRAM_EINVAL);
  amp.amp_scale = __builtin_inff();
  EXPECT(ngram::describe(&amp, &L) == NGRAM_EINVAL);
  amp = c;
  amp.amp = NGRAM_AMP_LAYERNORM;
  amp.amp_scale = 3.0f;            // ignored by the layer normalisation
  amp.ln_eps = 1e-5f;
  EXPECT(ngram::describe(&amp, &L) == NGRAM_OK && L.scale == 1.0f && L.ln_eps == 1e-5f);
  // the layer normalisation keeps the unrounded fp32 rows in the workspace
  EXPECT(ngram::ws_layout(L, 1000, &w) && w.pre_off == w.idx_off + 16128 &&
         w.total == w.pre_off + 1000 * 64 * 4);
  amp.ln_eps = 0.0f;
  EXPECT(ngram::describe(&amp, &L) == NGRAM_EINVAL);
  amp.ln_eps = -1.0f;
  EXPECT(ngram::describe(&amp, &L) == NGRAM_EINVAL);
  amp.ln_eps = __builtin_nanf("");
  EXPECT(ngram::describe(&amp, &L) == NGRAM_EINVAL);
  amp.ln_eps = 1e-5f;
  amp.D = 8192 + 64;               // rows longer than one block normalises
  amp.K = 1;                       // S = 2 divides D; d = 4128 bf16 is whole 16-byte vectors
  EXPECT(ngram::describe(&amp, &L) == NGRAM_EINVAL);
  amp.D = 8192;
  EXPECT(ngram::describe(&amp, &L) == NGRAM_OK);
  amp = c;
  amp.amp = 3;
  EXPECT(ngram::describe(&amp, &L) == NGRAM_EINVAL);
  amp.amp = -1;
  EXPECT(ngram::describe(&amp, &L) == NGRAM_EINVAL);
  // the basic form (Eq. 1): K = 1, full-width tables (d = D, no divisibility by S)
  ngram_embed_config basic{4, 1, 64, NGRAM_BF16, 1000, V};
  EXPECT(ngram::describe(&basic, &L) == NGRAM_EINVAL);      // final form: 64 % 3 != 0
  basic.form = NGRAM_FORM_BASIC;
  EXPECT(ngram::describe(&basic, &L) == NGRAM_OK && L.S == 3 && L.d == 64 &&
         L.form == NGRAM_FORM_BASIC);
  ngram::BwLayout bl;                                        // no product operands
  EXPECT(ngram::bw_layout(L, 100, &bl) && bl.wt_off == bl.ident_off + 512 &&
         bl.dg_off == bl.wt_off && bl.part_off == bl.wt_off);
  LayerDesc Lb{};
  basic.D = 68;                                              // 136 bytes: not 16-byte rows
  EXPECT(ngram::describe(&basic, &Lb) == NGRAM_EINVAL);
  basic.D = 64;
  basic.K = 2;                                               // one table per order
  EXPECT(ngram::describe(&basic, &Lb) == NGRAM_EINVAL);
  basic.K = 1;
  basic.form = 2;
  EXPECT(ngram::describe(&basic, &Lb) == NGRAM_EINVAL);
  // hash statistics: exact n-gram values while V0^n <= 2^63, their width for the sort
  ngram::StatsLayout sl;
  const int64_t sizes[3] = {7, 64, 33};
  EXPECT(ngram::stats_layout(10, 2, 100, sizes, 3, &sl) == NGRAM_OK && sl.exact &&
         sl.key_bits == 7 && sl.bits_off == 256);
  EXPECT(ngram::stats_layout(131072, 3, 100, sizes, 3, &sl) == NGRAM_OK && sl.key_bits == 51);
  EXPECT(ngram::stats_layout(int64_t(1) << 21, 3, 100, sizes, 3, &sl) == NGRAM_OK &&
         sl.exact && sl.key_bits == 63);
  EXPECT(ngram::stats_layout((int64_t(1) << 21) + 1, 3, 100, sizes, 3, &sl) == NGRAM_OK &&
         !sl.exact && sl.keys0_off == sl.keys1_off);
  const int64_t bad_sizes[1] = {0};
  EXPECT(ngram::stats_layout(10, 2, 100, bad_sizes, 1, &sl) == NGRAM_EINVAL);
  EXPECT(ngram::stats_layout(10, 0, 100, sizes, 3, &sl) == NGRAM_EINVAL);
  EXPECT(ngram::stats_layout(10, 2, -1, sizes, 3, &sl) == NGRAM_EINVAL);
  EXPECT(ngram::aligned(reinterpret_cast<void*>(0x1000), 256));
  EXPECT(!ngram::aligned(reinterpret_cast<void*>(0x1004), 16));
  EXPECT(!ngram::aligned(nullptr, 4));

  if (failures == 0) std::printf("all passed\n");
  return failures == 0 ? 0 : 1;
}
