// C-ABI entry points: host validation, then stream-ordered kernel launches.
// Declarations and the contract of every function: include/ngram_embed.h.
#include <algorithm>
#include <atomic>

#include "kernels.h"

using ngram::LayerDesc;

namespace {

int hip_status(hipError_t e) { return e == hipSuccess ? NGRAM_OK : NGRAM_EHIP; }

// Tables: E0 and W always; the S sub-table pointers when S > 0. All 16-byte aligned.
int check_tables(const LayerDesc& L, const ngram_embed_tables* T, bool need_e0_w) {
  if (T == nullptr) return NGRAM_EALIGN;
  // the basic form has no projection: W is not read
  if (need_e0_w && (!ngram::aligned(T->E0, 16) ||
                    (L.form == NGRAM_FORM_FINAL && !ngram::aligned(T->W, 16))))
    return NGRAM_EALIGN;
  if (L.S > 0) {
    if (T->E == nullptr) return NGRAM_EALIGN;
    for (int s = 0; s < L.S; ++s)
      if (!ngram::aligned(T->E[s], 16)) return NGRAM_EALIGN;
  }
  // optional layer-normalisation parameters: null, or 16-byte aligned
  if (L.amp == NGRAM_AMP_LAYERNORM &&
      ((T->ln_weight != nullptr && !ngram::aligned(T->ln_weight, 16)) ||
       (T->ln_bias != nullptr && !ngram::aligned(T->ln_bias, 16))))
    return NGRAM_EALIGN;
  return NGRAM_OK;
}

// Projection of `rows` rows into `out`, then the amplification: the scale is part of the
// projection's epilogue; the layer normalisation reads the unrounded rows from the
// workspace.
// `map` places the compact rows in `out` (decode windows); the unrounded rows of the layer
// normalisation stay compact in the workspace.
int project_amplified(const LayerDesc& L, const ngram_embed_tables* T, const int32_t* idx,
                      const int32_t* tok, int64_t rows, void* out, void* ws,
                      const ngram::WsLayout& lay, const ngram::RowMap& map, hipStream_t st) {
  if (L.amp != NGRAM_AMP_LAYERNORM)
    return hip_status(ngram::launch_project(L, T->E0, T->E, T->W, idx, tok, rows, out, false,
                                            map, st));
  float* pre = reinterpret_cast<float*>(static_cast<char*>(ws) + lay.pre_off);
  int rc = hip_status(ngram::launch_project(L, T->E0, T->E, T->W, idx, tok, rows, pre, true,
                                            ngram::RowMap{}, st));
  if (rc != NGRAM_OK) return rc;
  return hip_status(ngram::launch_layernorm(L, pre, tok, T->ln_weight, T->ln_bias, rows, out,
                                            map, st));
}

// The same for nlayers layers with tables T[l] and outputs outs[l] (per-layer embeddings):
// the projections of several layers share one launch; with the layer normalisation the
// layers go one after another through the workspace's unrounded rows.
int project_layers(const LayerDesc& L, const ngram_embed_tables* T, int32_t nlayers,
                   const int32_t* idx, const int32_t* tok, int64_t rows, void* const* outs,
                   void* ws, const ngram::WsLayout& lay, const ngram::RowMap& map,
                   hipStream_t st) {
  if (L.amp == NGRAM_AMP_LAYERNORM || nlayers == 1) {
    for (int32_t l = 0; l < nlayers; ++l) {
      const int rc = project_amplified(L, &T[l], idx, tok, rows, outs[l], ws, lay, map, st);
      if (rc != NGRAM_OK) return rc;
    }
    return NGRAM_OK;
  }
  ngram::LayerParams p[ngram::kMaxLaunchLayers];
  for (int32_t l0 = 0; l0 < nlayers; l0 += ngram::kMaxLaunchLayers) {
    const int32_t n = std::min<int32_t>(ngram::kMaxLaunchLayers, nlayers - l0);
    for (int32_t l = 0; l < n; ++l) p[l] = {T[l0 + l].E0, T[l0 + l].E, T[l0 + l].W, outs[l0 + l]};
    const int rc = hip_status(ngram::launch_project_layers(L, p, n, idx, tok, rows, false, map,
                                                           st));
    if (rc != NGRAM_OK) return rc;
  }
  return NGRAM_OK;
}

// Tables and outputs of nlayers layers: present and aligned.
int check_layers(const LayerDesc& L, const ngram_embed_tables* T, int32_t nlayers,
                 void* const* outs) {
  if (T == nullptr || outs == nullptr) return NGRAM_EALIGN;
  for (int32_t l = 0; l < nlayers; ++l) {
    const int rc = check_tables(L, &T[l], true);
    if (rc != NGRAM_OK) return rc;
    if (!ngram::aligned(outs[l], 16)) return NGRAM_EALIGN;
  }
  return NGRAM_OK;
}

int prefill_impl(const ngram_embed_config* cfg, const ngram_embed_tables* tables,
                 int32_t nlayers, const int32_t* tokens, const int32_t* cu_seqlens,
                 int32_t nseq, int64_t ntok, void* const* outs, ngram_cache* cache, void* ws,
                 size_t ws_bytes, void* stream);
int decode_impl(const ngram_embed_config* cfg, const ngram_embed_tables* tables,
                int32_t nlayers, ngram_cache* cache, const int32_t* new_tokens,
                const int32_t* n_new, int32_t tmax, const int32_t* n_commit,
                void* const* outs, void* ws, size_t ws_bytes, void* stream);

int check_ws(const LayerDesc& L, const void* ws, size_t ws_bytes, int64_t rows,
             ngram::WsLayout* lay) {
  if (!ngram::ws_layout(L, rows, lay)) return NGRAM_EINVAL;
  if (!ngram::aligned(ws, 256) || ws_bytes < lay->total) return NGRAM_EWORKSPACE;
  return NGRAM_OK;
}

int32_t* ws_flags(void* ws) { return static_cast<int32_t*>(ws); }

int prefill_impl(const ngram_embed_config* cfg, const ngram_embed_tables* tables,
                 int32_t nlayers, const int32_t* tokens, const int32_t* cu_seqlens,
                 int32_t nseq, int64_t ntok, void* const* outs, ngram_cache* cache, void* ws,
                 size_t ws_bytes, void* stream) {
  LayerDesc L;
  int rc = ngram::describe(cfg, &L);
  if (rc != NGRAM_OK) return rc;
  if (ntok < 0 || nseq < 0 || (ntok > 0 && nseq < 1)) return NGRAM_EINVAL;
  if (cache != nullptr && cache->nseq != nseq) return NGRAM_EINVAL;
  ngram::WsLayout lay;
  if ((rc = check_ws(L, ws, ws_bytes, ntok, &lay)) != NGRAM_OK) return rc;
  if (cache != nullptr && nseq > 0) {
    if (!ngram::aligned(cache->len, 8) || !ngram::aligned(cu_seqlens, 4)) return NGRAM_EALIGN;
    if (L.N > 1 && !ngram::aligned(cache->ring, 4)) return NGRAM_EALIGN;
  }
  if (ntok > 0) {
    if ((rc = check_layers(L, tables, nlayers, outs)) != NGRAM_OK) return rc;
    if (!ngram::aligned(tokens, 4) || !ngram::aligned(cu_seqlens, 4)) return NGRAM_EALIGN;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the cache of the prompts (section 4.2): their lengths and last N-1 ids, as
  // ngram_cache_init fills it (empty sequences included, so also when ntok = 0)
  if (cache != nullptr && nseq > 0) {
    rc = hip_status(ngram::launch_cache_init(L, cache->ring, cache->len, nullptr, cache->nseq,
                                             tokens, cu_seqlens, nseq, ntok, ws_flags(ws), st));
    if (rc != NGRAM_OK) return rc;
  }
  if (ntok == 0) return NGRAM_OK;
  int32_t* idx = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + lay.idx_off);
  if (L.S > 0) {
    rc = hip_status(ngram::launch_hash_prefill(L, tokens, cu_seqlens, nseq, ntok, idx,
                                               ws_flags(ws), st));
    if (rc != NGRAM_OK) return rc;
  }
  return project_layers(L, tables, nlayers, idx, tokens, ntok, outs, ws, lay, ngram::RowMap{},
                        st);
}

// Host checks of a decode step's pointers (the config, counts and scratch are checked by the
// caller).
int check_decode(const LayerDesc& L, const ngram_embed_tables* tables, int32_t nlayers,
                 const ngram_cache* cache, const int32_t* new_tokens, const int32_t* n_new,
                 const int32_t* n_commit, void* const* outs) {
  const int rc = check_layers(L, tables, nlayers, outs);
  if (rc != NGRAM_OK) return rc;
  if (!ngram::aligned(cache->len, 8) || !ngram::aligned(new_tokens, 4) ||
      !ngram::aligned(n_new, 4))
    return NGRAM_EALIGN;
  if (L.N > 1 && !ngram::aligned(cache->ring, 4)) return NGRAM_EALIGN;
  if (n_commit != nullptr && !ngram::aligned(n_commit, 4)) return NGRAM_EALIGN;
  return NGRAM_OK;
}

// The launches of a decode step, with the step's scratch (tokens, indices, unrounded rows)
// laid out by `lay` from `base` and the flags OR-ed into `flags` (may be null).
int decode_launch(const LayerDesc& L, const ngram_embed_tables* tables, int32_t nlayers,
                  ngram_cache* cache, const int32_t* new_tokens, const int32_t* n_new,
                  int32_t tmax, const int32_t* n_commit, void* const* outs, char* base,
                  const ngram::WsLayout& lay, int32_t* flags, hipStream_t st) {
  const int64_t rows = int64_t(cache->nseq) * tmax;
  int32_t* tok = reinterpret_cast<int32_t*>(base + lay.tok_off);
  int32_t* idx = reinterpret_cast<int32_t*>(base + lay.idx_off);
  // hash (and commit, when asked) in one kernel; the projection reads only tok/idx, so the
  // cache may advance before it runs
  ngram::DecodeArgs d{cache->ring, cache->len, nullptr, cache->nseq, new_tokens, n_new,
                      n_commit, cache->nseq, tmax, 0, tmax, -1, tok, idx, flags};
  const int rc = hip_status(ngram::launch_hash_decode(L, d, st));
  if (rc != NGRAM_OK) return rc;
  return project_layers(L, tables, nlayers, idx, tok, rows, outs, base, lay, ngram::RowMap{},
                        st);
}

int decode_impl(const ngram_embed_config* cfg, const ngram_embed_tables* tables,
                int32_t nlayers, ngram_cache* cache, const int32_t* new_tokens,
                const int32_t* n_new, int32_t tmax, const int32_t* n_commit,
                void* const* outs, void* ws, size_t ws_bytes, void* stream) {
  LayerDesc L;
  int rc = ngram::describe(cfg, &L);
  if (rc != NGRAM_OK) return rc;
  if (cache == nullptr || cache->nseq < 0) return NGRAM_EINVAL;
  if (tmax < 1 || tmax > NGRAM_MAX_DECODE_TOKENS) return NGRAM_EINVAL;
  const int64_t rows = int64_t(cache->nseq) * tmax;
  ngram::WsLayout lay;
  if ((rc = check_ws(L, ws, ws_bytes, rows, &lay)) != NGRAM_OK) return rc;
  if (rows == 0) return NGRAM_OK;
  rc = check_decode(L, tables, nlayers, cache, new_tokens, n_new, n_commit, outs);
  if (rc != NGRAM_OK) return rc;
  return decode_launch(L, tables, nlayers, cache, new_tokens, n_new, tmax, n_commit, outs,
                       static_cast<char*>(ws), lay, ws_flags(ws),
                       static_cast<hipStream_t>(stream));
}

// ------------------------------------------------------------------ fixed scratch
// The scratch of ngram_embed_decode_noalloc: one array per GPU, declared in device memory
// (the code object's loader places it when the library is loaded on a device; it lives until
// the process ends). In host code `scratch` names a host-side stand-in, not the device
// array: only the address hipGetSymbolAddress returns for the current device is ever passed
// to a kernel.
static __device__ __align__(256) char scratch[NGRAM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 256;
std::atomic<char*> g_scratch[kMaxScratchDevices];   // device address of `scratch`, per GPU

// The current device's scratch (looked up once per device; the stream must be on it).
int device_scratch(hipStream_t st, char** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return NGRAM_EHIP;
  if (st != nullptr) {
    hipDevice_t sdev = 0;
    if (hipStreamGetDevice(st, &sdev) != hipSuccess) return NGRAM_EHIP;
    if (int(sdev) != dev) return NGRAM_EINVAL;
  }
  if (dev < 0 || dev >= kMaxScratchDevices) return NGRAM_EINVAL;
  char* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr)
      return NGRAM_EHIP;
    p = static_cast<char*>(q);
    g_scratch[dev].store(p, std::memory_order_release);   // the same address if two race
  }
  *out = p;
  return NGRAM_OK;
}

}  // namespace

extern "C" {

size_t ngram_embed_workspace_size(const ngram_embed_config* cfg, int64_t max_rows) {
  LayerDesc L;
  ngram::WsLayout lay;
  if (ngram::describe(cfg, &L) != NGRAM_OK || !ngram::ws_layout(L, max_rows, &lay)) return 0;
  return lay.total;
}

int ngram_embed_workspace_layout(const ngram_embed_config* cfg, int64_t max_rows,
                                 size_t* tok_off, size_t* idx_off) {
  LayerDesc L;
  const int rc = ngram::describe(cfg, &L);
  if (rc != NGRAM_OK) return rc;
  ngram::WsLayout lay;
  if (!ngram::ws_layout(L, max_rows, &lay)) return NGRAM_EINVAL;
  if (tok_off) *tok_off = lay.tok_off;
  if (idx_off) *idx_off = lay.idx_off;
  return NGRAM_OK;
}

int ngram_embed_hash(const ngram_embed_config* cfg, const int32_t* tokens,
                     const int32_t* cu_seqlens, int32_t nseq, int64_t ntok, int32_t* idx,
                     int32_t* err_flags, void* stream) {
  LayerDesc L;
  int rc = ngram::describe(cfg, &L);
  if (rc != NGRAM_OK) return rc;
  if (ntok < 0 || nseq < 0 || (ntok > 0 && nseq < 1)) return NGRAM_EINVAL;
  if (ntok == 0) return NGRAM_OK;
  if (!ngram::aligned(tokens, 4) || !ngram::aligned(cu_seqlens, 4)) return NGRAM_EALIGN;
  if (L.S > 0 && !ngram::aligned(idx, 4)) return NGRAM_EALIGN;
  if (err_flags != nullptr && !ngram::aligned(err_flags, 4)) return NGRAM_EALIGN;
  if (L.S == 0) return NGRAM_OK;  // N = 1: nothing to hash
  return hip_status(ngram::launch_hash_prefill(L, tokens, cu_seqlens, nseq, ntok, idx,
                                               err_flags, static_cast<hipStream_t>(stream)));
}

int ngram_embed_gather(const ngram_embed_config* cfg, const ngram_embed_tables* tables,
                       const int32_t* idx, int64_t nrows, void* G, void* stream) {
  LayerDesc L;
  int rc = ngram::describe(cfg, &L);
  if (rc != NGRAM_OK) return rc;
  if (nrows < 0) return NGRAM_EINVAL;
  if (nrows == 0 || L.S == 0) return NGRAM_OK;
  if ((rc = check_tables(L, tables, false)) != NGRAM_OK) return rc;
  if (!ngram::aligned(idx, 4) || !ngram::aligned(G, 16)) return NGRAM_EALIGN;
  return hip_status(ngram::launch_gather(L, tables->E, idx, nrows, G,
                                         static_cast<hipStream_t>(stream)));
}

int ngram_embed_gather_checksum(const ngram_embed_config* cfg, const ngram_embed_tables* tables,
                                const int32_t* idx, int64_t nrows, uint32_t* sums,
                                void* stream) {
  LayerDesc L;
  int rc = ngram::describe(cfg, &L);
  if (rc != NGRAM_OK) return rc;
  if (nrows < 0) return NGRAM_EINVAL;
  if (nrows == 0 || L.S == 0) return NGRAM_OK;
  if ((rc = check_tables(L, tables, false)) != NGRAM_OK) return rc;
  if (!ngram::aligned(idx, 4) || !ngram::aligned(sums, 4)) return NGRAM_EALIGN;
  return hip_status(ngram::launch_gather_lds(L, tables->E, idx, nrows, sums,
                                             static_cast<hipStream_t>(stream)));
}

int ngram_embed_project(const ngram_embed_config* cfg, const ngram_embed_tables* tables,
                        const int32_t* idx, const int32_t* tok, int64_t nrows, void* out,
                        void* stream) {
  LayerDesc L;
  int rc = ngram::describe(cfg, &L);
  if (rc != NGRAM_OK) return rc;
  if (nrows < 0) return NGRAM_EINVAL;
  if (L.amp == NGRAM_AMP_LAYERNORM) return NGRAM_EINVAL;   // needs a workspace
  if (nrows == 0) return NGRAM_OK;
  if ((rc = check_tables(L, tables, true)) != NGRAM_OK) return rc;
  if ((L.S > 0 && !ngram::aligned(idx, 4)) || !ngram::aligned(tok, 4) ||
      !ngram::aligned(out, 16))
    return NGRAM_EALIGN;
  return hip_status(ngram::launch_project(L, tables->E0, tables->E, tables->W, idx, tok, nrows,
                                          out, false, ngram::RowMap{},
                                          static_cast<hipStream_t>(stream)));
}

int ngram_embed_prefill(const ngram_embed_config* cfg, const ngram_embed_tables* tables,
                        const int32_t* tokens, const int32_t* cu_seqlens, int32_t nseq,
                        int64_t ntok, void* out, ngram_cache* cache_or_null, void* ws,
                        size_t ws_bytes, void* stream) {
  void* outs[1] = {out};
  return prefill_impl(cfg, tables, 1, tokens, cu_seqlens, nseq, ntok, outs, cache_or_null, ws,
                      ws_bytes, stream);
}

int ngram_embed_prefill_layers(const ngram_embed_config* cfg, const ngram_embed_tables* tables,
                               int32_t nlayers, const int32_t* tokens,
                               const int32_t* cu_seqlens, int32_t nseq, int64_t ntok,
                               void* const* out, void* ws, size_t ws_bytes, void* stream) {
  if (nlayers < 1) return NGRAM_EINVAL;
  return prefill_impl(cfg, tables, nlayers, tokens, cu_seqlens, nseq, ntok, out, nullptr, ws,
                      ws_bytes, stream);
}

int ngram_cache_init(const ngram_embed_config* cfg, ngram_cache* cache, const int32_t* tokens,
                     const int32_t* cu_seqlens, int64_t ntok, void* stream) {
  LayerDesc L;
  int rc = ngram::describe(cfg, &L);
  if (rc != NGRAM_OK) return rc;
  if (cache == nullptr || cache->nseq < 0 || ntok < 0) return NGRAM_EINVAL;
  if (cache->nseq == 0) return NGRAM_OK;
  if (!ngram::aligned(cache->len, 8) || !ngram::aligned(cu_seqlens, 4)) return NGRAM_EALIGN;
  if (L.N > 1 && !ngram::aligned(cache->ring, 4)) return NGRAM_EALIGN;
  if (ntok > 0 && !ngram::aligned(tokens, 4)) return NGRAM_EALIGN;
  return hip_status(ngram::launch_cache_init(L, cache->ring, cache->len, nullptr, cache->nseq,
                                             tokens, cu_seqlens, cache->nseq, ntok, nullptr,
                                             static_cast<hipStream_t>(stream)));
}

int ngram_embed_decode(const ngram_embed_config* cfg, const ngram_embed_tables* tables,
                       ngram_cache* cache, const int32_t* new_tokens, const int32_t* n_new,
                       int32_t tmax, const int32_t* n_commit, void* out, void* ws,
                       size_t ws_bytes, void* stream) {
  void* outs[1] = {out};
  return decode_impl(cfg, tables, 1, cache, new_tokens, n_new, tmax, n_commit, outs, ws,
                     ws_bytes, stream);
}

int ngram_embed_decode_layers(const ngram_embed_config* cfg, const ngram_embed_tables* tables,
                              int32_t nlayers, ngram_cache* cache, const int32_t* new_tokens,
                              const int32_t* n_new, int32_t tmax, const int32_t* n_commit,
                              void* const* out, void* ws, size_t ws_bytes, void* stream) {
  if (nlayers < 1) return NGRAM_EINVAL;
  return decode_impl(cfg, tables, nlayers, cache, new_tokens, n_new, tmax, n_commit, out, ws,
                     ws_bytes, stream);
}

int ngram_cache_commit(const ngram_embed_config* cfg, ngram_cache* cache,
                       const int32_t* new_tokens, const int32_t* n_accept, int32_t tmax,
                       int32_t* err_flags, void* stream) {
  LayerDesc L;
  int rc = ngram::describe(cfg, &L);
  if (rc != NGRAM_OK) return rc;
  if (cache == nullptr || cache->nseq < 0) return NGRAM_EINVAL;
  if (tmax < 1 || tmax > NGRAM_MAX_DECODE_TOKENS) return NGRAM_EINVAL;
  if (cache->nseq == 0) return NGRAM_OK;
  if (!ngram::aligned(cache->len, 8) || !ngram::aligned(new_tokens, 4) ||
      !ngram::aligned(n_accept, 4))
    return NGRAM_EALIGN;
  if (L.N > 1 && !ngram::aligned(cache->ring, 4)) return NGRAM_EALIGN;
  if (err_flags != nullptr && !ngram::aligned(err_flags, 4)) return NGRAM_EALIGN;
  return hip_status(ngram::launch_cache_commit(L, cache->ring, cache->len, nullptr, cache->nseq,
                                               new_tokens, n_accept, cache->nseq, tmax,
                                               err_flags, static_cast<hipStream_t>(stream)));
}

int ngram_embed_decode_rows(const ngram_embed_config* cfg, const ngram_embed_tables* tables,
                            ngram_cache* cache, const int32_t* slots, int32_t nbatch,
                            const int32_t* new_tokens, const int32_t* n_new, int32_t tmax,
                            int32_t row_begin, int32_t row_end, const int32_t* n_commit,
                            void* out, void* ws, size_t ws_bytes, void* stream) {
  LayerDesc L;
  int rc = ngram::describe(cfg, &L);
  if (rc != NGRAM_OK) return rc;
  if (cache == nullptr || cache->nseq < 0 || nbatch < 0) return NGRAM_EINVAL;
  if (slots == nullptr && nbatch > cache->nseq) return NGRAM_EINVAL;
  if (tmax < 1 || tmax > NGRAM_MAX_DECODE_TOKENS) return NGRAM_EINVAL;
  if (row_begin < 0 || row_end <= row_begin || row_end > tmax) return NGRAM_EINVAL;
  const int32_t width = row_end - row_begin;
  const int64_t rows = int64_t(nbatch) * width;
  ngram::WsLayout lay;
  if ((rc = check_ws(L, ws, ws_bytes, rows, &lay)) != NGRAM_OK) return rc;
  if (rows == 0) return NGRAM_OK;
  if ((rc = check_tables(L, tables, true)) != NGRAM_OK) return rc;
  if (!ngram::aligned(cache->len, 8) || !ngram::aligned(new_tokens, 4) ||
      !ngram::aligned(n_new, 4) || !ngram::aligned(out, 16))
    return NGRAM_EALIGN;
  if (L.N > 1 && !ngram::aligned(cache->ring, 4)) return NGRAM_EALIGN;
  if ((n_commit != nullptr && !ngram::aligned(n_commit, 4)) ||
      (slots != nullptr && !ngram::aligned(slots, 4)))
    return NGRAM_EALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  int32_t* tok = reinterpret_cast<int32_t*>(w + lay.tok_off);
  int32_t* idx = reinterpret_cast<int32_t*>(w + lay.idx_off);
  ngram::DecodeArgs d{cache->ring, cache->len, slots, cache->nseq, new_tokens, n_new, n_commit,
                      nbatch, tmax, row_begin, width, ngram::kSkipRow, tok, idx, ws_flags(ws)};
  rc = hip_status(ngram::launch_hash_decode(L, d, st));
  if (rc != NGRAM_OK) return rc;
  // compact row b * width + (j - row_begin) is row b * tmax + j of out
  ngram::RowMap map;
  map.group = width;
  map.stride = tmax;
  map.off = row_begin;
  return project_amplified(L, tables, idx, tok, rows, out, ws, lay, map, st);
}

int ngram_cache_init_slots(const ngram_embed_config* cfg, ngram_cache* cache,
                           const int32_t* slots, int32_t nbatch, const int32_t* tokens,
                           const int32_t* cu_seqlens, int64_t ntok, int32_t* err_flags,
                           void* stream) {
  LayerDesc L;
  int rc = ngram::describe(cfg, &L);
  if (rc != NGRAM_OK) return rc;
  if (cache == nullptr || cache->nseq < 0 || nbatch < 0 || ntok < 0) return NGRAM_EINVAL;
  if (slots == nullptr && nbatch > cache->nseq) return NGRAM_EINVAL;
  if (nbatch == 0) return NGRAM_OK;
  if (!ngram::aligned(cache->len, 8) || !ngram::aligned(cu_seqlens, 4)) return NGRAM_EALIGN;
  if (L.N > 1 && !ngram::aligned(cache->ring, 4)) return NGRAM_EALIGN;
  if (ntok > 0 && !ngram::aligned(tokens, 4)) return NGRAM_EALIGN;
  if ((slots != nullptr && !ngram::aligned(slots, 4)) ||
      (err_flags != nullptr && !ngram::aligned(err_flags, 4)))
    return NGRAM_EALIGN;
  return hip_status(ngram::launch_cache_init(L, cache->ring, cache->len, slots, cache->nseq,
                                             tokens, cu_seqlens, nbatch, ntok, err_flags,
                                             static_cast<hipStream_t>(stream)));
}

int ngram_cache_commit_slots(const ngram_embed_config* cfg, ngram_cache* cache,
                             const int32_t* slots, int32_t nbatch, const int32_t* new_tokens,
                             const int32_t* n_accept, int32_t tmax, int32_t* err_flags,
                             void* stream) {
  LayerDesc L;
  int rc = ngram::describe(cfg, &L);
  if (rc != NGRAM_OK) return rc;
  if (cache == nullptr || cache->nseq < 0 || nbatch < 0) return NGRAM_EINVAL;
  if (slots == nullptr && nbatch > cache->nseq) return NGRAM_EINVAL;
  if (tmax < 1 || tmax > NGRAM_MAX_DECODE_TOKENS) return NGRAM_EINVAL;
  if (nbatch == 0) return NGRAM_OK;
  if (!ngram::aligned(cache->len, 8) || !ngram::aligned(new_tokens, 4) ||
      !ngram::aligned(n_accept, 4))
    return NGRAM_EALIGN;
  if (L.N > 1 && !ngram::aligned(cache->ring, 4)) return NGRAM_EALIGN;
  if ((slots != nullptr && !ngram::aligned(slots, 4)) ||
      (err_flags != nullptr && !ngram::aligned(err_flags, 4)))
    return NGRAM_EALIGN;
  return hip_status(ngram::launch_cache_commit(L, cache->ring, cache->len, slots, cache->nseq,
                                               new_tokens, n_accept, nbatch, tmax, err_flags,
                                               static_cast<hipStream_t>(stream)));
}

size_t ngram_embed_backward_workspace_size(const ngram_embed_config* cfg, int64_t ntok) {
  LayerDesc L;
  ngram::BwLayout lay;
  if (ngram::describe(cfg, &L) != NGRAM_OK || L.amp == NGRAM_AMP_LAYERNORM ||
      !ngram::bw_layout(L, ntok, &lay))
    return 0;
  return lay.total;
}

int ngram_embed_backward(const ngram_embed_config* cfg, const ngram_embed_tables* tables,
                         const int32_t* tokens, const int32_t* cu_seqlens, int32_t nseq,
                         int64_t ntok, const void* dout, float* dE0, float* const* dE,
                         float* dW, void* ws, size_t ws_bytes, void* stream) {
  LayerDesc L;
  int rc = ngram::describe(cfg, &L);
  if (rc != NGRAM_OK) return rc;
  if (L.amp == NGRAM_AMP_LAYERNORM) return NGRAM_EINVAL;   // not differentiated here
  if (L.form == NGRAM_FORM_BASIC && dW != nullptr) return NGRAM_EINVAL;   // no projection
  if (ntok < 0 || nseq < 0 || (ntok > 0 && nseq < 1)) return NGRAM_EINVAL;
  // positions are sort values (uint32) and the tile numbering stays in range
  if (ntok > (int64_t(1) << 31) / (L.S > 0 ? L.S : 1)) return NGRAM_EINVAL;
  ngram::BwLayout lay;
  if (!ngram::bw_layout(L, ntok, &lay)) return NGRAM_EINVAL;
  if (!ngram::aligned(ws, 256) || ws_bytes < lay.total) return NGRAM_EWORKSPACE;
  if (ntok == 0) return NGRAM_OK;
  if ((rc = check_tables(L, tables, true)) != NGRAM_OK) return rc;
  if (!ngram::aligned(tokens, 4) || !ngram::aligned(cu_seqlens, 4) || !ngram::aligned(dout, 16))
    return NGRAM_EALIGN;
  if ((dE0 != nullptr && !ngram::aligned(dE0, 16)) || (dW != nullptr && !ngram::aligned(dW, 16)))
    return NGRAM_EALIGN;
  if (dE != nullptr)
    for (int s = 0; s < L.S; ++s)
      if (!ngram::aligned(dE[s], 16)) return NGRAM_EALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  int32_t* idx = reinterpret_cast<int32_t*>(w + lay.idx_off);
  if (L.S > 0) {
    rc = hip_status(ngram::launch_hash_prefill(L, tokens, cu_seqlens, nseq, ntok, idx,
                                               ws_flags(ws), st));
    if (rc != NGRAM_OK) return rc;
  }
  ngram::BackwardArgs b{};
  b.E = tables->E;
  b.W = tables->W;
  b.tokens = tokens;
  b.idx = idx;
  b.dout = dout;
  b.dE0 = dE0;
  b.dE = dE;
  b.dW = dW;
  b.rows = ntok;
  b.ident = reinterpret_cast<int32_t*>(w + lay.ident_off);
  b.WT = w + lay.wt_off;
  b.doutT = w + lay.doutt_off;
  b.GT = w + lay.gt_off;
  b.dG = reinterpret_cast<float*>(w + lay.dg_off);
  b.part = reinterpret_cast<float*>(w + lay.part_off);
  b.keys0 = reinterpret_cast<uint64_t*>(w + lay.keys0_off);
  b.keys1 = reinterpret_cast<uint64_t*>(w + lay.keys1_off);
  b.vals0 = reinterpret_cast<uint32_t*>(w + lay.vals0_off);
  b.vals1 = reinterpret_cast<uint32_t*>(w + lay.vals1_off);
  b.hist = reinterpret_cast<uint32_t*>(w + lay.hist_off);
  b.head = reinterpret_cast<float*>(w + lay.head_off);
  b.tail = reinterpret_cast<float*>(w + lay.tail_off);
  b.owners = reinterpret_cast<uint32_t*>(w + lay.owners_off);
  return hip_status(ngram::launch_backward(L, b, st));
}

size_t ngram_hash_stats_workspace_size(int64_t V0, int32_t n, int64_t ntok,
                                       const int64_t* vocab, int32_t nvocab) {
  ngram::StatsLayout lay;
  if (ngram::stats_layout(V0, n, ntok, vocab, nvocab, &lay) != NGRAM_OK) return 0;
  return lay.total;
}

int ngram_hash_stats(int64_t V0, int32_t n, const int32_t* tokens, const int32_t* cu_seqlens,
                     int32_t nseq, int64_t ntok, const int64_t* vocab, int32_t nvocab,
                     int64_t* rows, int64_t* distinct, void* ws, size_t ws_bytes,
                     void* stream) {
  ngram::StatsLayout lay;
  int rc = ngram::stats_layout(V0, n, ntok, vocab, nvocab, &lay);
  if (rc != NGRAM_OK) return rc;
  if (nseq < 0 || (ntok > 0 && nseq < 1)) return NGRAM_EINVAL;
  if (distinct != nullptr && !lay.exact) return NGRAM_EOVERFLOW;
  if (!ngram::aligned(ws, 256) || ws_bytes < lay.total) return NGRAM_EWORKSPACE;
  if (nvocab == 0 && distinct == nullptr) return NGRAM_OK;
  if ((nvocab > 0 && !ngram::aligned(rows, 8)) ||
      (distinct != nullptr && !ngram::aligned(distinct, 8)))
    return NGRAM_EALIGN;
  if (ntok > 0 && (!ngram::aligned(tokens, 4) || !ngram::aligned(cu_seqlens, 4)))
    return NGRAM_EALIGN;
  char* w = static_cast<char*>(ws);
  ngram::StatsArgs a{};
  a.tokens = tokens;
  a.cu = cu_seqlens;
  a.nseq = nseq;
  a.ntok = ntok;
  a.V0 = V0;
  a.n = n;
  a.vocab = vocab;
  a.nvocab = nvocab;
  a.rows = rows;
  a.distinct = distinct;
  a.bits = reinterpret_cast<uint32_t*>(w + lay.bits_off);
  a.keys0 = reinterpret_cast<uint64_t*>(w + lay.keys0_off);
  a.keys1 = reinterpret_cast<uint64_t*>(w + lay.keys1_off);
  a.vals0 = reinterpret_cast<uint32_t*>(w + lay.vals0_off);
  a.vals1 = reinterpret_cast<uint32_t*>(w + lay.vals1_off);
  a.hist = reinterpret_cast<uint32_t*>(w + lay.hist_off);
  a.key_bits = lay.key_bits;
  a.flags = ws_flags(ws);
  return hip_status(ngram::launch_hash_stats(a, static_cast<hipStream_t>(stream)));
}

int ngram_embed_read_error_flag(const void* ws, int32_t* flags, void* stream) {
  if (!ngram::aligned(ws, 256) || flags == nullptr) return NGRAM_EALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(flags, ws, sizeof(int32_t), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  return hip_status(e);
}

int ngram_embed_clear_error_flag(void* ws, void* stream) {
  if (!ngram::aligned(ws, 256)) return NGRAM_EALIGN;
  return hip_status(ngram::launch_clear_flags(ws_flags(ws), static_cast<hipStream_t>(stream)));
}

int ngram_embed_decode_noalloc(const ngram_embed_config* cfg, const ngram_embed_tables* tables,
                               ngram_cache* cache, const int32_t* new_tokens,
                               const int32_t* n_new, int32_t tmax, const int32_t* n_commit,
                               void* out, int32_t* err_flags, void* stream) {
  LayerDesc L;
  int rc = ngram::describe(cfg, &L);
  if (rc != NGRAM_OK) return rc;
  if (cache == nullptr || cache->nseq < 0) return NGRAM_EINVAL;
  if (tmax < 1 || tmax > NGRAM_MAX_DECODE_TOKENS) return NGRAM_EINVAL;
  const int64_t rows = int64_t(cache->nseq) * tmax;
  ngram::WsLayout lay;
  if (!ngram::ws_layout(L, rows, &lay)) return NGRAM_EINVAL;
  if (lay.total > NGRAM_NOALLOC_SCRATCH_BYTES) return NGRAM_ESCRATCH;
  if (rows == 0) return NGRAM_OK;
  void* outs[1] = {out};
  rc = check_decode(L, tables, 1, cache, new_tokens, n_new, n_commit, outs);
  if (rc != NGRAM_OK) return rc;
  if (err_flags != nullptr && !ngram::aligned(err_flags, 4)) return NGRAM_EALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* base = nullptr;
  if ((rc = device_scratch(st, &base)) != NGRAM_OK) return rc;
  // nothing in the scratch is read before this step writes it (tokens and indices by the
  // hash kernel, the unrounded rows by the projection), so no clearing is needed
  return decode_launch(L, tables, 1, cache, new_tokens, n_new, tmax, n_commit, outs, base,
                       lay, err_flags, st);
}

const char* ngram_embed_status_string(int status) {
  switch (status) {
    case NGRAM_OK: return "ok";
    case NGRAM_EINVAL: return "invalid size, count or configuration";
    case NGRAM_EDTYPE: return "unknown dtype";
    case NGRAM_EALIGN: return "null or misaligned pointer";
    case NGRAM_EWORKSPACE: return "workspace missing, misaligned or too small";
    case NGRAM_EOVERFLOW: return "V0 * max V_{n,k} exceeds the exact 64-bit hash range";
    case NGRAM_EHIP: return "HIP runtime error at launch";
    case NGRAM_ESCRATCH:
      return "the step needs more than the fixed scratch of the allocation-free entry point";
    default: return "unknown status";
  }
}

}  // extern "C"
