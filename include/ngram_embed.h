/*
 * ngram_embed.h - C ABI of the MI355X (gfx950) N-gram embedding forward pass.
 *
 * The layer is the final ("Over-Encoding") form of the N-gram embedding described in
 * section A2 of the deep-notes page on "Scaling Embeddings Outperforms Scaling Experts in
 * Language Models" (Meituan LongCat team):
 *
 *   e_i = ( E_0(t_i) + sum_{n=2}^{N} sum_{k=1}^{K} W_{n,k} E_{n,k}(H_{n,k}(t_{i-n+1..i})) )
 *         / ((N-1)K + 1)
 *
 * with the polynomial rolling hash of the same section
 *
 *   H_{n,k}(t_{i-n+1..i}) = ( sum_{j=0}^{n-1} t_{i-j} * V0^j ) mod V_{n,k},
 *
 * sub-tables E_{n,k} of shape [V_{n,k}, d], d = D/((N-1)K), and projections W_{n,k} of
 * shape [D, d]. Section 4.2 of that page (N-gram cache, KV-cache-like management of n-gram
 * ids on the device) motivates the decode entry points. Section 3.2.4 of the same page
 * (embedding amplification) gives the optional output scale or layer normalisation that
 * the config's `amp` field selects. The config's `form` field selects instead the basic
 * form of the same section (its Eq. 1):
 *
 *   e_i = ( E_0(t_i) + sum_{n=2}^{N} E_n(H_n(t_{i-n+1..i})) ) / N,
 *
 * one table E_n of full width D per order (K = 1), no projection.
 *
 * Conventions used throughout:
 *  - S = (N-1)K sub-tables, ordered s = (n-2)*K + (k-1) (n-major, k-minor).
 *  - Positions before the first token of a sequence hash as the pad id 0. Ids of another
 *    sequence packed in the same batch are never used.
 *  - N = 1 is accepted: there are no sub-tables and e_i = E_0(t_i).
 *  - All matrices are row-major. "device" pointers are HIP device memory, "host" pointers
 *    are ordinary host memory read only during the call. The library allocates no memory
 *    and keeps no state between calls; the caller owns every buffer (the one exception is
 *    the fixed scratch array of ngram_embed_decode_noalloc, declared by the library).
 *  - Every entry point that takes a stream only enqueues work on that stream (a hipStream_t,
 *    or NULL for the null stream) and returns without waiting, except
 *    ngram_embed_read_error_flag, which waits for the stream.
 *  - Arguments are validated on the host before any work is enqueued; a failed check
 *    returns a negative status and enqueues nothing. Entry points never throw.
 *  - Floating-point: bf16 paths read bf16 tables, multiply on the matrix cores with fp32
 *    accumulation, add E_0 and scale in fp32, and round once (to nearest even) to bf16.
 *    fp32 paths compute in fp32 throughout.
 */
#ifndef NGRAM_EMBED_H
#define NGRAM_EMBED_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status codes */
enum {
  NGRAM_OK = 0,
  NGRAM_EINVAL = -1,     /* a size or count is out of range or inconsistent */
  NGRAM_EDTYPE = -2,     /* unknown dtype */
  NGRAM_EALIGN = -3,     /* a required pointer is NULL or misaligned */
  NGRAM_EWORKSPACE = -4, /* workspace missing, misaligned or too small */
  NGRAM_EOVERFLOW = -5,  /* V0 * max V_{n,k} does not fit the exact 64-bit hash */
  NGRAM_EHIP = -6,       /* the HIP runtime reported an error at launch */
  NGRAM_ESCRATCH = -7    /* the call needs more than the fixed scratch of
                            ngram_embed_decode_noalloc (NGRAM_NOALLOC_SCRATCH_BYTES) */
};

/* dtype of E_0, E_{n,k}, W and of every output */
enum { NGRAM_F32 = 0, NGRAM_BF16 = 1 };

/* device error flags, OR-ed into the int32 at the start of the workspace */
enum {
  NGRAM_FLAG_BAD_TOKEN = 1,   /* a token id outside [0, V0) was hashed */
  NGRAM_FLAG_BAD_SEQLENS = 2, /* cu_seqlens not 0 = c_0 <= c_1 <= ... <= c_nseq = ntok */
  NGRAM_FLAG_BAD_COUNT = 4,   /* n_new or n_accept outside [0, tmax] */
  NGRAM_FLAG_BAD_SLOT = 8,    /* a cache slot outside [0, cache->nseq) */
  NGRAM_FLAG_DUP_SLOT = 16    /* a cache slot that an earlier batch entry of the call uses */
};

/* Embedding amplification (section 3.2.4): what is applied to e_i before it is written.
 * The pages describe both strategies without a formula for the second; the layer
 * normalisation here is the usual one over the D values of a row:
 *   y = (e - mean) / sqrt(var + ln_eps) * ln_weight + ln_bias,  var the biased variance,
 * computed in fp32 from the unrounded e and rounded once. */
enum {
  NGRAM_AMP_NONE = 0,      /* out = e_i: the final form as is */
  NGRAM_AMP_SCALE = 1,     /* out = amp_scale * e_i, one rounding; amp_scale =
                              NGRAM_AMP_SCALE_SQRT_D selects the pages' factor sqrt(D) */
  NGRAM_AMP_LAYERNORM = 2  /* out = LayerNorm(e_i) as above; needs the workspace (prefill,
                              decode), so ngram_embed_project rejects it */
};

/* Form of the layer (section A2). In the basic form there are S = N-1 tables E[s] = E_{s+2}
 * of shape [V_{s+2}, D] (d = D), the hash is the same with one modulus per order, W is not
 * read (may be NULL), and every entry point works as for the final form with
 * W_{n,k} E_{n,k}(.) replaced by E_n(.) and (N-1)K + 1 by N. ngram_embed_gather then writes
 * G [nrows, (N-1)*D]. */
enum {
  NGRAM_FORM_FINAL = 0,  /* the final (Over-Encoding) form, with projections */
  NGRAM_FORM_BASIC = 1   /* the basic form (Eq. 1): K must be 1 */
};

/* amp_scale value that selects sqrt(D), the factor the pages use (section 3.2.4; the
 * popular article prints the radical); the library computes it as sqrtf(D) */
#define NGRAM_AMP_SCALE_SQRT_D 0.0f

#define NGRAM_MAX_ORDER 16         /* largest accepted N */
#define NGRAM_MAX_SUBTABLES 64     /* largest accepted (N-1)K */
#define NGRAM_MAX_DECODE_TOKENS 8  /* largest accepted tmax (1 + speculative drafts) */

/* Layer hyper-parameters (section A2). */
typedef struct ngram_embed_config {
  int32_t N;         /* largest n-gram order, 1 <= N <= NGRAM_MAX_ORDER */
  int32_t K;         /* sub-tables (hash functions) per order, K >= 1, (N-1)K <= 64 */
  int32_t D;         /* hidden size; D * sizeof(dtype) is a multiple of 16 bytes, and in
                        the final form D % ((N-1)K) == 0 and the sub-table row
                        d * sizeof(dtype) is a multiple of 16 bytes */
  int32_t dtype;     /* NGRAM_F32 or NGRAM_BF16 */
  int64_t V0;        /* base vocabulary, 1 <= V0 < 2^31 */
  const int64_t* V;  /* host, S entries: V_{n,k} in sub-table order, 1 <= V < 2^31,
                        and V0 * max V < 2^63 (else NGRAM_EOVERFLOW) */
  int32_t amp;       /* NGRAM_AMP_*; 0 (a zero-filled config) is the final form as is */
  float amp_scale;   /* NGRAM_AMP_SCALE: the factor, finite; NGRAM_AMP_SCALE_SQRT_D (0)
                        for sqrt(D) (ignored otherwise) */
  float ln_eps;      /* NGRAM_AMP_LAYERNORM: variance epsilon, finite and > 0; the layer
                        normalisation also needs D <= 8192 (ignored otherwise) */
  int32_t form;      /* NGRAM_FORM_*; 0 is the final form */
} ngram_embed_config;

/* Parameters of the layer, all in device memory, in the config's dtype. Every device
 * pointer here must be 16-byte aligned. */
typedef struct ngram_embed_tables {
  const void* E0;        /* [V0, D] base embedding E_0 */
  const void* const* E;  /* host array of S device pointers; E[s] is E_{n,k} [V_{n,k}, d] */
  const void* W;         /* [D, D] stacked projection: W[o, s*d + c] = W_{n,k}[o, c]
                            (final form only) */
  const void* ln_weight; /* [D] layer-normalisation weight, or NULL for all ones (read only
                            with NGRAM_AMP_LAYERNORM) */
  const void* ln_bias;   /* [D] layer-normalisation bias, or NULL for zeros (same) */
} ngram_embed_tables;

/* N-gram cache of a batch of sequences in decode (section 4.2): the last N-1 committed ids
 * of every sequence, kept on the device. Committed position p of sequence b sits in
 * ring[b*(N-1) + p mod (N-1)]; positions before 0 read as the pad id 0. */
typedef struct ngram_cache {
  int32_t* ring;  /* device [nseq, N-1] int32 (may be NULL when N = 1) */
  int64_t* len;   /* device [nseq] int64: ids committed so far */
  int32_t nseq;   /* sequences, >= 0 */
} ngram_cache;

/* ---------------------------------------------------------------- workspace
 * Scratch for up to `max_rows` output rows: the error flags (int32 at offset 0), the E_0
 * token of every row (int32 [max_rows] at *tok_off), the hash indices (int32
 * [max_rows, S] at *idx_off) and, with NGRAM_AMP_LAYERNORM, the unrounded rows e_i (fp32
 * [max_rows, D], after the indices) that the normalisation reads. Must be 256-byte
 * aligned and zero-filled once before first use (the flags are sticky until cleared).
 * Returns the size in bytes, 0 on a bad config. */
size_t ngram_embed_workspace_size(const ngram_embed_config* cfg, int64_t max_rows);
int ngram_embed_workspace_layout(const ngram_embed_config* cfg, int64_t max_rows,
                                 size_t* tok_off, size_t* idx_off);

/* ---------------------------------------------------------------- kernel 1: hash
 * idx[i*S + s] = H_{n,k} of position i (section A2 rolling hash), for ntok packed tokens
 * split into nseq sequences by cu_seqlens (device int32 [nseq+1], c_0 = 0, c_nseq = ntok).
 * tokens: device int32 [ntok]; idx: device int32 [ntok, S]. The reduction is Horner's rule
 * modulo V_{n,k} in exact 64-bit integers, so no intermediate overflows.
 * err_flags: device int32 or NULL; bad ids and bad cu_seqlens are OR-ed into it (their
 * rows hold unspecified but in-range indices). */
int ngram_embed_hash(const ngram_embed_config* cfg, const int32_t* tokens,
                     const int32_t* cu_seqlens, int32_t nseq, int64_t ntok, int32_t* idx,
                     int32_t* err_flags, void* stream);

/* ---------------------------------------------------------------- kernel 2: gather
 * G[r, s*d + c] = E_{n,k}[idx[r*S + s], c] for nrows rows: the concatenation of the S
 * sub-table rows that the final form reads (section A2). G: device [nrows, D] in the
 * config's dtype, 16-byte aligned. Indices are clamped into [0, V_{n,k}) so a bad index
 * never reads outside its table. Stand-alone form of the gather that ngram_embed_project
 * fuses into its matrix-core loads. */
int ngram_embed_gather(const ngram_embed_config* cfg, const ngram_embed_tables* tables,
                       const int32_t* idx, int64_t nrows, void* G, void* stream);

/* The same gather in the form the projection performs it (kernel 2 into on-chip memory):
 * each sub-table row goes from HBM straight into LDS (16 bytes per lane, the projection's
 * A-loader instruction) and is reduced where it lands to one checksum per gathered row,
 *   sums[r] = sum_k w_k * (2k + 1)  mod 2^32,
 * w_k the 32-bit words (little-endian) of row r of the G that ngram_embed_gather writes.
 * Only sums [nrows] (device uint32, 4-byte aligned) is written, so the call moves the
 * gather's HBM reads alone; indices are clamped as in ngram_embed_gather. For measuring the
 * gather's HBM -> LDS rate, and for checking byte for byte what the LDS loads deliver. */
int ngram_embed_gather_checksum(const ngram_embed_config* cfg, const ngram_embed_tables* tables,
                                const int32_t* idx, int64_t nrows, uint32_t* sums,
                                void* stream);

/* ---------------------------------------------------------------- kernels 2+3: projection
 * out[r, :] = ( E_0[tok[r], :] + sum_s W_{n,k} E_{n,k}[idx[r*S + s], :] ) / (S + 1)
 * (times amp_scale with NGRAM_AMP_SCALE; NGRAM_AMP_LAYERNORM returns NGRAM_EINVAL here)
 * for nrows rows: the sub-table rows are gathered straight into on-chip memory and
 * multiplied by the stacked W on the matrix cores, with the E_0 add and the scale in the
 * epilogue. tok: device int32 [nrows]; rows whose tok is outside [0, V0) are written as
 * zeros (decode uses -1 for unused slots). idx as produced by ngram_embed_hash (clamped
 * like ngram_embed_gather). out: device [nrows, D] in the config's dtype. */
int ngram_embed_project(const ngram_embed_config* cfg, const ngram_embed_tables* tables,
                        const int32_t* idx, const int32_t* tok, int64_t nrows, void* out,
                        void* stream);

/* ---------------------------------------------------------------- prefill
 * The whole forward pass over packed sequences: ngram_embed_hash into the workspace, then
 * ngram_embed_project with tok = tokens, then the amplification the config selects (the
 * layer normalisation as a second pass over the unrounded rows kept in the workspace; rows
 * of ids outside [0, V0) stay zero). out: device [ntok, D]. ws: workspace of at least
 * ngram_embed_workspace_size(cfg, ntok) bytes; bad ids set NGRAM_FLAG_BAD_TOKEN there.
 * cache_or_null: NULL, or an N-gram cache with cache->nseq == nseq that the same call fills
 * for decoding on after the prompts (section 4.2), exactly as ngram_cache_init would: slot b
 * gets sequence b's length and its last N-1 ids (pad id 0 before its start); bad cu_seqlens
 * set NGRAM_FLAG_BAD_SEQLENS in the workspace. A cache with another nseq is NGRAM_EINVAL. */
int ngram_embed_prefill(const ngram_embed_config* cfg, const ngram_embed_tables* tables,
                        const int32_t* tokens, const int32_t* cu_seqlens, int32_t nseq,
                        int64_t ntok, void* out, ngram_cache* cache_or_null, void* ws,
                        size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- kernel 4: decode
 * Fill a cache from prefilled sequences: len[b] = sequence length, ring = its last N-1 ids
 * (slots of positions before 0 hold the pad id 0). tokens/cu_seqlens as in
 * ngram_embed_hash with nseq = cache->nseq. */
int ngram_cache_init(const ngram_embed_config* cfg, ngram_cache* cache, const int32_t* tokens,
                     const int32_t* cu_seqlens, int64_t ntok, void* stream);

/* One decode / speculative-verify step. new_tokens: device int32 [nseq, tmax]; sequence b
 * proposes its first n_new[b] entries (device int32 [nseq], 0 <= n_new <= tmax <= 8) as the
 * positions len[b], len[b]+1, ... . out[b, j, :] (device [nseq, tmax, D]) is the embedding
 * that a prefill of (committed history, new_tokens[b, 0..j]) gives its last position; rows
 * j >= n_new[b] are zeros (also with amplification, which applies as in prefill). The
 * context comes from the cache (the last N-1 committed ids),
 * never from the host. If n_commit (device int32 [nseq], 0 <= n_commit <= n_new) is not
 * NULL, the first n_commit[b] new ids are then appended to the cache, as by
 * ngram_cache_commit. ws: at least ngram_embed_workspace_size(cfg, nseq * tmax) bytes; the
 * step's indices stay there (layout above) until the next call. */
int ngram_embed_decode(const ngram_embed_config* cfg, const ngram_embed_tables* tables,
                       ngram_cache* cache, const int32_t* new_tokens, const int32_t* n_new,
                       int32_t tmax, const int32_t* n_commit, void* out, void* ws,
                       size_t ws_bytes, void* stream);

/* Append the first n_accept[b] (device int32 [nseq], 0 <= n_accept <= tmax) ids of
 * new_tokens[b, :] (device int32 [nseq, tmax]) to sequence b's cache and advance len[b].
 * err_flags: device int32 or NULL (NGRAM_FLAG_BAD_COUNT; such counts are clamped). */
int ngram_cache_commit(const ngram_embed_config* cfg, ngram_cache* cache,
                       const int32_t* new_tokens, const int32_t* n_accept, int32_t tmax,
                       int32_t* err_flags, void* stream);

/* ---------------------------------------------------------------- pooled cache, row windows
 * For schedulers with dynamic batches and for speculative decoding (section 4.2: the N-gram
 * cache is managed like a KV cache; n-gram embeddings computed while the draft model
 * proposes tokens are reused by the verify step).
 *
 * The cache is a pool of cache->nseq slots. Batch entry b (0 <= b < nbatch) uses slot
 * slots[b] (device int32 [nbatch]; NULL means slot b, and then nbatch <= cache->nseq).
 * Slots of one call must be distinct. An out-of-range slot sets NGRAM_FLAG_BAD_SLOT in the
 * workspace (or err_flags) and the entry is ignored (no rows written, no commit); so does a
 * slot that an earlier entry of the call (smaller b) uses, with NGRAM_FLAG_DUP_SLOT (the
 * earlier entry is served as usual). The check compares each entry with the earlier ones
 * (quadratic in nbatch, negligible at batch sizes of thousands).
 *
 * ngram_embed_decode_rows computes, for each batch entry b, the rows j in
 * [row_begin, min(row_end, n_new[b])) exactly as ngram_embed_decode would (same bits), and
 * writes nothing else: rows outside that range keep their contents. Contexts come from the
 * slot's committed ids and new_tokens[b, 0..j] (ids before row_begin included), so a caller
 * can fill out[b, j] as each draft id j appears (row_begin = j, row_end = j + 1) and find
 * every row ready at verify time. 0 <= row_begin < row_end <= tmax <= 8. n_commit (optional)
 * commits as in ngram_embed_decode. ws: at least
 * ngram_embed_workspace_size(cfg, nbatch * (row_end - row_begin)) bytes.
 * ngram_cache_init_slots fills slot slots[b] from sequence b of the packed tokens (entries
 * joining the pool; other slots untouched); ngram_cache_commit_slots appends the first
 * n_accept[b] ids of new_tokens[b, :] to slot slots[b]. */
int ngram_embed_decode_rows(const ngram_embed_config* cfg, const ngram_embed_tables* tables,
                            ngram_cache* cache, const int32_t* slots, int32_t nbatch,
                            const int32_t* new_tokens, const int32_t* n_new, int32_t tmax,
                            int32_t row_begin, int32_t row_end, const int32_t* n_commit,
                            void* out, void* ws, size_t ws_bytes, void* stream);
int ngram_cache_init_slots(const ngram_embed_config* cfg, ngram_cache* cache,
                           const int32_t* slots, int32_t nbatch, const int32_t* tokens,
                           const int32_t* cu_seqlens, int64_t ntok, int32_t* err_flags,
                           void* stream);
int ngram_cache_commit_slots(const ngram_embed_config* cfg, ngram_cache* cache,
                             const int32_t* slots, int32_t nbatch, const int32_t* new_tokens,
                             const int32_t* n_accept, int32_t tmax, int32_t* err_flags,
                             void* stream);

/* ---------------------------------------------------------------- per-layer embeddings
 * Per-layer N-gram embedding (PLNE, section 5.2 of the same page): every layer l of a model
 * computes the layer's output with embedding tables and projections of its own, from the
 * same token ids (the model then uses out[l] inside layer l's feed-forward block). One
 * config serves every layer, so the hash indices are computed once and shared; the
 * projections of up to 8 layers (at most 128 sub-table pointers in all) run in one launch,
 * blockIdx.z selecting the layer. Each layer's output has the same bits as a single-layer
 * call with that layer's tables.
 * tables: host array of nlayers >= 1 tables (each as for one layer); out: host array of
 * nlayers device pointers, out[l] [ntok, D] (prefill) or [nseq, tmax, D] (decode), 16-byte
 * aligned. ws: as for one layer (its size does not depend on nlayers). With
 * NGRAM_AMP_LAYERNORM the layers run one after another through the workspace. The decode
 * cache and n_commit work as in ngram_embed_decode: the step is committed once. */
int ngram_embed_prefill_layers(const ngram_embed_config* cfg, const ngram_embed_tables* tables,
                               int32_t nlayers, const int32_t* tokens,
                               const int32_t* cu_seqlens, int32_t nseq, int64_t ntok,
                               void* const* out, void* ws, size_t ws_bytes, void* stream);
int ngram_embed_decode_layers(const ngram_embed_config* cfg, const ngram_embed_tables* tables,
                              int32_t nlayers, ngram_cache* cache, const int32_t* new_tokens,
                              const int32_t* n_new, int32_t tmax, const int32_t* n_commit,
                              void* const* out, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- backward (training)
 * Gradients of the layer for one batch, given the upstream gradient dout = dL/dout
 * (device [ntok, D], config dtype, 16-byte aligned) of out = ngram_embed_prefill(tokens).
 * The pages train the layer from scratch but state no backward; these are the plain
 * derivatives of the final form (section A2), with c = amp_scale / ((N-1)K + 1) for
 * NGRAM_AMP_SCALE and 1 / ((N-1)K + 1) otherwise:
 *   dE0[t, :]  += c * sum of dout[i, :] over positions i with token t
 *   dW         += c * dout^T G,  G[i, s*d + j] = E_{n,k}[h_{i,s}, j]  (W's stacked layout)
 *   dE[s][r, :] += c * sum over positions i with h_{i,s} = r of (dout W)[i, s*d : (s+1)*d]
 * All gradient buffers are caller-owned fp32 device memory, accumulated into (zero them to
 * start a step): dE0 [V0, D], dE = host array of S device pointers to [V_{n,k}, d], dW
 * [D, D]; any of them may be NULL to skip it. Positions whose token is outside [0, V0)
 * contribute nothing (their forward rows are zero). The result does not depend on thread
 * timing: repeated ids are summed in position order (sort + segmented sums, no atomics).
 * NGRAM_AMP_LAYERNORM is not differentiated here (NGRAM_EINVAL). In the basic form there is
 * no W: dE[s][r, :] += c * sum over positions i with h_{i,s} = r of dout[i, :], with
 * c = amp_scale / N or 1 / N, and dW must be NULL (else NGRAM_EINVAL). tokens/cu_seqlens/nseq as
 * in ngram_embed_prefill; ntok * max(S, 1) < 2^31. ws: at least
 * ngram_embed_backward_workspace_size(cfg, ntok) bytes, 256-byte aligned, flags at offset 0
 * as for the forward workspace (bad ids set NGRAM_FLAG_BAD_TOKEN). */
size_t ngram_embed_backward_workspace_size(const ngram_embed_config* cfg, int64_t ntok);
int ngram_embed_backward(const ngram_embed_config* cfg, const ngram_embed_tables* tables,
                         const int32_t* tokens, const int32_t* cu_seqlens, int32_t nseq,
                         int64_t ntok, const void* dout, float* dE0, float* const* dE,
                         float* dW, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- hash statistics
 * Hash collisions and table hit counts of order n (section 3.2.2 and Fig. 3 of the same
 * page), over every position of ntok packed tokens (the n-grams a layer hashes: pad id 0
 * before a sequence's start; tokens/cu_seqlens/nseq as in ngram_embed_hash):
 *   rows[v]   = number of distinct table rows H_n = (n-gram value) mod vocab[v] in use,
 *   *distinct = number of distinct n-grams (if distinct is not NULL).
 * The pages count as collisions the unique n-grams lost to the modulo, distinct - rows[v];
 * the hit rate is rows[v] / vocab[v]. Exact integers: H_n by the same Horner reduction as
 * ngram_embed_hash; distinct from the exact n-gram values, which needs V0^n <= 2^63 (else
 * NGRAM_EOVERFLOW; rows alone work for any n). vocab: host array of nvocab >= 0 table sizes,
 * 1 <= vocab[v] < 2^31; 1 <= n <= NGRAM_MAX_ORDER; 1 <= V0 < 2^31. rows: device int64
 * [nvocab]; distinct: device int64 [1]; both overwritten. ws: at least
 * ngram_hash_stats_workspace_size(...) bytes (0 on bad arguments), 256-byte aligned, error
 * flags at offset 0 as in the forward workspace: zero-filled once before first use, sticky
 * until cleared (NGRAM_FLAG_BAD_TOKEN, NGRAM_FLAG_BAD_SEQLENS; counts then unspecified). The
 * rest of the workspace is written by the call before it is read, so it needs no clearing. */
size_t ngram_hash_stats_workspace_size(int64_t V0, int32_t n, int64_t ntok,
                                       const int64_t* vocab, int32_t nvocab);
int ngram_hash_stats(int64_t V0, int32_t n, const int32_t* tokens, const int32_t* cu_seqlens,
                     int32_t nseq, int64_t ntok, const int64_t* vocab, int32_t nvocab,
                     int64_t* rows, int64_t* distinct, void* ws, size_t ws_bytes,
                     void* stream);

/* ---------------------------------------------------------------- allocation-free decode
 * For callers that cannot allocate device memory or bring a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation. The same step as
 * ngram_embed_decode (same kernels, same output bits, same cache update), with the scratch
 * that the workspace would hold (each row's E_0 token and hash indices, and the unrounded
 * rows of NGRAM_AMP_LAYERNORM) in a fixed array of NGRAM_NOALLOC_SCRATCH_BYTES in device
 * memory that the library declares statically: each GPU the library runs on holds one copy
 * until the process ends. The call allocates nothing; it needs
 * ngram_embed_workspace_size(cfg, cache->nseq * tmax) <= NGRAM_NOALLOC_SCRATCH_BYTES (for
 * example 256 sequences x 5 ids of a 12-sub-table layer take 67 KB, 15.8 MB with the layer
 * normalisation at D = 3072), else it returns NGRAM_ESCRATCH and enqueues nothing.
 * err_flags: device int32 the step's flags are OR-ed into, or NULL. `stream` must belong to
 * the current device (NGRAM_EINVAL otherwise). Every call on one GPU uses that GPU's one
 * array and leaves its contents there: calls that overlap in time on one GPU (other streams,
 * other host threads) race and must be ordered by the caller. Other arguments as in
 * ngram_embed_decode. */
#define NGRAM_NOALLOC_SCRATCH_BYTES (16u << 20)
int ngram_embed_decode_noalloc(const ngram_embed_config* cfg, const ngram_embed_tables* tables,
                               ngram_cache* cache, const int32_t* new_tokens,
                               const int32_t* n_new, int32_t tmax, const int32_t* n_commit,
                               void* out, int32_t* err_flags, void* stream);

/* ---------------------------------------------------------------- errors
 * Wait for `stream`, then copy the workspace's error flags to *flags (host). */
int ngram_embed_read_error_flag(const void* ws, int32_t* flags, void* stream);
/* Enqueue a reset of the workspace's error flags to 0 (a kernel, not a memset, so it may be
 * captured in a HIP graph). */
int ngram_embed_clear_error_flag(void* ws, void* stream);
/* Static English text for a status code. */
const char* ngram_embed_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* NGRAM_EMBED_H */
