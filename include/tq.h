/*
 * tq.h -- C ABI of the MI355X TurboQuant library (libtq.so).
 *
 * What the library computes (pages cited by title and section):
 *  - [ebisuda] "TurboQuant: Google's 6x KV Cache Compression Algorithm Gains
 *    Open-Source Momentum", section 第1段階：PolarQuant: rotate every vector by
 *    a random orthogonal matrix (QR of a Gaussian matrix), then quantize each
 *    rotated coordinate with a precomputed, data-oblivious Lloyd-Max codebook;
 *    no per-block scale or zero point.
 *  - [ebisuda] section 第2段階：QJL残差補正: a 1-bit QJL sketch of the residual
 *    corrects the inner-product bias of stage 1.
 *  - [hakusoku] "TurboQuant: 極限圧縮によるAI効率の再定義", section QJL: the
 *    sketch keeps only sign bits and is paired with a full-precision query.
 *  - [gemilab] TurboQuant technical deep dive, section Attention機構:
 *    softmax(q K^T / sqrt(d_k)) V over the cached K/V.
 *
 * Conventions
 *  - Pointers named d_* are device pointers owned by the caller; the library
 *    never allocates, frees or retains them. Pointers named h_* are host
 *    pointers, read or written only during the call.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Hot
 *    calls only enqueue work on it and never synchronize; tq_ctx_create and
 *    tq_ctx_destroy synchronize the device.
 *  - Every call validates its arguments before launching anything. On failure
 *    it returns a non-zero tq_status, writes no output, and sets a message
 *    readable with tq_last_error() (thread-local). A failed kernel launch
 *    returns TQ_ERR_HIP. No C++ exception crosses this boundary.
 *  - The library runs on the device that is current when tq_ctx_create is
 *    called; later calls must be made with that device current.
 *  - Dimensions: d is a multiple of 32 in [32, 4096]; the sketch has m = d
 *    rows (the sizes the workloads fix); MSE bit widths are 1..4 (0 for pure
 *    QJL keys).
 *
 * Packed formats (fixed by this library; the pages fix none)
 *  Keys (B MSE bits + Q QJL bits per coordinate), one record per vector,
 *  W = d/32 coordinate groups. Q = 1 is TurboQuant (stage 1 + the QJL
 *  sketch of the residual); Q = 0 keeps stage 1 alone (MSE-only keys, a
 *  biased inner product); B = 0 with Q = 1 keeps the sketch alone (pure QJL
 *  keys: the residual is the whole rotated unit vector):
 *    bits  uint32 [n][W][B+Q]: for group w, word p < B holds bit p of the
 *          codebook index of coordinate 32w+k at bit k; word B (Q = 1) holds
 *          the QJL sign bit of sketch row 32w+k at bit k (1 = non-negative).
 *    norms float32 [n][1+Q] = (||k||) or (||k||, ||r||), r the rotated-domain
 *          residual.
 *    A zero vector has an all-zero record.
 *  Values (B MSE bits per coordinate, no sketch), token-major 32-token
 *  blocks:
 *    bits  uint32 [n/32][d][B]: word [t/32][j][p] holds bit p of the index of
 *          token t, coordinate j, at bit t%32.
 *    norms float32 [n] = ||v||.
 *  Bytes per token at d = 128: keys 56 (b=3) / 72 (b=4) / 52 (3-bit MSE-only)
 *  / 24 (pure QJL); 3-bit values 52.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TQ_OK = 0,
  TQ_ERR_ARG = 1,          /* invalid argument (NULL, size, stride, dtype) */
  TQ_ERR_UNSUPPORTED = 2,  /* valid but not supported (d, bits, heads)      */
  TQ_ERR_CAPACITY = 3,     /* cache full / workspace too small              */
  TQ_ERR_HIP = 4,          /* HIP runtime or launch failure                 */
  TQ_ERR_NOMEM = 5         /* host or device allocation failed (ctx only)   */
} tq_status;

typedef enum { TQ_F32 = 0, TQ_BF16 = 1 } tq_dtype;

#define TQ_MAX_BITS 4
#define TQ_MAX_DIM 4096

/* Version of the packed record formats below (bit planes, sign words, norms,
 * value blocks, PolarQuant records). Records written by a library of one
 * version are read only by a library of the same version; tq_format_version()
 * returns the version the loaded library implements, so a caller can check it
 * against the header it was compiled with. */
#define TQ_FORMAT_VERSION 1
int32_t tq_format_version(void);

/* Lloyd-Max codebook for one rotated coordinate of a d-dimensional unit
 * vector ([ebisuda] 第1段階: the coordinate law is Beta, close to N(0,1/d)).
 * Density used: f_d(x) = (1-x^2)^((d-3)/2) / B(1/2,(d-1)/2) on [-1,1].
 * centroid[0..2^bits-1] ascending, fp32 of the fp64 fixed point (made exactly
 * antisymmetric); boundary[i] = fp32 of the fp64 midpoint of centroids i,i+1;
 * a coordinate y gets index #{i : boundary[i] <= y}. walsh[] holds the odd
 * Walsh coefficients of the centroid table (see tq_ctx internals) and
 * distortion the per-coordinate MSE of the stored table under f_d. */
typedef struct {
  int32_t d;
  int32_t bits;
  float centroid[16];
  float boundary[15];
  float walsh[8];
  double distortion;
} tq_codebook;

/* Host only, deterministic, no GPU. d in [3, TQ_MAX_DIM], bits in [1, 4].
 * Errors: TQ_ERR_ARG (out NULL), TQ_ERR_UNSUPPORTED (d or bits out of range). */
tq_status tq_codebook_build(int32_t d, int32_t bits, tq_codebook *out);

/* Host only, no GPU: the fp32 rotation tq_ctx_create would use for the
 * row-major d x d float64 Gaussian matrix h_g (Householder QR, Q made unique
 * by a positive diag(R), sign(0)=+1; [ebisuda] 第1段階), written row-major to
 * h_out (d*d floats, caller-owned). d in [2, TQ_MAX_DIM].
 * Errors: TQ_ERR_ARG (NULL), TQ_ERR_UNSUPPORTED (d). */
tq_status tq_rotation_build(int32_t d, const double *h_g, float *h_out);

/* PolarQuant angle codebook ([arxiv-summary] 3.中核となる技術的要素: codebooks
 * designed from the distribution of the angles of the recursive polar
 * transformation). Level 1 (angles of coordinate pairs, uniform on the circle):
 * the uniform grid with cells from -pi. Level l >= 2 (angles of radius pairs,
 * m = 2^(l-1): sin^2(psi) ~ Beta(m/2, m/2) on [0, pi/2]): Lloyd-Max, made
 * symmetric about pi/4. centroid: fp64; boundary, cos_c, sin_c: fp32 (of the
 * fp64 midpoints / cos / sin of the centroids); code = #{boundary <= psi}. */
#define TQ_POLAR_MAX_LEVEL 12
typedef struct {
  int32_t level;
  int32_t bits;
  double centroid[16];
  float boundary[15];
  float cos_c[16];
  float sin_c[16];
} tq_angle_codebook;

/* Host only. level in [1, 12], bits in [1, 4].
 * Errors: TQ_ERR_ARG (out NULL), TQ_ERR_UNSUPPORTED (level or bits). */
tq_status tq_angle_codebook_build(int32_t level, int32_t bits, tq_angle_codebook *out);

/* A packed array of PolarQuant key records, d = 128 ([arxiv-summary]
 * 3.中核となる技術的要素; [gemilab] PolarQuant：極座標変換による根本的削減).
 * Vector x: y = Pi x (random preconditioning by the context's rotation), then
 * the recursive polar transformation: level 1 turns coordinate pair i into
 * (hypot, atan2(y[2i+1], y[2i])), level l >= 2 turns the radius pair (2i,
 * 2i+1) of level l-1 into (hypot, atan2(right, left)); 64 + 63 angles and the
 * radius ||x||. Each angle is coded by its level's tq_angle_codebook (b1 bits
 * at level 1, b2 at the higher levels). Record: w1 = ceil(64 b1 / 32) words of
 * level-1 codes (code i at bit i*b1 of that little-endian stream), then
 * w2 = ceil(63 b2 / 32) words of higher codes (level 2 nodes first, code j at
 * bit j*b2); norms[i] = ||x|| (fp32). 60 bytes per vector at (b1, b2) = (4, 3):
 * 4.27x against fp16. */
typedef struct {
  uint32_t *bits;  /* d_: [n][w1 + w2] */
  float *norms;    /* d_: [n] */
  int64_t n;       /* records */
  int32_t b1, b2;  /* bits per level-1 / higher-level angle, 1..4 */
} tq_polar_packed;

/* Library context: the rotation Pi (d x d), the sketch S (d x d) and the
 * codebooks for bits 1..4, on host and device. Immutable after creation and
 * safe to share across streams on its device. */
typedef struct tq_ctx tq_ctx;

/* h_g_rot, h_g_sketch: row-major d x d float64 matrices of i.i.d. N(0,1)
 * draws supplied by the caller (the random numbers the method draws).
 * Pi = Q diag(sign(diag R)) from the Householder QR of h_g_rot (sign(0)=+1),
 * rounded to fp32, used as y = Pi u ([ebisuda] 第1段階); S = fp32(h_g_sketch)
 * ([gemilab] QJLの応用). Synchronizes the current device.
 * Errors: TQ_ERR_ARG, TQ_ERR_UNSUPPORTED (d), TQ_ERR_NOMEM, TQ_ERR_HIP. */
tq_status tq_ctx_create(int32_t d, const double *h_g_rot, const double *h_g_sketch, tq_ctx **out);

/* Seeded Gaussian draws, host only, no GPU. The pages fix only that the
 * rotation is the QR factor of a Gaussian matrix ([ebisuda] 第1段階) and that
 * the sketch is a Gaussian matrix ([gemilab] QJLの応用); the seed-to-matrix map
 * is this library's: word i = mix(seed ^ stream * 0x9E3779B97F4A7C15 ^ i)
 * (mod 2^64), mix the SplitMix64 output function (Steele, Lea & Flood,
 * OOPSLA 2014), u_i = (word_i >> 11) * 2^-53; entries 2k, 2k + 1 (row-major)
 * are r cos(2 pi u_{2k+1}), r sin(2 pi u_{2k+1}) with r = sqrt(-2 ln(1 -
 * u_{2k})) (Box-Muller), fp64. Stream TQ_STREAM_ROTATION draws the matrix
 * behind Pi, TQ_STREAM_SKETCH the sketch. h_out: rows * cols doubles,
 * caller-owned; rows * cols must be even.
 * Errors: TQ_ERR_ARG (NULL, sizes). */
#define TQ_STREAM_ROTATION 1
#define TQ_STREAM_SKETCH 2
tq_status tq_gaussian_matrix(uint64_t seed, uint32_t stream, int32_t rows, int32_t cols, double *h_out);

/* A context from a seed alone: tq_ctx_create(d, G_rot, G_sketch) with
 * G_rot = tq_gaussian_matrix(seed, TQ_STREAM_ROTATION, d, d) and
 * G_sketch = tq_gaussian_matrix(seed, TQ_STREAM_SKETCH, d, d) ([ebisuda]
 * 第1段階: QR of a seeded Gaussian matrix). Synchronizes the current device.
 * Errors: as tq_ctx_create. */
tq_status tq_ctx_create_seeded(int32_t d, uint64_t seed, tq_ctx **out);
tq_status tq_ctx_destroy(tq_ctx *ctx);
int32_t tq_ctx_dim(const tq_ctx *ctx);
/* Host copies of the fp32 tables (either output may be NULL). */
tq_status tq_ctx_export(const tq_ctx *ctx, float *h_rot, float *h_sketch);
tq_status tq_ctx_codebook(const tq_ctx *ctx, int32_t bits, tq_codebook *out);

/* A packed array of key or value records (formats above). */
typedef struct {
  uint32_t *bits;  /* d_: keys [n][W][B+Q]; values [n/32][d][B]     */
  void *norms;     /* d_: keys [n][1+Q]; values [n]; fp32, or fp16
                      when norm_f16                                   */
  int64_t n;       /* record capacity; a multiple of 32 for values   */
  int32_t mse_bits;/* B: 1..4 (keys with qjl = 1: 0..4)              */
  int32_t is_key;  /* 1 = key format, 0 = values                     */
  int32_t qjl;     /* keys: Q, 1 = QJL sign word and ||r||, 0 = none;
                      values: 0                                       */
  int32_t norm_f16;/* 1: norms stored as fp16 (round to nearest even,
                      saturated at 65504): 2 bytes per norm instead of
                      4, the compact-norm record format; 0: fp32      */
} tq_packed;

/* Quantize vectors ([ebisuda] 第1段階 and, for keys, 第2段階).
 * Input element (s, t, j) is at d_x[s*x_stream_stride + t*x_token_stride + j]
 * (strides in elements, j contiguous) for s < n_streams, t < n_tokens.
 * Its record goes to index s*out_stream_stride + out_offset + t of `out`.
 * Keys: norm, rotation, codebook index, residual r (rotated domain), ||r||,
 * sign(S r). Values: norm, rotation, codebook index; a value call writes
 * whole 32-token blocks, so out_offset and out_stream_stride must be
 * multiples of 32 (bits of tokens past n_tokens in the last block are 0).
 * d_work: device workspace of tq_quantize_ws_bytes() bytes (keys only; may
 * be NULL for values).
 * Errors: TQ_ERR_ARG (NULL, negative sizes, records out of range, alignment),
 * TQ_ERR_UNSUPPORTED (bits), TQ_ERR_CAPACITY (workspace), TQ_ERR_HIP. */
size_t tq_quantize_ws_bytes(const tq_ctx *ctx, int64_t n_streams, int64_t n_tokens, int32_t is_key);
tq_status tq_quantize_kv(const tq_ctx *ctx, const void *d_x, tq_dtype dtype, int64_t n_streams, int64_t n_tokens,
                         int64_t x_stream_stride, int64_t x_token_stride, const tq_packed *out,
                         int64_t out_stream_stride, int64_t out_offset, void *d_work, size_t work_bytes,
                         void *stream);

/* KV cache. Contiguous layout (d_block_table NULL): the record of token t of
 * stream (b, h) is [(b*kv_heads + h)*capacity + t]; k.n, v.n >=
 * batch*kv_heads*capacity. Paged layout (d_block_table non-NULL): the arrays
 * are a pool of n_pages = k.n / (kv_heads*page_tokens) pages of page_tokens
 * tokens per KV head, and token t of stream (b, h) is record
 * (page*kv_heads + h)*page_tokens + t % page_tokens with
 * page = d_block_table[b*(capacity/page_tokens) + t/page_tokens] (device
 * int32, [batch][capacity/page_tokens], caller-owned; sequences may share or
 * reorder pages freely). page_tokens is a positive multiple of 256 dividing
 * capacity; k.n = v.n = a multiple of kv_heads*page_tokens. A table entry
 * outside [0, n_pages) is a caller error: it is clamped, so no access leaves
 * the arrays, but the data read or written is then another page's. Pages of
 * 1024 tokens or more keep the decode kernel at its full chunk size.
 * capacity is a multiple of 32. d_seq_len[b] is the number of valid tokens of
 * every KV head of sequence b. host_max_len is an upper bound of all
 * d_seq_len kept by the caller after prefill and advanced by
 * tq_append_token; it sizes the decode launch and guards capacity. */
typedef struct {
  tq_packed k, v;
  int32_t batch, kv_heads, capacity;
  int32_t *d_seq_len;
  int32_t host_max_len;
  const int32_t *d_block_table; /* NULL: contiguous layout */
  int32_t page_tokens;          /* paged layout only */
} tq_kv_cache;

/* Write n_tokens tokens of every stream into the cache (contiguous or paged)
 * at positions pos0 .. pos0 + n_tokens - 1, keys and values
 * ([ebisuda] 第1段階 and 第2段階, as tq_quantize_kv): K/V element (s, t, j) of
 * stream s = b*kv_heads + h is d_k / d_v[s*x_stream_stride + t*x_token_stride
 * + j] (strides in elements, both inputs alike). pos0 is a multiple of 32
 * (value records are written in whole 32-token blocks; bits of positions past
 * the last token in its block are 0). d_seq_len and host_max_len are not
 * changed: the caller sets them. d_work: tq_quantize_ws_bytes(ctx,
 * batch*kv_heads, n_tokens, 1) bytes.
 * Errors: TQ_ERR_ARG (NULL, strides, alignment, pos0, positions past
 * capacity), TQ_ERR_CAPACITY (workspace), TQ_ERR_HIP. */
tq_status tq_cache_write(const tq_ctx *ctx, const tq_kv_cache *cache, const void *d_k, const void *d_v,
                         tq_dtype dtype, int64_t n_tokens, int64_t x_stream_stride, int64_t x_token_stride,
                         int64_t pos0, void *d_work, size_t work_bytes, void *stream);

/* Append one token per sequence: quantize d_k[b][h][:] / d_v[b][h][:]
 * (contiguous [batch][kv_heads][d]) and write them at position d_seq_len[b]
 * of stream (b, h), then increment d_seq_len[b] (O(1) append; the cache
 * requirement is stated in the fractal KV-archive summary on gist.science).
 * Increments cache->host_max_len.
 * Errors: TQ_ERR_ARG, TQ_ERR_CAPACITY (host_max_len + 1 > capacity),
 * TQ_ERR_HIP. */
tq_status tq_append_token(const tq_ctx *ctx, tq_kv_cache *cache, const void *d_k, const void *d_v, tq_dtype dtype,
                          void *stream);

/* One decode step ([gemilab] Attention機構 with the estimator of [ebisuda]
 * 第2段階): for every sequence b and query head h (KV head h / (q_heads /
 * kv_heads)), out[b][h] = sum_t p_t v_hat_t with p = softmax(scale * s_t)
 * over t < d_seq_len[b], s_t the TurboQuant score of q against key t, and
 * v_hat_t = ||v_t|| Pi^T c[idx_t]. d_q: [batch][q_heads][d]; d_out: fp32
 * [batch][q_heads][d]. q_heads must be a multiple of kv_heads. A sequence
 * with length 0 gets a zero output.
 * d_ws: workspace of tq_attention_decode_ws_bytes() bytes.
 * Errors: TQ_ERR_ARG, TQ_ERR_UNSUPPORTED (d != 128, group > 16),
 * TQ_ERR_CAPACITY (workspace), TQ_ERR_HIP. */
size_t tq_attention_decode_ws_bytes(const tq_ctx *ctx, const tq_kv_cache *cache, int32_t q_heads);
tq_status tq_attention_decode(const tq_ctx *ctx, const tq_kv_cache *cache, const void *d_q, tq_dtype dtype,
                              int32_t q_heads, float scale, float *d_out, void *d_ws, size_t ws_bytes,
                              void *stream);

/* tq_attention_decode without a caller workspace, for callers that cannot
 * allocate device memory or pass one (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation). The same kernels and
 * result as tq_attention_decode; the workspace (query fragments, per-chunk
 * softmax partials) is a library-held scratch array of TQ_SCRATCH_BYTES per
 * device, whose device address is looked up once per device when a context
 * is created there, and which lives until the process ends. The call itself
 * allocates nothing (no hipMalloc, no hipFree) and clears nothing: every byte
 * a call reads from the scratch is written by that call first. All calls on
 * one device share that device's array, so calls that overlap on one device
 * (two streams, or two threads) race and must be serialized by the caller.
 * Errors: as tq_attention_decode; TQ_ERR_CAPACITY when the call needs more
 * than TQ_SCRATCH_BYTES (tq_attention_decode_ws_bytes() > TQ_SCRATCH_BYTES;
 * e.g. 64 sequences x 8 KV heads x 32 query heads at 8K tokens need 14 MB). */
#define TQ_SCRATCH_BYTES (32u << 20)
tq_status tq_attention_decode_noalloc(const tq_ctx *ctx, const tq_kv_cache *cache, const void *d_q, tq_dtype dtype,
                                      int32_t q_heads, float scale, float *d_out, void *stream);

/* Attention of many query positions per sequence over the packed cache (the
 * cache part of chunked prefill; [gemilab] Attention機構 with the estimator
 * of [ebisuda] 第2段階, as tq_attention_decode): for every sequence b, query
 * position i < n_q and query head h, out[b][i][h] = sum_t p_t v_hat_t with
 * p = softmax(scale * s_t) over the visible tokens t: t < d_seq_len[b], and
 * with causal != 0 only t < d_seq_len[b] - n_q + i + 1 (the chunk's own
 * tokens already appended, each position sees itself and what precedes it).
 * A query with no visible token gets a zero output.
 * d_q: [batch][n_q][q_heads][d]; d_out: fp32 [batch][n_q][q_heads][d]. q_heads
 * a multiple of kv_heads; the n_q * group (query position, head) pairs of a KV
 * head are its virtual heads. With at least 16 of them, n_q >= 2, values of at
 * most 3 bits and a contiguous cache (or pages of a multiple of 512 tokens) a
 * prefill kernel scores 16 virtual heads per work-group; otherwise the decode
 * kernels run over groups of 4. d_ws: workspace of
 * tq_attention_prefill_ws_bytes() bytes.
 * Errors: TQ_ERR_ARG, TQ_ERR_UNSUPPORTED (d != 128, group > 16),
 * TQ_ERR_CAPACITY (workspace), TQ_ERR_HIP. */
size_t tq_attention_prefill_ws_bytes(const tq_ctx *ctx, const tq_kv_cache *cache, int32_t n_q, int32_t q_heads);
tq_status tq_attention_prefill(const tq_ctx *ctx, const tq_kv_cache *cache, const void *d_q, tq_dtype dtype,
                               int32_t n_q, int32_t q_heads, int32_t causal, float scale, float *d_out, void *d_ws,
                               size_t ws_bytes, void *stream);

/* Fused serving step: the same result as tq_append_token(d_k, d_v) followed by
 * tq_attention_decode(d_q) on the same stream (the new token is attended),
 * in three launches instead of five: the query preparation encodes the new
 * token of each stream, decode reads the post-append lengths from the
 * workspace, and the merge launch advances d_seq_len. d_k, d_v: contiguous
 * [batch][kv_heads][d]; d_q: [batch][q_heads][d]; all of `dtype`. Increments
 * cache->host_max_len. The O(1) append requirement is the one stated in the
 * fractal KV-archive summary on gist.science.
 * d_ws: workspace of tq_decode_step_ws_bytes() bytes (not shared with a
 * concurrent call).
 * Errors: TQ_ERR_ARG, TQ_ERR_UNSUPPORTED (d != 128, group > 16),
 * TQ_ERR_CAPACITY (cache full or workspace too small), TQ_ERR_HIP. */
size_t tq_decode_step_ws_bytes(const tq_ctx *ctx, const tq_kv_cache *cache, int32_t q_heads);
tq_status tq_decode_step(const tq_ctx *ctx, tq_kv_cache *cache, const void *d_k, const void *d_v, const void *d_q,
                         tq_dtype dtype, int32_t q_heads, float scale, float *d_out, void *d_ws, size_t ws_bytes,
                         void *stream);

/* Scores of nq queries against n packed keys ([ebisuda] 第2段階; [hakusoku]
 * QJL: full-precision query, low-precision data):
 *   s[q][t] = ||k_t|| (<Pi q, c[idx_t]> + sqrt(pi/2)/m ||r_t|| <S Pi q, 2 sigma_t - 1>).
 * d_q: [nq][d]. If d_scores is non-NULL it receives fp32 [nq][n]. If topk > 0
 * (<= 64), d_top_idx/d_top_val receive [nq][topk] ordered by (-score, index).
 * d_ws: workspace of tq_scores_ws_bytes() bytes.
 * Errors: TQ_ERR_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_CAPACITY (workspace),
 * TQ_ERR_HIP. */
size_t tq_scores_ws_bytes(const tq_ctx *ctx, int64_t nq, int64_t n, int32_t topk, int32_t want_scores);
tq_status tq_scores(const tq_ctx *ctx, const void *d_q, tq_dtype dtype, int64_t nq, const tq_packed *keys,
                    float *d_scores, int32_t topk, int32_t *d_top_idx, float *d_top_val, void *d_ws,
                    size_t ws_bytes, void *stream);

/* PolarQuant encode of n_streams x n_tokens vectors: vector (s, t) is row
 * s*n_tokens + t of d_x (row stride x_stride elements, fp32 or bf16, 16-byte
 * aligned) and goes to record s*out_stream_stride + out_offset + t. d = 128
 * only. d_ws: tq_polar_quantize_ws_bytes(ctx, n_streams * n_tokens) bytes (the
 * rotated rows).
 * Errors: TQ_ERR_ARG (NULL, strides, overlapping or out-of-range records),
 * TQ_ERR_UNSUPPORTED (d, bits), TQ_ERR_CAPACITY (workspace), TQ_ERR_HIP. */
size_t tq_polar_quantize_ws_bytes(const tq_ctx *ctx, int64_t n);
tq_status tq_polar_quantize(const tq_ctx *ctx, const void *d_x, tq_dtype dtype, int64_t n_streams, int64_t n_tokens,
                            int64_t x_stride, const tq_polar_packed *out, int64_t out_stream_stride,
                            int64_t out_offset, void *d_ws, size_t ws_bytes, void *stream);

/* Decode attention with PolarQuant keys: for every sequence b and query head h,
 * out[b][h] = sum_t p_t v_hat_t, p = softmax(scale * s_t) over t < d_seq_len[b],
 * s_t = <q, x_hat_t> from record (b*kv_heads + h/group)*values->capacity + t of
 * `keys` ([gemilab] Attention機構; the scores of tq_polar_scores), v_hat from
 * `values`' stage-1 value records (contiguous layout, fp32 norms; its key
 * array is not read). d_q: [batch][q_heads][128]; d_out fp32 likewise.
 * d_ws: tq_polar_attention_decode_ws_bytes() bytes.
 * Errors: TQ_ERR_ARG, TQ_ERR_UNSUPPORTED (d, group > 16, paged or compact
 * values), TQ_ERR_CAPACITY (workspace), TQ_ERR_HIP. */
size_t tq_polar_attention_decode_ws_bytes(const tq_ctx *ctx, const tq_kv_cache *values, int32_t q_heads);
tq_status tq_polar_attention_decode(const tq_ctx *ctx, const tq_polar_packed *keys, const tq_kv_cache *values,
                                    const void *d_q, tq_dtype dtype, int32_t q_heads, float scale, float *d_out,
                                    void *d_ws, size_t ws_bytes, void *stream);

/* PolarQuant scores: d_scores[q][i] = <Pi q, y_hat_i> = <q, x_hat_i> with y_hat_i
 * rebuilt from record i's codes (top-down: ||x|| times the cos / sin of the
 * ancestors' angle centroids, then the pair's own angle), fp32, [nq][keys->n].
 * d_q: [nq][128] fp32 or bf16. d_ws: tq_polar_scores_ws_bytes() bytes (the
 * rotated queries and the rebuilt rows, 512 bytes per key).
 * Errors: TQ_ERR_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_CAPACITY, TQ_ERR_HIP. */
size_t tq_polar_scores_ws_bytes(const tq_ctx *ctx, int64_t nq, int64_t n);
tq_status tq_polar_scores(const tq_ctx *ctx, const void *d_q, tq_dtype dtype, int64_t nq, const tq_polar_packed *keys,
                          float *d_scores, void *d_ws, size_t ws_bytes, void *stream);

/* Decode logits, a measurement aid: the query preparation and the key phase of
 * tq_attention_decode's own kernels, which write what they would feed the
 * softmax: d_logits[b][h][t] = scale * s_t (natural units, fp32) for t <
 * d_seq_len[b], row stride `capacity` floats ([batch][q_heads][capacity],
 * caller-owned; entries at t >= d_seq_len[b] are not written). s_t is the
 * estimator of tq_attention_decode ([ebisuda] 第2段階; [gemilab] Attention機構),
 * so this measures the accuracy of the decode path's scores directly.
 * Contiguous caches only. d_ws: tq_attention_decode_ws_bytes() bytes.
 * Errors: as tq_attention_decode; TQ_ERR_UNSUPPORTED for a paged cache. */
tq_status tq_decode_logits(const tq_ctx *ctx, const tq_kv_cache *cache, const void *d_q, tq_dtype dtype,
                           int32_t q_heads, float scale, float *d_logits, void *d_ws, size_t ws_bytes, void *stream);

/* Kernel timing, a measurement aid. Arms the calling thread so that its next
 * tq_attention_decode, tq_attention_prefill or tq_decode_step records start_event on its stream
 * right before the score/attention kernel (after the query preparation) and
 * stop_event right after it (before the merge of the chunk partials); that
 * call then disarms the thread. The events are hipEvent_t handles created
 * and owned by the caller (with timing enabled, for hipEventElapsedTime).
 * Both NULL disarms. A call that fails before its launches leaves the thread
 * disarmed. tq_polar_attention_decode takes the events too and records them
 * around its scoring kernel (the PolarQuant tree evaluation).
 * Errors: TQ_ERR_ARG (exactly one of the two is NULL). */
tq_status tq_time_next_decode(void *start_event, void *stop_event);

/* Read-bandwidth probe, a measurement aid: the practical HBM read ceiling that
 * the decode kernel's roofline is read against. `grid` work-groups of 256
 * threads stream `bytes` bytes of d_src (device, 16-byte aligned, bytes a
 * multiple of 16), each work-group its own contiguous slice, with 16-byte
 * non-temporal loads, four in flight per thread, and write one XOR-fold word
 * per thread to d_sink (device, grid * 256 uint32, so the loads are not
 * optimized away; the XOR of all folds is the XOR of all words read).
 * Asynchronous on `stream`.
 * Errors: TQ_ERR_ARG (NULL, alignment, size, grid not in [1, 65536]), TQ_ERR_HIP. */
tq_status tq_read_probe(const void *d_src, size_t bytes, int32_t grid, uint32_t *d_sink, void *stream);

/* Message for the last non-OK status on this thread ("" if none). */
const char *tq_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* TQ_H */
