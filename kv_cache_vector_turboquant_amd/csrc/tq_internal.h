// Internal declarations shared by the host code and the HIP kernels of libtq.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/tq.h"

namespace tq {

// Per bit width (index = bits, 1..4): stored codebook tables in the layout the
// kernels read. walsh[] are the odd Walsh coefficients of the centroid table,
// in the subset order of walsh_subset(bits, i); ctop = centroid[2^bits - 1]
// (the sum of all walsh coefficients).
struct DeviceTables {
  float centroid[TQ_MAX_BITS + 1][16];
  float boundary[TQ_MAX_BITS + 1][16];
  float walsh[TQ_MAX_BITS + 1][8];
  float ctop[TQ_MAX_BITS + 1];
  // PolarQuant angle tables, [level 1..7][bits 1..4]: boundaries (INFINITY past
  // the last), cos and sin of the centroids
  float pbound[8][TQ_MAX_BITS + 1][16];
  float pcos[8][TQ_MAX_BITS + 1][16];
  float psin[8][TQ_MAX_BITS + 1][16];
};

// Where the record of token t of stream s lands in a packed array: contiguous
// s * os + oo + t, or, with a block table (paged cache; s = b * heads + h and
// position T = oo + t), (page * heads + h) * page_tokens + T mod page_tokens
// with page = table[b * cols + T / page_tokens]. A page id outside [0, npages)
// is a caller error; it is clamped so every access stays inside the arrays.
struct RecMap {
  int64_t os = 0, oo = 0;
  const int32_t *table = nullptr;
  int32_t page_tokens = 0, heads = 1, cols = 0, npages = 1;
  __host__ __device__ __forceinline__ int64_t rec(int64_t s, int64_t t) const {
    if (table == nullptr) return s * os + oo + t;
    const int64_t T = oo + t, b = s / heads, h = s - b * heads;
    int pg = table[b * cols + T / page_tokens];
    pg = pg < 0 ? 0 : (pg >= npages ? npages - 1 : pg);
    return ((int64_t)pg * heads + h) * page_tokens + T % page_tokens;
  }
};

// i-th odd-cardinality subset of {0..bits-1} (as a bit mask), ordered by
// (popcount, value); there are 2^(bits-1) of them.
int walsh_subset(int bits, int i);

void set_error(const std::string &msg);
tq_status fail(tq_status s, const std::string &msg);
tq_status hip_fail(hipError_t e, const char *what);

}  // namespace tq

struct tq_ctx {
  int32_t d = 0;
  int device = 0;
  std::vector<float> rot;     // host fp32 Pi, row-major d x d
  std::vector<float> sketch;  // host fp32 S, row-major d x d
  tq_codebook cb[TQ_MAX_BITS + 1];
  float *d_rot = nullptr;
  float *d_sketch = nullptr;
  float *d_rot_t = nullptr;     // Pi^T, row-major (coalesced matrix-vector products)
  float *d_sketch_t = nullptr;  // S^T, row-major
  float *d_rs_t = nullptr;      // [Pi ; S Pi]^T: d x 2d row-major (query rotation and sketch in one pass)
  uint16_t *d_rot3 = nullptr;   // d = 128: Pi as three bf16 parts (hi, mid, lo), [3][d][d]
  uint16_t *d_sk2 = nullptr;    // d = 128: S as two bf16 parts (hi, lo), [2][d][d]
  tq::DeviceTables *d_tables = nullptr;
  tq::DeviceTables h_tables;
};

namespace tq {
// Kernel launchers (tq_kernels.hip). All return hipSuccess or the launch error.
hipError_t launch_quantize_keys(const tq_ctx *ctx, const void *x, int is_bf16, int64_t n_streams, int64_t n_tokens,
                                int64_t xs, int64_t xt, const tq_packed *out, const RecMap &map, float *work,
                                hipStream_t st);
hipError_t launch_quantize_values(const tq_ctx *ctx, const void *x, int is_bf16, int64_t n_streams,
                                  int64_t n_tokens, int64_t xs, int64_t xt, const tq_packed *out, const RecMap &map,
                                  hipStream_t st);
// The record map of a cache (contiguous or paged) for positions starting at oo.
RecMap cache_map(const tq_kv_cache *cache, int64_t oo);
hipError_t launch_append(const tq_ctx *ctx, const tq_kv_cache *cache, const void *k, const void *v, int is_bf16,
                         hipStream_t st);
size_t decode_ws_bytes(const tq_ctx *ctx, const tq_kv_cache *cache, int32_t q_heads, int *chunk_out,
                       int *nchunks_out, int n_q = 1);
// n_q query positions per sequence (q: [batch][n_q][q_heads][d], out likewise);
// causal: position i attends to t < seq_len - n_q + i + 1.
// With k_new / v_new non-NULL (fused step) the new token of every stream is
// appended first and the sequence lengths advance by one. Non-NULL ev0 / ev1 are
// recorded on st right before / after the score/attention kernel.
// With ext non-NULL the logits (log2 units, [stream*hgroups][4][ext_stride]) are
// given: keys in another format, scored beforehand; q is unused and only the
// cache's values and lengths are read (contiguous layout, fp32 norms).
// With logits non-NULL (measurement, contiguous caches) only the query
// preparation and the key phase run: logits[b][i][h][t] = scale * s_t for the
// visible tokens (row stride = capacity), and out is not written.
hipError_t launch_decode(const tq_ctx *ctx, const tq_kv_cache *cache, const void *q, int is_bf16, int32_t q_heads,
                         float scale, float *out, void *ws, hipStream_t st, const void *k_new = nullptr,
                         const void *v_new = nullptr, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr,
                         int n_q = 1, int causal = 0, const float *ext = nullptr, int64_t ext_stride = 0,
                         float *logits = nullptr);
// Log-sum-exp merge of per-chunk attention partials ([stream][n_q * group][nchunks][d + 2]:
// rotated output, max logit in log2 units, weight sum) and o = Pi^T o_rot into
// out [batch][n_q][q_heads][d].
hipError_t launch_merge_partials(const tq_ctx *ctx, const tq_kv_cache *cache, int32_t q_heads, int n_q,
                                 float *partial, int nchunks, float *out, hipStream_t st);
// Prefill attention with sixteen virtual heads per work-group (prefill_kernels.hip):
// contiguous caches, d = 128, value bits <= 3 and n_q * group >= 16.
bool prefill_supported(const tq_ctx *ctx, const tq_kv_cache *cache, int32_t q_heads, int n_q);
size_t prefill_ws_bytes(const tq_kv_cache *cache, int32_t q_heads, int n_q);
hipError_t launch_prefill(const tq_ctx *ctx, const tq_kv_cache *cache, const void *q, int is_bf16, int32_t q_heads,
                          int n_q, int causal, float scale, float *out, void *ws, hipStream_t st, hipEvent_t ev0,
                          hipEvent_t ev1);
hipError_t launch_read_probe(const void *src, size_t bytes, int grid, uint32_t *sink, hipStream_t st);
// C[M][N] = A[M][K] B[N][K]^T on fp32 MFMA (A fp32 or bf16, B fp32; row strides in elements)
hipError_t launch_gemm_store(const void *a, int a_bf16, int64_t lda, int64_t M, const float *b, int64_t ldb,
                             int64_t N, int K, float *c, int64_t ldc, hipStream_t st);
// PolarQuant keys (polar_kernels.hip), d = 128: y = Pi x of n_streams * n_tokens
// vectors (rows of x, stride xs, stream-major) into records
// s * out_stream_stride + out_offset + t of `out`; ws: rows * 128 floats.
hipError_t launch_polar_quantize(const tq_ctx *ctx, const void *x, int is_bf16, int64_t n_streams, int64_t n_tokens,
                                 int64_t xs, const tq_polar_packed *out, int64_t out_stream_stride, int64_t out_offset,
                                 void *ws, hipStream_t st);
// scores [nq][keys->n] = <Pi q, y_hat>; ws: (nq + keys->n) * 128 floats (256-aligned parts)
hipError_t launch_polar_scores(const tq_ctx *ctx, const void *q, int is_bf16, int64_t nq, const tq_polar_packed *keys,
                               float *scores, void *ws, hipStream_t st);
// decode attention with PolarQuant keys (records of stream s at s * capacity + t)
// and the cache's stage-1 values; ws: polar_attention_ws_bytes()
size_t polar_attention_ws_bytes(const tq_ctx *ctx, const tq_kv_cache *values, int32_t q_heads);
hipError_t launch_polar_attention(const tq_ctx *ctx, const tq_polar_packed *keys, const tq_kv_cache *values,
                                  const void *q, int is_bf16, int32_t q_heads, float scale, float *out, void *ws,
                                  hipStream_t st, hipEvent_t ev0, hipEvent_t ev1);
size_t scores_ws_bytes(const tq_ctx *ctx, int64_t nq, int64_t n, int32_t topk, int32_t want_scores);
// The library-held scratch array (TQ_SCRATCH_BYTES per device): scratch_init
// looks up its device address once per device (that device current);
// scratch_ptr returns it (NULL before scratch_init on that device).
hipError_t scratch_init(int device);
void *scratch_ptr(int device);
hipError_t launch_scores(const tq_ctx *ctx, const void *q, int is_bf16, int64_t nq, const tq_packed *keys,
                         float *scores, int32_t topk, int32_t *top_idx, float *top_val, void *ws, hipStream_t st);
}  // namespace tq
