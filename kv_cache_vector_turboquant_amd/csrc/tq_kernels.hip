// HIP kernels of libtq for CDNA4 (gfx950), wave64.
//
// Pages cited by title and section:
//  [ebisuda] "TurboQuant: Google's 6x KV Cache Compression Algorithm Gains
//            Open-Source Momentum", sections 第1段階 (rotation, Lloyd-Max,
//            no per-block constants) and 第2段階 (1-bit QJL residual).
//  [hakusoku] "TurboQuant: 極限圧縮によるAI効率の再定義", section QJL (sign
//            bits, full-precision query against low-precision data).
//  [gemilab] TurboQuant technical deep dive, sections Attention機構 (softmax
//            attention over cached K/V) and GPU Kernel 最適化 (transform and
//            projection kernels, memory layout; prior art for other hardware).
//
// Kernels
//  gemm_kernel<MODE>   fp32-MFMA (32x32x2) tiled GEMM C = A B^T with fused
//                      epilogues: key codes + residual, key QJL signs, value
//                      codes (token-major), plain store, and packed-key scores.
//  decode_prep_kernel  rotates/sketches the decode queries and splits them into
//                      exact int8 digits laid out as MFMA A fragments.
//  decode_kernel       split-K decode attention over packed K/V: scores and
//                      value sums run on int8 MFMA over 0/1 bit masks.
//  decode_merge_kernel log-sum-exp merge of the chunks and inverse rotation.
//  append_kernel       quantizes one K and one V vector per stream in place.
//  topk_kernel         per-query top-k by (-score, index).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cfloat>
#include <climits>
#include <cmath>

#include "tq_internal.h"

namespace tq {

typedef float f16v __attribute__((ext_vector_type(16)));
typedef int i4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16f(uint32_t b16) { return __uint_as_float(b16 << 16); }

// ---------------------------------------------------------------------------
// GEMM: C[M][N] = A[M][K] . B[N][K]^T, fp32 MFMA, 64x128 tiles, BK = 16.
// ---------------------------------------------------------------------------

constexpr int GBM = 64, GBN = 128, GBK = 16, GLD = 20;  // LDS row stride (floats), conflict-free float4 reads

enum { MODE_KEY_CODES = 0, MODE_KEY_SIGNS = 1, MODE_VAL_CODES = 2, MODE_STORE = 3, MODE_SCORES = 4 };

struct DenseSrc {
  const void *base;    // row 0 of this stream
  int64_t row_stride;  // elements
  int64_t nrows;       // rows >= nrows read as zero
  int is_bf16;
};

struct GemmArgs {
  DenseSrc a, b;
  int K;                 // contraction length (multiple of 16)
  int64_t M, N;          // logical sizes (per stream)
  int64_t a_stream_stride, b_stream_stride;  // elements between streams (0 = shared)
  // quantize epilogues
  const DeviceTables *tables;
  int bits, d;
  uint32_t *bits_out;
  float *norms_out;
  float *resid;          // keys: residual rows [stream*n_tokens + t][d]
  int64_t n_tokens;
  int64_t out_stream_stride, out_offset;
  // store / scores epilogues
  float *c;
  int64_t ldc;
  // scores B loader (packed keys)
  const uint32_t *kbits;
  const float *knorm;
  float qjl_scale;       // sqrt(pi/2)/m
  int rows_on_x;         // 1: blockIdx.x indexes row tiles (y: column tiles); 0: the reverse
};

template <int ROWS>
__device__ __forceinline__ void load_dense(const DenseSrc &s, int64_t row0, int k0, int tid, float4 (&v)[ROWS / 64],
                                           float (&ss)[ROWS / 64]) {
#pragma unroll
  for (int g = 0; g < ROWS / 64; ++g) {
    const int r = (tid >> 2) + 64 * g;
    const int kk = (tid & 3) * 4;
    const int64_t row = row0 + r;
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row < s.nrows) {
      if (s.is_bf16) {
        const uint2 u = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(s.base) +
                                                         row * s.row_stride + k0 + kk);
        x = make_float4(bf16f(u.x & 0xFFFFu), bf16f(u.x >> 16), bf16f(u.y & 0xFFFFu), bf16f(u.y >> 16));
      } else {
        x = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(s.base) + row * s.row_stride + k0 + kk);
      }
    }
    v[g] = x;
    ss[g] += x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w;
  }
}

// B tile for packed-key scores: row = key t, columns k0..k0+15 of
// [c[idx_t] (d values) | qjl_scale * rho_t * (2 sigma_t - 1) (d values)].
__device__ __forceinline__ void load_keys(const GemmArgs &g, const float *cent, int64_t row0, int k0, int tid,
                                          float4 (&v)[2]) {
  const int W = g.d >> 5, B = g.bits;
#pragma unroll
  for (int gg = 0; gg < 2; ++gg) {
    const int r = (tid >> 2) + 64 * gg;
    const int k = k0 + (tid & 3) * 4;
    const int64_t t = row0 + r;
    float e[4] = {0.f, 0.f, 0.f, 0.f};
    if (t < g.b.nrows) {
      const uint32_t *rec = g.kbits + t * (int64_t)(W * (B + 1));
      if (k < g.d) {
        const int w = k >> 5, o = k & 31;
        int idx[4] = {0, 0, 0, 0};
        for (int p = 0; p < B; ++p) {
          const uint32_t word = rec[w * (B + 1) + p] >> o;
#pragma unroll
          for (int q = 0; q < 4; ++q) idx[q] |= ((word >> q) & 1u) << p;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) e[q] = cent[idx[q]];
      } else {
        const int i = k - g.d, w = i >> 5, o = i & 31;
        const uint32_t word = rec[w * (B + 1) + B] >> o;
        const float a = g.qjl_scale * g.knorm[2 * t + 1];
#pragma unroll
        for (int q = 0; q < 4; ++q) e[q] = ((word >> q) & 1u) ? a : -a;
      }
    }
    v[gg] = make_float4(e[0], e[1], e[2], e[3]);
  }
}

__device__ __forceinline__ int quant_index(float y, const float *bnd, int L) {
  int idx = 0;
  for (int i = 0; i < L - 1; ++i) idx += (y >= bnd[i]) ? 1 : 0;
  return idx;
}

template <int MODE>
__global__ void __launch_bounds__(256) gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) float As[2][GBM * GLD];
  __shared__ __attribute__((aligned(16))) float Bs[2][GBN * GLD];
  __shared__ float stat[GBN];
  __shared__ float cent[16], bnd[16];
  __shared__ uint32_t cw[GBM * (GBN / 32) * 4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1, li = lane & 31, lh = lane >> 5;
  const int64_t s = blockIdx.z;
  const int64_t rt = g.rows_on_x ? blockIdx.x : blockIdx.y, ct = g.rows_on_x ? blockIdx.y : blockIdx.x;
  const int64_t row0 = rt * GBM, col0 = ct * GBN;
  const int L = 1 << g.bits;

  if (MODE == MODE_KEY_CODES || MODE == MODE_VAL_CODES || MODE == MODE_SCORES) {
    if (tid < 16) {
      cent[tid] = g.tables->centroid[g.bits][tid];
      bnd[tid] = g.tables->boundary[g.bits][tid];
    }
    __syncthreads();
  }

  DenseSrc sa = g.a, sb = g.b;
  if (sa.is_bf16) sa.base = (const uint16_t *)sa.base + s * g.a_stream_stride;
  else sa.base = (const float *)sa.base + s * g.a_stream_stride;
  if (sb.is_bf16) sb.base = (const uint16_t *)sb.base + s * g.b_stream_stride;
  else sb.base = (const float *)sb.base + s * g.b_stream_stride;

  float4 ra[1], rb[2];
  float ssa[1] = {0.f}, ssb[2] = {0.f, 0.f};
  auto load_tile = [&](int k0) {
    load_dense<GBM>(sa, row0, k0, tid, ra, ssa);
    if constexpr (MODE == MODE_SCORES) load_keys(g, cent, col0, k0, tid, rb);
    else load_dense<GBN>(sb, col0, k0, tid, rb, ssb);
  };
  auto store_tile = [&](int buf) {
    const int r = tid >> 2, kk = (tid & 3) * 4;
    *reinterpret_cast<float4 *>(&As[buf][r * GLD + kk]) = ra[0];
    *reinterpret_cast<float4 *>(&Bs[buf][r * GLD + kk]) = rb[0];
    *reinterpret_cast<float4 *>(&Bs[buf][(r + 64) * GLD + kk]) = rb[1];
  };

  f16v acc[2];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[b][r] = 0.f;

  const int KT = g.K / GBK;
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load_tile((kt + 1) * GBK);
    const float *ap = &As[cur][(wm * 32 + li) * GLD + lh * 8];
    const float4 a0 = *reinterpret_cast<const float4 *>(ap), a1 = *reinterpret_cast<const float4 *>(ap + 4);
    const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const float *bp = &Bs[cur][(wn * 64 + b * 32 + li) * GLD + lh * 8];
      const float4 b0 = *reinterpret_cast<const float4 *>(bp), b1 = *reinterpret_cast<const float4 *>(bp + 4);
      const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
      for (int st = 0; st < 8; ++st) acc[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[st], bv[st], acc[b], 0, 0, 0);
    }
    if (kt + 1 < KT) store_tile(cur ^ 1);
    __syncthreads();
  }

  // Row (A) / column (B) sums of squares gathered over the K loop: the 4
  // loader threads of a row are adjacent lanes.
  if constexpr (MODE == MODE_KEY_CODES || MODE == MODE_KEY_SIGNS) {
    float v = ssa[0];
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    if ((tid & 3) == 0) stat[tid >> 2] = v;
  }
  if constexpr (MODE == MODE_VAL_CODES) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      float v = ssb[q];
      v += __shfl_xor(v, 1);
      v += __shfl_xor(v, 2);
      if ((tid & 3) == 0) stat[(tid >> 2) + 64 * q] = v;
    }
  }
  __syncthreads();

  const int B = g.bits;
  if constexpr (MODE == MODE_STORE || MODE == MODE_SCORES) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t col = col0 + wn * 64 + b * 32 + li;
      float scale = 1.f;
      if constexpr (MODE == MODE_SCORES) scale = (col < g.N) ? g.knorm[2 * col] : 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = row0 + wm * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
        if (row < g.M && col < g.N) g.c[row * g.ldc + col] = acc[b][r] * scale;
      }
    }
  } else if constexpr (MODE == MODE_KEY_CODES || MODE == MODE_KEY_SIGNS) {
    // rows = tokens of stream s, columns = coordinates (codes) or sketch rows (signs)
    const int W = g.d >> 5;
    const int64_t rec_base = s * g.out_stream_stride + g.out_offset;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t col = col0 + wn * 64 + b * 32 + li;
      const int wl = (wn * 64 + b * 32) >> 5;  // local 32-column group
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rl = wm * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
        const int64_t t = row0 + rl;
        const bool in = t < g.n_tokens && col < g.d;
        bool live;
        uint32_t mybits = 0;
        if constexpr (MODE == MODE_KEY_CODES) {
          const float nrm = sqrtf(stat[rl]);
          live = in && nrm > 0.f;
          const float y = live ? acc[b][r] / nrm : 0.f;
          const int idx = quant_index(y, bnd, L);
          if (in) g.resid[(s * g.n_tokens + t) * (int64_t)g.d + col] = live ? y - cent[idx] : 0.f;
          mybits = live ? (uint32_t)idx : 0u;
        } else {
          live = in && g.norms_out[2 * (rec_base + t)] > 0.f;
          mybits = (live && acc[b][r] >= 0.f) ? 1u : 0u;
        }
        const int np = (MODE == MODE_KEY_CODES) ? B : 1;
        for (int p = 0; p < np; ++p) {
          const uint64_t bal = __builtin_amdgcn_ballot_w64(((mybits >> p) & 1u) != 0u);
          if (li == 0) {
            const int rr = wm * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
            cw[(rr * (GBN / 32) + wl) * 4 + p] = lh ? (uint32_t)(bal >> 32) : (uint32_t)bal;
          }
        }
      }
    }
    __syncthreads();
    {
      const int rl = tid >> 2, gl = tid & 3;
      const int64_t t = row0 + rl;
      const int w = (int)(col0 >> 5) + gl;
      if (t < g.n_tokens && w < W) {
        uint32_t *dst = g.bits_out + ((rec_base + t) * W + w) * (int64_t)(B + 1);
        if constexpr (MODE == MODE_KEY_CODES) {
          for (int p = 0; p < B; ++p) dst[p] = cw[(rl * (GBN / 32) + gl) * 4 + p];
        } else {
          dst[B] = cw[(rl * (GBN / 32) + gl) * 4];
        }
      }
      if (ct == 0 && gl == 0 && t < g.n_tokens) {
        if constexpr (MODE == MODE_KEY_CODES) g.norms_out[2 * (rec_base + t)] = sqrtf(stat[rl]);
        else g.norms_out[2 * (rec_base + t) + 1] = sqrtf(stat[rl]);
      }
    }
  } else if constexpr (MODE == MODE_VAL_CODES) {
    // rows = coordinates, columns = tokens of stream s; ballots are token-major words.
    const int64_t rec_base = s * g.out_stream_stride + g.out_offset;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int cl = wn * 64 + b * 32 + li;
      const int64_t t = col0 + cl;
      const int64_t blk_t0 = col0 + wn * 64 + b * 32;  // first token of this 32-token block
      const float nrm = sqrtf(stat[cl]);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t j = row0 + wm * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
        const bool live = t < g.n_tokens && nrm > 0.f && j < g.d;
        const float y = live ? acc[b][r] / nrm : 0.f;
        const uint32_t idx = live ? (uint32_t)quant_index(y, bnd, L) : 0u;
        for (int p = 0; p < B; ++p) {
          const uint64_t bal = __builtin_amdgcn_ballot_w64(((idx >> p) & 1u) != 0u);
          if (li == 0 && blk_t0 < g.n_tokens && j < g.d) {
            const int64_t blk = (rec_base + blk_t0) >> 5;
            g.bits_out[(blk * g.d + j) * B + p] = lh ? (uint32_t)(bal >> 32) : (uint32_t)bal;
          }
        }
      }
    }
    if (rt == 0 && (tid & 3) == 0) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int cl = (tid >> 2) + 64 * q;
        const int64_t t = col0 + cl;
        if (t < g.n_tokens) g.norms_out[rec_base + t] = sqrtf(stat[cl]);
      }
    }
  }
}

hipError_t launch_quantize_keys(const tq_ctx *ctx, const void *x, int is_bf16, int64_t n_streams, int64_t n_tokens,
                                int64_t xs, int64_t xt, const tq_packed *out, int64_t os, int64_t oo, float *work,
                                hipStream_t st) {
  const int d = ctx->d;
  GemmArgs g = {};
  g.a = {x, xt, n_tokens, is_bf16};
  g.a_stream_stride = xs;
  g.b = {ctx->d_rot, d, d, 0};
  g.b_stream_stride = 0;
  g.K = d;
  g.M = n_tokens;
  g.N = d;
  g.tables = ctx->d_tables;
  g.bits = out->mse_bits;
  g.d = d;
  g.bits_out = out->bits;
  g.norms_out = out->norms;
  g.resid = work;
  g.n_tokens = n_tokens;
  g.out_stream_stride = os;
  g.out_offset = oo;
  g.rows_on_x = 1;
  dim3 grid((unsigned)((n_tokens + GBM - 1) / GBM), (d + GBN - 1) / GBN, (unsigned)n_streams);
  hipLaunchKernelGGL(gemm_kernel<MODE_KEY_CODES>, grid, dim3(256), 0, st, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // stage 2: z = S r on the residual rows, sign bits and ||r||
  GemmArgs g2 = g;
  g2.a = {work, d, n_tokens, 0};
  g2.a_stream_stride = n_tokens * (int64_t)d;
  g2.b = {ctx->d_sketch, d, d, 0};
  hipLaunchKernelGGL(gemm_kernel<MODE_KEY_SIGNS>, grid, dim3(256), 0, st, g2);
  return hipGetLastError();
}

hipError_t launch_quantize_values(const tq_ctx *ctx, const void *x, int is_bf16, int64_t n_streams,
                                  int64_t n_tokens, int64_t xs, int64_t xt, const tq_packed *out, int64_t os,
                                  int64_t oo, hipStream_t st) {
  const int d = ctx->d;
  GemmArgs g = {};
  g.a = {ctx->d_rot, d, d, 0};
  g.a_stream_stride = 0;
  g.b = {x, xt, n_tokens, is_bf16};
  g.b_stream_stride = xs;
  g.K = d;
  g.M = d;
  g.N = n_tokens;
  g.tables = ctx->d_tables;
  g.bits = out->mse_bits;
  g.d = d;
  g.bits_out = out->bits;
  g.norms_out = out->norms;
  g.n_tokens = n_tokens;
  g.out_stream_stride = os;
  g.out_offset = oo;
  dim3 grid((unsigned)((n_tokens + GBN - 1) / GBN), (d + GBM - 1) / GBM, (unsigned)n_streams);
  hipLaunchKernelGGL(gemm_kernel<MODE_VAL_CODES>, grid, dim3(256), 0, st, g);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Top-k per query row by (-score, index).
// ---------------------------------------------------------------------------

__device__ __forceinline__ bool better(float v1, int i1, float v2, int i2) { return v1 > v2 || (v1 == v2 && i1 < i2); }

template <int KS, int BS>
__global__ void __launch_bounds__(BS) topk_kernel(const float *scores, int64_t n, int topk, int32_t *out_idx,
                                                  float *out_val) {
  __shared__ float cv[BS * KS];
  __shared__ int ci[BS * KS];
  __shared__ float rv[BS];
  __shared__ int ri[BS], rt[BS];
  const int tid = threadIdx.x;
  const int64_t q = blockIdx.x;
  const float *row = scores + q * n;
  float v[KS];
  int ix[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    v[s] = -INFINITY;
    ix[s] = INT_MAX;
  }
  for (int64_t i = tid; i < n; i += BS) {
    const float x = row[i];
    const int xi = (int)i;
    if (!better(x, xi, v[KS - 1], ix[KS - 1])) continue;
    // insertion into the sorted list (descending)
    bool placed = false;
#pragma unroll
    for (int s = KS - 1; s > 0; --s) {
      if (!placed) {
        if (better(x, xi, v[s - 1], ix[s - 1])) {
          v[s] = v[s - 1];
          ix[s] = ix[s - 1];
        } else {
          v[s] = x;
          ix[s] = xi;
          placed = true;
        }
      }
    }
    if (!placed) {
      v[0] = x;
      ix[0] = xi;
    }
  }
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    cv[tid * KS + s] = v[s];
    ci[tid * KS + s] = ix[s];
  }
  __syncthreads();
  int head = 0;  // next unused candidate of this thread
  for (int k = 0; k < topk; ++k) {
    rv[tid] = head < KS ? cv[tid * KS + head] : -INFINITY;
    ri[tid] = head < KS ? ci[tid * KS + head] : INT_MAX;
    rt[tid] = tid;
    __syncthreads();
    for (int off = BS / 2; off > 0; off >>= 1) {
      if (tid < off && better(rv[tid + off], ri[tid + off], rv[tid], ri[tid])) {
        rv[tid] = rv[tid + off];
        ri[tid] = ri[tid + off];
        rt[tid] = rt[tid + off];
      }
      __syncthreads();
    }
    if (tid == 0) {
      out_val[q * topk + k] = rv[0];
      out_idx[q * topk + k] = ri[0];
    }
    const int winner = rt[0];
    __syncthreads();
    if (tid == winner) ++head;
  }
}

size_t scores_ws_bytes(const tq_ctx *ctx, int64_t nq, int64_t n, int32_t topk, int32_t want_scores) {
  size_t b = (size_t)nq * 2 * ctx->d * sizeof(float);  // [q_rot | q_s]
  b = (b + 255) & ~(size_t)255;
  if (topk > 0 && !want_scores) b += (size_t)nq * (size_t)n * sizeof(float);
  return b;
}

hipError_t launch_scores(const tq_ctx *ctx, const void *q, int is_bf16, int64_t nq, const tq_packed *keys,
                         float *scores, int32_t topk, int32_t *top_idx, float *top_val, void *ws, hipStream_t st) {
  const int d = ctx->d;
  float *qa = (float *)ws;  // [nq][2d]
  size_t off = ((size_t)nq * 2 * d * sizeof(float) + 255) & ~(size_t)255;
  float *sc = scores ? scores : (float *)((char *)ws + off);
  // q_rot = Pi q  -> columns [0, d)
  GemmArgs g = {};
  g.a = {q, d, nq, is_bf16};
  g.b = {ctx->d_rot, d, d, 0};
  g.K = d;
  g.M = nq;
  g.N = d;
  g.c = qa;
  g.ldc = 2 * d;
  g.rows_on_x = 1;
  dim3 grid1((unsigned)((nq + GBM - 1) / GBM), (d + GBN - 1) / GBN, 1);
  hipLaunchKernelGGL(gemm_kernel<MODE_STORE>, grid1, dim3(256), 0, st, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // q_s = S q_rot -> columns [d, 2d)
  GemmArgs g2 = g;
  g2.a = {qa, 2 * d, nq, 0};
  g2.b = {ctx->d_sketch, d, d, 0};
  g2.c = qa + d;
  hipLaunchKernelGGL(gemm_kernel<MODE_STORE>, grid1, dim3(256), 0, st, g2);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // scores = n_t * ([q_rot | q_s] . [c[idx_t] | qjl * rho_t * (2 sigma_t - 1)])
  GemmArgs g3 = {};
  g3.a = {qa, 2 * d, nq, 0};
  g3.b = {nullptr, 0, keys->n, 0};
  g3.K = 2 * d;
  g3.M = nq;
  g3.N = keys->n;
  g3.tables = ctx->d_tables;
  g3.bits = keys->mse_bits;
  g3.d = d;
  g3.kbits = keys->bits;
  g3.knorm = keys->norms;
  g3.qjl_scale = (float)(std::sqrt(M_PI / 2.0) / d);
  g3.c = sc;
  g3.ldc = keys->n;
  dim3 grid3((unsigned)((keys->n + GBN - 1) / GBN), (unsigned)((nq + GBM - 1) / GBM), 1);
  hipLaunchKernelGGL(gemm_kernel<MODE_SCORES>, grid3, dim3(256), 0, st, g3);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (topk > 0) {
    if (topk <= 16)
      hipLaunchKernelGGL((topk_kernel<16, 256>), dim3((unsigned)nq), dim3(256), 0, st, sc, keys->n, topk, top_idx, top_val);
    else
      hipLaunchKernelGGL((topk_kernel<64, 64>), dim3((unsigned)nq), dim3(64), 0, st, sc, keys->n, topk, top_idx, top_val);
    e = hipGetLastError();
  }
  return e;
}

// ---------------------------------------------------------------------------
// Decode attention (d = 128).
//
// Scores and value sums are linear in 0/1 masks of the packed bit-planes. The
// centroid table is antisymmetric (c[L-1-i] = -c[i]), so with s_p = 2 b_p - 1
// it expands over odd Walsh functions: c[idx] = sum_S w_S prod_{p in S} s_p,
// and prod_{p in S} s_p = 2 (XOR of planes in S) - 1. Hence
//   sum_j q_j c[idx_j] = sum_S w_S (2 M_S - sum_j q_j),  M_S = sum_j q_j mask_S,j.
// The query (and, for values, the softmax weight) is split into exact signed
// int8 digits (fixed point, 3 digits = 23-24 bits), the masks are 0/1 bytes
// made from a plane word w as (w >> q) & 0x01010101, and every masked sum is an
// exact int32 from v_mfma_i32_16x16x64_i8. A fragment row = 4*head + digit.
// ---------------------------------------------------------------------------

constexpr int DD = 128;          // head dim
constexpr int DW = DD / 32;      // 32-coordinate groups
constexpr float QMAX = 8323072.f;  // |fixed-point query| bound with 3 signed digits
constexpr float WSCALE = 4194304.f;  // 2^22: fixed point of the value weights

struct DecodeArgs {
  const uint32_t *kbits;
  const float *knorm;
  const uint32_t *vbits;
  const float *vnorm;
  const int32_t *seq_len;
  int kbitsB, vbitsB;    // MSE bits of keys / values
  int kv_heads, capacity, q_heads, group, hgroups;
  int chunk, nchunks;
  float scale_log2;      // softmax scale * log2(e)
  float qjl_scale;
  const DeviceTables *tables;
  const void *q;
  int q_bf16;
  const float *rot, *sketch;
  int8_t *qfrag;         // [stream*hgroups][2][2][64][16]
  float *qconst;         // [stream*hgroups][4][4]: scale_r, scale_s, Qsum (int bits), Qssum (int bits)
  float *partial;        // [batch*q_heads][nchunks][DD + 2]
  float *out;
};

__device__ __forceinline__ int8_t sdigit(int v) { return (int8_t)(((v & 0xFF) ^ 0x80) - 0x80); }

// One block per (stream, head group): q_rot = Pi q, q_s = S q_rot for up to 4
// heads, fixed-point split and A-fragment layout.
__global__ void __launch_bounds__(256) decode_prep_kernel(DecodeArgs a) {
  __shared__ float qf[4][DD], qr[4][DD], qs[4][DD];
  __shared__ int qi[2][4][DD];
  __shared__ float mx[2][4];
  const int tid = threadIdx.x;
  const int sg = blockIdx.x;  // stream * hgroups + hg
  const int hg = sg % a.hgroups, stream = sg / a.hgroups;
  const int b = stream / a.kv_heads, kvh = stream % a.kv_heads;
  const int h0 = kvh * a.group + hg * 4;
  const int nh = min(4, a.group - hg * 4);
  for (int e = tid; e < 4 * DD; e += 256) {
    const int hh = e / DD, j = e % DD;
    float v = 0.f;
    if (hh < nh) {
      const int64_t off = ((int64_t)b * a.q_heads + h0 + hh) * DD + j;
      v = a.q_bf16 ? bf16f(((const uint16_t *)a.q)[off]) : ((const float *)a.q)[off];
    }
    qf[hh][j] = v;
  }
  __syncthreads();
  for (int e = tid; e < 4 * DD; e += 256) {
    const int hh = e / DD, j = e % DD;
    float acc = 0.f;
    for (int k = 0; k < DD; ++k) acc += a.rot[j * DD + k] * qf[hh][k];
    qr[hh][j] = acc;
  }
  __syncthreads();
  for (int e = tid; e < 4 * DD; e += 256) {
    const int hh = e / DD, i = e % DD;
    float acc = 0.f;
    for (int k = 0; k < DD; ++k) acc += a.sketch[i * DD + k] * qr[hh][k];
    qs[hh][i] = acc;
  }
  __syncthreads();
  if (tid < 8) {
    const int T = tid >> 2, hh = tid & 3;
    float m = 0.f;
    for (int j = 0; j < DD; ++j) m = fmaxf(m, fabsf(T ? qs[hh][j] : qr[hh][j]));
    mx[T][hh] = m;
  }
  __syncthreads();
  for (int e = tid; e < 2 * 4 * DD; e += 256) {
    const int T = e / (4 * DD), hh = (e / DD) & 3, j = e % DD;
    const float m = mx[T][hh];
    const float v = T ? qs[hh][j] : qr[hh][j];
    qi[T][hh][j] = m > 0.f ? (int)rintf(v * (QMAX / m)) : 0;
  }
  __syncthreads();
  if (tid < 8) {
    const int T = tid >> 2, hh = tid & 3;
    int sum = 0;
    for (int j = 0; j < DD; ++j) sum += qi[T][hh][j];
    float *qc = a.qconst + ((int64_t)sg * 4 + hh) * 4;
    const float m = mx[T][hh];
    qc[T] = m > 0.f ? m / QMAX : 0.f;
    qc[2 + T] = __int_as_float(sum);
  }
  {
    // fragment (T, instr, lane): 16 digits of row (4*hh + dig), k-slot 4q'+b <-> coordinate 32g + 4i + q' + 8b
    const int T = tid >> 7, ins = (tid >> 6) & 1, L = tid & 63;
    const int g = L >> 4, row = L & 15, hh = row >> 2, dig = row & 3;
    uint32_t wv[4];
    for (int qq = 0; qq < 4; ++qq) {
      uint32_t w = 0;
      for (int bb = 0; bb < 4; ++bb) {
        const int j = 32 * g + 4 * ins + qq + 8 * bb;
        int v = qi[T][hh][j];
        int d0 = sdigit(v);
        int v1 = (v - d0) >> 8;
        int d1 = sdigit(v1);
        int d2 = (v1 - d1) >> 8;
        const int dv = dig == 0 ? d0 : dig == 1 ? d1 : dig == 2 ? d2 : 0;
        w |= ((uint32_t)(dv & 0xFF)) << (8 * bb);
      }
      wv[qq] = w;
    }
    uint4 *dst = reinterpret_cast<uint4 *>(a.qfrag + ((((int64_t)sg * 2 + T) * 2 + ins) * 64 + L) * 16);
    *dst = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  }
}

__device__ __forceinline__ void mask_bytes(uint32_t m, i4v &lo, i4v &hi) {
  lo[0] = (int)(m & 0x01010101u);
  lo[1] = (int)((m >> 1) & 0x01010101u);
  lo[2] = (int)((m >> 2) & 0x01010101u);
  lo[3] = (int)((m >> 3) & 0x01010101u);
  hi[0] = (int)((m >> 4) & 0x01010101u);
  hi[1] = (int)((m >> 5) & 0x01010101u);
  hi[2] = (int)((m >> 6) & 0x01010101u);
  hi[3] = (int)((m >> 7) & 0x01010101u);
}

__device__ __forceinline__ uint32_t xor_planes(const uint32_t *pl, int S) {
  uint32_t m = 0;
#pragma unroll
  for (int p = 0; p < 4; ++p)
    if (S & (1 << p)) m ^= pl[p];
  return m;
}

__device__ __forceinline__ int combine_digits(const i4v &acc) { return acc[0] + (acc[1] << 8) + (acc[2] << 16); }

template <int KB, int VB>
__global__ void __launch_bounds__(256) decode_kernel(DecodeArgs a) {
  constexpr int KM = 1 << (KB - 1);  // key Walsh masks
  constexpr int VM = 1 << (VB - 1);  // value Walsh masks
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float *lg = reinterpret_cast<float *>(smem);                         // [4][chunk]
  int8_t *av = reinterpret_cast<int8_t *>(smem + 4 * a.chunk * 4);     // [chunk/128][2][64][16]
  __shared__ float red[4][4];
  __shared__ double wsum[4];
  __shared__ float hmax[4], hsum[4], vmaxs;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x;
  const int sg = blockIdx.y;
  const int hg = sg % a.hgroups, stream = sg / a.hgroups;
  const int b = stream / a.kv_heads;
  const int nh = min(4, a.group - hg * 4);
  const int len = a.seq_len[b];
  const int t0 = c * a.chunk;
  const int t1 = min(len, t0 + a.chunk);
  const int h0 = (stream % a.kv_heads) * a.group + hg * 4;
  float *part_base = a.partial;
  auto part = [&](int hh) { return part_base + (((int64_t)b * a.q_heads + h0 + hh) * a.nchunks + c) * (DD + 2); };

  if (t0 >= t1) {
    for (int e = tid; e < nh * (DD + 2); e += 256) {
      const int hh = e / (DD + 2), j = e % (DD + 2);
      part(hh)[j] = (j == DD) ? -INFINITY : 0.f;
    }
    return;
  }
  const int n = t1 - t0;
  const int64_t srec = (int64_t)stream * a.capacity;
  const float *wk = a.tables->walsh[KB];
  const float *wv = a.tables->walsh[VB];

  // ---- phase K: logits of all tokens of the chunk (log2 units) ----
  const int8_t *qf = a.qfrag + (int64_t)sg * 2 * 2 * 64 * 16;
  const i4v aqr0 = *reinterpret_cast<const i4v *>(qf + ((0 * 2 + 0) * 64 + lane) * 16);
  const i4v aqr1 = *reinterpret_cast<const i4v *>(qf + ((0 * 2 + 1) * 64 + lane) * 16);
  const i4v aqs0 = *reinterpret_cast<const i4v *>(qf + ((1 * 2 + 0) * 64 + lane) * 16);
  const i4v aqs1 = *reinterpret_cast<const i4v *>(qf + ((1 * 2 + 1) * 64 + lane) * 16);
  const int tn = lane & 15, G = lane >> 4;  // MFMA column (token), row group (head)
  const float *qc = a.qconst + ((int64_t)sg * 4 + G) * 4;
  const float sr = qc[0], ss = qc[1];
  const int qsum = __float_as_int(qc[2]), qssum = __float_as_int(qc[3]);
  float vmx = 0.f;
  const int ntile = (n + 15) >> 4;
  for (int tile = wave; tile < ntile; tile += 4) {
    const int tl = tile * 16 + tn;
    const bool valid = tl < n;
    const int64_t rec = srec + t0 + tl;
    uint32_t pl[5] = {0, 0, 0, 0, 0};
    float2 kn = make_float2(0.f, 0.f);
    if (valid) {
      const uint32_t *src = a.kbits + (rec * DW + G) * (KB + 1);
#pragma unroll
      for (int p = 0; p <= KB; ++p) pl[p] = src[p];
      kn = *reinterpret_cast<const float2 *>(a.knorm + 2 * rec);
      if (G == 0) vmx = fmaxf(vmx, a.vnorm[rec]);
    }
    float code = 0.f;
#pragma unroll
    for (int mi = 0; mi < KM; ++mi) {
      const int S = (mi < KB) ? (1 << mi) : (KB == 3 ? 7 : (mi == 4 ? 7 : mi == 5 ? 11 : mi == 6 ? 13 : 14));
      i4v lo, hi, acc = {0, 0, 0, 0};
      mask_bytes(xor_planes(pl, S), lo, hi);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(aqr0, lo, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(aqr1, hi, acc, 0, 0, 0);
      const int T = 2 * combine_digits(acc) - qsum;
      code += wk[mi] * (float)T;
    }
    int Ts;
    {
      i4v lo, hi, acc = {0, 0, 0, 0};
      mask_bytes(pl[KB], lo, hi);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(aqs0, lo, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(aqs1, hi, acc, 0, 0, 0);
      Ts = 2 * combine_digits(acc) - qssum;
    }
    const float s = kn.x * (sr * code + a.qjl_scale * kn.y * ss * (float)Ts);
    if (G < nh && valid) lg[G * a.chunk + tl] = s * a.scale_log2;
  }
  // wave max of the value norms
  for (int off = 32; off > 0; off >>= 1) vmx = fmaxf(vmx, __shfl_xor(vmx, off));
  if (lane == 0) red[0][wave] = vmx;
  // zero the value A fragments
  const int ngrp = (n + 127) >> 7;
  for (int e = tid; e < ngrp * 2 * 64 * 16 / 16; e += 256) reinterpret_cast<uint4 *>(av)[e] = make_uint4(0, 0, 0, 0);
  __syncthreads();
  if (tid == 0) vmaxs = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  // per-head max: wave w handles head w
  if (wave < nh) {
    float m = -INFINITY;
    for (int t = lane; t < n; t += 64) m = fmaxf(m, lg[wave * a.chunk + t]);
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if (lane == 0) hmax[wave] = m;
  }
  __syncthreads();
  // ---- softmax weights -> fixed-point value digits ----
  const float vmax = vmaxs;
  const float wq = vmax > 0.f ? WSCALE / vmax : 0.f;
  if (wave < nh) {
    const float m = hmax[wave];
    float l = 0.f;
    double ws = 0.0;
    for (int t = lane; t < n; t += 64) {
      const float p = exp2f(lg[wave * a.chunk + t] - m);
      l += p;
      const float w = p * a.vnorm[srec + t0 + t];
      const int W = (int)rintf(w * wq);
      ws += (double)W;
      const uint32_t u = (uint32_t)W + 0x808080u;
      const int grp = t >> 7, tp = t & 127, gg = tp >> 5, rem = tp & 31, q = rem & 7, bb = rem >> 3;
      const int ins = q >> 2, qq = q & 3;
      int8_t *base = av + (((grp * 2 + ins) * 64 + gg * 16 + 4 * wave) * 16) + 4 * qq + bb;
      base[0] = (int8_t)((u & 0xFF) ^ 0x80);
      base[16] = (int8_t)(((u >> 8) & 0xFF) ^ 0x80);
      base[32] = (int8_t)(((u >> 16) & 0xFF) ^ 0x80);
    }
    for (int off = 32; off > 0; off >>= 1) {
      l += __shfl_xor(l, off);
      ws += __shfl_xor(ws, off);
    }
    if (lane == 0) {
      hsum[wave] = l;
      wsum[wave] = ws;
    }
  }
  __syncthreads();

  // ---- phase V: value sums on MFMA; wave w owns coordinates 32w .. 32w+31 ----
  i4v accv[2][VM];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int mi = 0; mi < VM; ++mi) accv[nt][mi] = i4v{0, 0, 0, 0};
  const int vn = lane & 15, vg = lane >> 4;  // coordinate column, token block in the 128-token group
  for (int grp = 0; grp < ngrp; ++grp) {
    const i4v a0 = *reinterpret_cast<const i4v *>(av + ((grp * 2 + 0) * 64 + lane) * 16);
    const i4v a1 = *reinterpret_cast<const i4v *>(av + ((grp * 2 + 1) * 64 + lane) * 16);
    const int tb = grp * 128 + vg * 32;  // first token of this lane's block, chunk-relative
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int j = wave * 32 + nt * 16 + vn;
      uint32_t pl[4] = {0, 0, 0, 0};
      if (tb < n) {
        const int64_t blk = (srec + t0 + tb) >> 5;
        const uint32_t *src = a.vbits + (blk * DD + j) * VB;
#pragma unroll
        for (int p = 0; p < VB; ++p) pl[p] = src[p];
      }
#pragma unroll
      for (int mi = 0; mi < VM; ++mi) {
        const int S = (mi < VB) ? (1 << mi) : (VB == 3 ? 7 : (mi == 4 ? 7 : mi == 5 ? 11 : mi == 6 ? 13 : 14));
        i4v lo, hi;
        mask_bytes(xor_planes(pl, S), lo, hi);
        accv[nt][mi] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, lo, accv[nt][mi], 0, 0, 0);
        accv[nt][mi] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, hi, accv[nt][mi], 0, 0, 0);
      }
    }
  }
  // flush: lane (coordinate vn, head vg) holds digits 0..2 of every mask sum
  if (vg < nh) {
    const double W = wsum[vg];
    const double unit = (double)vmax / (double)WSCALE;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      double o = 0.0;
#pragma unroll
      for (int mi = 0; mi < VM; ++mi) {
        const i4v &x = accv[nt][mi];
        const double M = (double)x[0] + 256.0 * (double)x[1] + 65536.0 * (double)x[2];
        o += (double)wv[mi] * (2.0 * M - W);
      }
      part(vg)[wave * 32 + nt * 16 + vn] = (float)(o * unit);
    }
  }
  if (tid < nh) {
    part(tid)[DD] = hmax[tid];
    part(tid)[DD + 1] = hsum[tid];
  }
}

__global__ void __launch_bounds__(128) decode_merge_kernel(DecodeArgs a) {
  __shared__ float orot[DD];
  const int bh = blockIdx.x;  // b * q_heads + h
  const int j = threadIdx.x;
  const float *p = a.partial + (int64_t)bh * a.nchunks * (DD + 2);
  float M = -INFINITY;
  for (int c = 0; c < a.nchunks; ++c) M = fmaxf(M, p[c * (DD + 2) + DD]);
  float L = 0.f, o = 0.f;
  if (M > -INFINITY) {
    for (int c = 0; c < a.nchunks; ++c) {
      const float m = p[c * (DD + 2) + DD];
      if (m == -INFINITY) continue;
      const float f = exp2f(m - M);
      L += f * p[c * (DD + 2) + DD + 1];
      o += f * p[c * (DD + 2) + j];
    }
  }
  orot[j] = L > 0.f ? o / L : 0.f;
  __syncthreads();
  float acc = 0.f;
  for (int k = 0; k < DD; ++k) acc += a.rot[k * DD + j] * orot[k];  // o = Pi^T o_rot
  a.out[(int64_t)bh * DD + j] = acc;
}

size_t decode_ws_bytes(const tq_ctx *ctx, const tq_kv_cache *cache, int32_t q_heads, int *chunk_out,
                       int *nchunks_out) {
  const int group = q_heads / cache->kv_heads;
  const int hgroups = (group + 3) / 4;
  const int maxlen = cache->host_max_len > 0 ? cache->host_max_len : cache->capacity;
  const int64_t streams = (int64_t)cache->batch * cache->kv_heads * hgroups;
  int chunk = 1024;
  while (chunk > 256 && streams * ((maxlen + chunk - 1) / chunk) < 2048) chunk >>= 1;
  const int nchunks = std::max(1, (maxlen + chunk - 1) / chunk);
  if (chunk_out) *chunk_out = chunk;
  if (nchunks_out) *nchunks_out = nchunks;
  size_t b = 0;
  b += (size_t)streams * 2 * 2 * 64 * 16;  // qfrag
  b = (b + 255) & ~(size_t)255;
  b += (size_t)streams * 16 * sizeof(float);  // qconst
  b = (b + 255) & ~(size_t)255;
  b += (size_t)cache->batch * q_heads * nchunks * (DD + 2) * sizeof(float);  // partials
  (void)ctx;
  return b;
}

template <int KB, int VB>
static hipError_t launch_decode_kv(const DecodeArgs &a, dim3 grid, size_t shm, hipStream_t st) {
  hipLaunchKernelGGL((decode_kernel<KB, VB>), grid, dim3(256), shm, st, a);
  return hipGetLastError();
}

hipError_t launch_decode(const tq_ctx *ctx, const tq_kv_cache *cache, const void *q, int is_bf16, int32_t q_heads,
                         float scale, float *out, void *ws, hipStream_t st) {
  int chunk = 0, nchunks = 0;
  decode_ws_bytes(ctx, cache, q_heads, &chunk, &nchunks);
  DecodeArgs a = {};
  a.kbits = cache->k.bits;
  a.knorm = cache->k.norms;
  a.vbits = cache->v.bits;
  a.vnorm = cache->v.norms;
  a.seq_len = cache->d_seq_len;
  a.kbitsB = cache->k.mse_bits;
  a.vbitsB = cache->v.mse_bits;
  a.kv_heads = cache->kv_heads;
  a.capacity = cache->capacity;
  a.q_heads = q_heads;
  a.group = q_heads / cache->kv_heads;
  a.hgroups = (a.group + 3) / 4;
  a.chunk = chunk;
  a.nchunks = nchunks;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.qjl_scale = (float)(std::sqrt(M_PI / 2.0) / DD);
  a.tables = ctx->d_tables;
  a.q = q;
  a.q_bf16 = is_bf16;
  a.rot = ctx->d_rot;
  a.sketch = ctx->d_sketch;
  const int streams = cache->batch * cache->kv_heads * a.hgroups;
  char *p = (char *)ws;
  a.qfrag = (int8_t *)p;
  p += (((size_t)streams * 2 * 2 * 64 * 16) + 255) & ~(size_t)255;
  a.qconst = (float *)p;
  p += (((size_t)streams * 16 * sizeof(float)) + 255) & ~(size_t)255;
  a.partial = (float *)p;
  a.out = out;
  hipLaunchKernelGGL(decode_prep_kernel, dim3(streams), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t shm = (size_t)4 * chunk * sizeof(float) + (size_t)(chunk / 128) * 2 * 64 * 16;
  dim3 grid(nchunks, streams);
  const int kb = cache->k.mse_bits, vb = cache->v.mse_bits;
  if (kb == 3 && vb == 3) e = launch_decode_kv<3, 3>(a, grid, shm, st);
  else if (kb == 2 && vb == 3) e = launch_decode_kv<2, 3>(a, grid, shm, st);
  else if (kb == 2 && vb == 2) e = launch_decode_kv<2, 2>(a, grid, shm, st);
  else if (kb == 1 && vb == 3) e = launch_decode_kv<1, 3>(a, grid, shm, st);
  else if (kb == 3 && vb == 2) e = launch_decode_kv<3, 2>(a, grid, shm, st);
  else if (kb == 4 && vb == 4) e = launch_decode_kv<4, 4>(a, grid, shm, st);
  else if (kb == 4 && vb == 3) e = launch_decode_kv<4, 3>(a, grid, shm, st);
  else if (kb == 1 && vb == 1) e = launch_decode_kv<1, 1>(a, grid, shm, st);
  else return hipErrorInvalidValue;
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(cache->batch * q_heads), dim3(DD), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Append: one block of 128 threads (thread = coordinate) per (b, h) stream.
// ---------------------------------------------------------------------------

struct AppendArgs {
  const void *k, *v;
  int bf16;
  const float *rot, *sketch;
  const DeviceTables *tables;
  uint32_t *kbits;
  float *knorm;
  uint32_t *vbits;
  float *vnorm;
  const int32_t *seq_len;
  int kB, vB, kv_heads, capacity;
};

__device__ __forceinline__ float block_sum128(float v, float *red) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = red[0] + red[1];
  __syncthreads();
  return r;
}

__global__ void __launch_bounds__(128) append_kernel(AppendArgs a) {
  __shared__ float xs[DD], rs[DD];
  __shared__ float red[2];
  const int stream = blockIdx.x, j = threadIdx.x, lane = j & 63, wv = j >> 6;
  const int b = stream / a.kv_heads;
  const int t = a.seq_len[b];
  if (t >= a.capacity) return;
  const int64_t rec = (int64_t)stream * a.capacity + t;
  // ---- key ----
  {
    const int64_t off = (int64_t)stream * DD + j;
    const float x = a.bf16 ? bf16f(((const uint16_t *)a.k)[off]) : ((const float *)a.k)[off];
    xs[j] = x;
    const float nrm = sqrtf(block_sum128(x * x, red));  // also orders the xs writes
    float y = 0.f;
    for (int k = 0; k < DD; ++k) y += a.rot[j * DD + k] * xs[k];
    const bool live = nrm > 0.f;
    y = live ? y / nrm : 0.f;
    const int L = 1 << a.kB;
    int idx = 0;
    for (int i = 0; i < L - 1; ++i) idx += (y >= a.tables->boundary[a.kB][i]) ? 1 : 0;
    if (!live) idx = 0;
    const float r = live ? y - a.tables->centroid[a.kB][idx] : 0.f;
    rs[j] = r;
    const float rho = sqrtf(block_sum128(r * r, red));
    float z = 0.f;
    for (int k = 0; k < DD; ++k) z += a.sketch[j * DD + k] * rs[k];
    const bool sg = live && z >= 0.f;
    uint32_t words[5];
    for (int p = 0; p < a.kB; ++p) {
      const uint64_t bal = __builtin_amdgcn_ballot_w64(((idx >> p) & 1) != 0);
      words[p] = (lane < 32) ? (uint32_t)bal : (uint32_t)(bal >> 32);
    }
    {
      const uint64_t bal = __builtin_amdgcn_ballot_w64(sg);
      words[a.kB] = (lane < 32) ? (uint32_t)bal : (uint32_t)(bal >> 32);
    }
    if ((lane & 31) == 0) {
      const int w = wv * 2 + (lane >> 5);
      uint32_t *dst = a.kbits + (rec * DW + w) * (a.kB + 1);
      for (int p = 0; p <= a.kB; ++p) dst[p] = words[p];
    }
    if (j == 0) {
      a.knorm[2 * rec] = nrm;
      a.knorm[2 * rec + 1] = live ? rho : 0.f;
    }
  }
  __syncthreads();
  // ---- value ----
  {
    const int64_t off = (int64_t)stream * DD + j;
    const float x = a.bf16 ? bf16f(((const uint16_t *)a.v)[off]) : ((const float *)a.v)[off];
    xs[j] = x;
    const float nrm = sqrtf(block_sum128(x * x, red));
    float y = 0.f;
    for (int k = 0; k < DD; ++k) y += a.rot[j * DD + k] * xs[k];
    const bool live = nrm > 0.f;
    y = live ? y / nrm : 0.f;
    const int L = 1 << a.vB;
    int idx = 0;
    for (int i = 0; i < L - 1; ++i) idx += (y >= a.tables->boundary[a.vB][i]) ? 1 : 0;
    if (!live) idx = 0;
    const int64_t blk = rec >> 5;
    const int pos = (int)(rec & 31);
    uint32_t *dst = a.vbits + (blk * DD + j) * a.vB;
    for (int p = 0; p < a.vB; ++p) {
      const uint32_t bit = (uint32_t)((idx >> p) & 1) << pos;
      dst[p] = (pos == 0) ? bit : ((dst[p] & ~(1u << pos)) | bit);
    }
    if (j == 0) a.vnorm[rec] = nrm;
  }
}

__global__ void append_len_kernel(int32_t *seq_len, int batch, int capacity) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < batch && seq_len[b] < capacity) seq_len[b] += 1;
}

hipError_t launch_append(const tq_ctx *ctx, const tq_kv_cache *cache, const void *k, const void *v, int is_bf16,
                         hipStream_t st) {
  AppendArgs a = {};
  a.k = k;
  a.v = v;
  a.bf16 = is_bf16;
  a.rot = ctx->d_rot;
  a.sketch = ctx->d_sketch;
  a.tables = ctx->d_tables;
  a.kbits = cache->k.bits;
  a.knorm = cache->k.norms;
  a.vbits = cache->v.bits;
  a.vnorm = cache->v.norms;
  a.seq_len = cache->d_seq_len;
  a.kB = cache->k.mse_bits;
  a.vB = cache->v.mse_bits;
  a.kv_heads = cache->kv_heads;
  a.capacity = cache->capacity;
  hipLaunchKernelGGL(append_kernel, dim3(cache->batch * cache->kv_heads), dim3(DD), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(append_len_kernel, dim3((cache->batch + 255) / 256), dim3(256), 0, st, cache->d_seq_len,
                     cache->batch, cache->capacity);
  return hipGetLastError();
}

}  // namespace tq
