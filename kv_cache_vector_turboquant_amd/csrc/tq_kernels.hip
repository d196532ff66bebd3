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
//                      exact fp6 digits laid out as MFMA A fragments.
//  decode_kernel       split-K decode attention over packed K/V: key scores on
//                      fp6 x fp4 MFMA, value sums on int8 MFMA, both over bit
//                      masks.
//  decode_merge_kernel log-sum-exp merge of the chunks and inverse rotation.
//  append_kernel       quantizes one K and one V vector per stream in place.
//  topk_kernel         per-query top-k by (-score, index).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cfloat>
#include <climits>
#include <cmath>
#include <mutex>

#include "tq_device.h"
#include "tq_internal.h"
#include <hip/hip_fp16.h>

namespace tq {

// Norms are stored as fp32, or as fp16 (round to nearest even, saturated at the
// largest finite fp16) when the array's norm_f16 flag is set.
__device__ __forceinline__ void store_norm(void *base, int64_t i, float x, int f16) {
  if (f16) reinterpret_cast<__half *>(base)[i] = __float2half_rn(fminf(x, 65504.f));
  else reinterpret_cast<float *>(base)[i] = x;
}
__device__ __forceinline__ float load_norm(const void *base, int64_t i, int f16) {
  return f16 ? __half2float(reinterpret_cast<const __half *>(base)[i]) : reinterpret_cast<const float *>(base)[i];
}

typedef float f16v __attribute__((ext_vector_type(16)));

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
  int qjl;               // keys: 1 = QJL sign word and |r| in the record, 0 = MSE-only
  uint32_t *bits_out;
  void *norms_out;
  int nf16;              // norms_out holds fp16 norms
  float *resid;          // keys: residual rows [stream*n_tokens + t][d]
  int64_t n_tokens;
  RecMap map;            // record of (stream, token)
  // store / scores epilogues
  float *c;
  int64_t ldc;
  // scores B loader (packed keys)
  const uint32_t *kbits;
  const void *knorm;
  int knf16;             // knorm holds fp16 norms
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
  const int W = g.d >> 5, B = g.bits, Q = g.qjl;
#pragma unroll
  for (int gg = 0; gg < 2; ++gg) {
    const int r = (tid >> 2) + 64 * gg;
    const int k = k0 + (tid & 3) * 4;
    const int64_t t = row0 + r;
    float e[4] = {0.f, 0.f, 0.f, 0.f};
    if (t < g.b.nrows) {
      const uint32_t *rec = g.kbits + t * (int64_t)(W * (B + Q));
      if (k < g.d) {
        if (B > 0) {  // pure QJL keys have no codebook term
          const int w = k >> 5, o = k & 31;
          int idx[4] = {0, 0, 0, 0};
          for (int p = 0; p < B; ++p) {
            const uint32_t word = rec[w * (B + Q) + p] >> o;
#pragma unroll
            for (int q = 0; q < 4; ++q) idx[q] |= ((word >> q) & 1u) << p;
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) e[q] = cent[idx[q]];
        }
      } else if (Q) {  // MSE-only keys have no QJL term
        const int i = k - g.d, w = i >> 5, o = i & 31;
        const uint32_t word = rec[w * (B + 1) + B] >> o;
        const float a = g.qjl_scale * load_norm(g.knorm, 2 * t + 1, g.knf16);
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
      if constexpr (MODE == MODE_SCORES) scale = (col < g.N) ? load_norm(g.knorm, (1 + g.qjl) * col, g.knf16) : 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = row0 + wm * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
        if (row < g.M && col < g.N) g.c[row * g.ldc + col] = acc[b][r] * scale;
      }
    }
  } else if constexpr (MODE == MODE_KEY_CODES || MODE == MODE_KEY_SIGNS) {
    // rows = tokens of stream s, columns = coordinates (codes) or sketch rows (signs)
    const int W = g.d >> 5;
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
          const int idx = B > 0 ? quant_index(y, bnd, L) : 0;
          // the residual feeds the sketch (pure QJL keys: the whole rotated vector)
          if (in && g.qjl) g.resid[(s * g.n_tokens + t) * (int64_t)g.d + col] = live ? y - (B > 0 ? cent[idx] : 0.f) : 0.f;
          mybits = live ? (uint32_t)idx : 0u;
        } else {
          live = in && load_norm(g.norms_out, 2 * g.map.rec(s, t), g.nf16) > 0.f;  // signs only exist with the QJL stage: 2 norms
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
      const int64_t rec = t < g.n_tokens ? g.map.rec(s, t) : 0;
      if (t < g.n_tokens && w < W) {
        uint32_t *dst = g.bits_out + (rec * W + w) * (int64_t)(B + g.qjl);
        if constexpr (MODE == MODE_KEY_CODES) {
          for (int p = 0; p < B; ++p) dst[p] = cw[(rl * (GBN / 32) + gl) * 4 + p];
        } else {
          dst[B] = cw[(rl * (GBN / 32) + gl) * 4];
        }
      }
      if (ct == 0 && gl == 0 && t < g.n_tokens) {
        if constexpr (MODE == MODE_KEY_CODES) store_norm(g.norms_out, (1 + g.qjl) * rec, sqrtf(stat[rl]), g.nf16);
        else store_norm(g.norms_out, 2 * rec + 1, sqrtf(stat[rl]), g.nf16);
      }
    }
  } else if constexpr (MODE == MODE_VAL_CODES) {
    // rows = coordinates, columns = tokens of stream s; ballots are token-major words.
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
            const int64_t blk = g.map.rec(s, blk_t0) >> 5;
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
        if (t < g.n_tokens) store_norm(g.norms_out, g.map.rec(s, t), sqrtf(stat[cl]), g.nf16);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Fused quantize for d = 128 and bf16 input, one work-group per 64 tokens.
//
// The products run on bf16 MFMA (16x16x32 for keys, 32x32x16 for values). The
// input is exact in bf16 and Pi
// is split into three bf16 parts (hi + mid + lo carry its 24 bits), so
// y = Pi x accumulates in fp32 exactly as an fp32 GEMM would, up to rounding
// order. For keys the residual r = y - c[idx] and S are split into two parts
// each (hi*hi + hi*lo + lo*hi): z = S r is then accurate to ~2^-17 relative,
// which only decides signs of |z| far below the 1e-5 band. The residual never
// leaves the chip: it is staged in LDS as bf16 (hi, lo) between the products.
//
// Codes come from |y| against the positive boundaries (the table is
// antisymmetric and its middle boundary is 0): mag = #{t_j <= |y|}, idx =
// L/2 + mag for y >= 0, L/2 - 1 - mag for y < 0 (only exact ties differ from
// #{t_i <= y}). Key codes (7-bit fields, bit 6 = QJL sign) are staged in LDS and a
// last pass gathers them into the bit-plane words; value codes go straight to
// bit-plane words through ballots.
// ---------------------------------------------------------------------------

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
constexpr int QT = 64;   // tokens per work-group
constexpr int QD = 128;  // vector dimension of this path
constexpr int QW = QD / 32;

struct Q128Args {
  const uint16_t *x;       // bf16 input
  int64_t n_streams, n_tokens, xs, xt;  // tokens per stream; stream / token strides (elements)
  const uint16_t *rot3;    // [3][128][128] bf16 parts of Pi: [part][output coordinate][k]
  const uint16_t *sk2;     // [2][128][128] bf16 parts of S: [part][sketch row][coordinate]
  const DeviceTables *tables;
  uint32_t *bits_out;
  void *norms_out;
  int nf16;                // norms_out holds fp16 norms
  RecMap map;              // record of (stream, token)
};

__device__ __forceinline__ bf16x8 ld_bf8(const uint16_t *p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(p));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// sum of squares of 8 bf16 values (products exact, fp32 accumulation)
__device__ __forceinline__ float sumsq8(bf16x8 v, float s) {
  const uint4 u = __builtin_bit_cast(uint4, v);
  const bf16x2 p0 = __builtin_bit_cast(bf16x2, u.x), p1 = __builtin_bit_cast(bf16x2, u.y);
  const bf16x2 p2 = __builtin_bit_cast(bf16x2, u.z), p3 = __builtin_bit_cast(bf16x2, u.w);
  s = __builtin_amdgcn_fdot2_f32_bf16(p0, p0, s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(p1, p1, s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(p2, p2, s, false);
  return __builtin_amdgcn_fdot2_f32_bf16(p3, p3, s, false);
}

// two fp32 values as bf16 (round to nearest even) hi parts packed in a dword,
// and the bf16 parts of what is left
__device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
  const bf16x2 h = {(__bf16)a, (__bf16)b};
  hi = __builtin_bit_cast(uint32_t, h);
  const float ra = a - __uint_as_float(hi << 16), rb = b - __uint_as_float(hi & 0xFFFF0000u);
  const bf16x2 l = {(__bf16)ra, (__bf16)rb};
  lo = __builtin_bit_cast(uint32_t, l);
}

// Staged code words hold four 7-bit fields (field k at bit 7k: code in bits 0..3,
// QJL sign of a key in bit 6). gather4 collects bit p of the four fields into bits
// 0..3 (field k -> bit k) with one full-rate 24-bit multiply: the masked bits sit
// at 0, 7, 14, 21 (below 2^24 after the shift), and the multiplier
// 2^18 + 2^12 + 2^6 + 1 moves field k's bit to 18 + k while every cross term
// lands on a distinct bit outside 18..21, so no carry reaches them.
constexpr uint32_t FIELD_MASK = 0x00204081u;
constexpr int QJL_FIELD_BIT = 6;
__device__ __forceinline__ uint32_t gather4(uint32_t w, int p) {
  return (__umul24((w >> p) & FIELD_MASK, 0x00041041u) >> 18) & 0xFu;
}

// LDS swizzle of 16-byte granules: row r of `gran` granules, granule g at g ^ (r & mask)
__device__ __forceinline__ int swz(int row, int gran_per_row, int g, int mask) {
  return row * gran_per_row + (g ^ (row & mask));
}

// Values, d = 128 with bf16 input: four waves per work-group, two work-groups
// per compute unit (one's MFMA phase overlaps the other's epilogue). Wave w owns
// the output coordinates 32w .. 32w + 31, with its rows of the three Pi parts in
// registers, and computes them as 32 x 32 blocks (coordinates x tokens) on the
// 32x32x16 bf16 MFMA. In that output each lane holds one token, so a wave-wide
// ballot of a comparison is already a token-major bit plane: its low dword for
// coordinate row 8 (r / 4) + r % 4 of accumulator register r, its high dword for
// the row four below. With c_j the ballot of |y| >= t_j over the increasing
// positive boundaries (a thermometer code of the magnitude index) and s the
// ballot of y < 0, the code bits are
//   bit p < B - 1:  s ^ (XOR of c_j over j + 1 = 2^p, 2 * 2^p, 3 * 2^p, ...)
//   bit B - 1:      ~s
// which is the code H + mag for y >= 0 and its mirror 2H - 1 - (H + mag) for
// y < 0. The plane words are formed on the scalar unit and moved into the lanes
// that store them, one writelane each.
// lane L of v takes the wave-uniform value x (v_writelane_b32; L a constant),
// through the compiler's own intrinsic so that the scheduler sees a VALU op
extern "C" __device__ int tq_llvm_writelane(int, int, int) __asm("llvm.amdgcn.writelane.i32");
__device__ __forceinline__ void writelane(uint32_t &v, uint32_t x, int lane) {
  v = (uint32_t)tq_llvm_writelane((int)x, lane, (int)v);
}

template <int B>
__global__ void __launch_bounds__(256, 2) quant128_values_kernel(Q128Args a) {
  constexpr int H = 1 << (B - 1);  // centroids per sign
  constexpr int NT = 256;          // threads
  constexpr int XG = QT * 16 / NT; // X granules per thread
  constexpr int NW = 32 * B;       // plane words of a wave per 32-token block
  constexpr int NV = (NW + 63) / 64;
  // X tile: token row t (64 rows of 16 granules of 8 bf16), granule g at t * 16 + (g ^ (t & 15))
  __shared__ __attribute__((aligned(16))) uint4 xs[QT * 16];
  __shared__ float ssq[QT];  // squared norms of the staged tile's tokens
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c32 = lane & 31, kh = lane >> 5;
  const int64_t tps = (a.n_tokens + QT - 1) / QT, total = tps * a.n_streams;
  float tp[H > 1 ? H - 1 : 1];  // positive boundaries
#pragma unroll
  for (int j = 0; j < H - 1; ++j) tp[j] = a.tables->boundary[B][H + j];
  // A fragments: row 32 wave + c32 of each Pi part, k = 16 ks + 8 kh .. + 7
  bf16x8 pf[8][3];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
    for (int sp = 0; sp < 3; ++sp) pf[ks][sp] = ld_bf8(a.rot3 + (sp * QD + 32 * wave + c32) * QD + ks * 16 + kh * 8);
  }
  // X granule P (0..1023) of the tile at token tt0 of stream st, for slot P of the
  // swizzled LDS tile (rows past the stream's end re-read its last token)
  auto x_granule = [&](int64_t st, int64_t tt0, int P) {
    const int last = (int)min((int64_t)QT, a.n_tokens - tt0) - 1;
    const int t = P >> 4, g = (P & 15) ^ (t & 15);
    return *reinterpret_cast<const uint4 *>(a.x + st * a.xs + (tt0 + min(t, last)) * a.xt + g * 8);
  };
  // a tile's X into LDS, with each token's squared norm: the 16 slots of token t
  // are 16 consecutive threads (a 16-lane shuffle sum of their bf16 squares,
  // each product exact in fp32)
  auto stage_x = [&](const uint4 (&v)[XG]) {
#pragma unroll
    for (int i = 0; i < XG; ++i) {
      xs[i * NT + tid] = v[i];
      float q = sumsq8(__builtin_bit_cast(bf16x8, v[i]), 0.f);
      q += __shfl_xor(q, 1);
      q += __shfl_xor(q, 2);
      q += __shfl_xor(q, 4);
      q += __shfl_xor(q, 8);
      if ((tid & 15) == 0) ssq[(i * NT + tid) >> 4] = q;
    }
  };

  // work-groups loop over (stream, 64-token tile) pairs (tiles of stream s are
  // s * tps .. s * tps + tps - 1), advancing by the grid size with one division
  // per launch. Software pipeline: a step multiplies the current tile while it
  // forms and stores the codes of the previous one (its products held in the
  // other set of accumulators), in one region without branches so that the
  // matrix core and the VALU work side by side within each wave; the next
  // tile's X is loaded into registers meanwhile and written to LDS once every
  // wave is past its reads of the current X.
  int64_t tile = blockIdx.x;
  if (tile >= total) return;
  const int64_t dS = (int64_t)gridDim.x / tps, dR = (int64_t)gridDim.x % tps;
  int64_t s = tile / tps, tr = tile % tps;  // the current tile: stream, tile in the stream
  uint4 xr[XG];
#pragma unroll
  for (int i = 0; i < XG; ++i) xr[i] = x_granule(s, tr * QT, i * NT + tid);
  stage_x(xr);
  // the pending tile: products in accumulators, codes still to store
  bool pv = false;
  int64_t sP = s, t0P = tr * QT;
  int nvP = 0;
  float invP[2] = {0.f, 0.f};
  bool liveP[2] = {false, false};
  f16v accA[2], accB[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int r = 0; r < 16; ++r) accA[h][r] = accB[h][r] = 0.f;

  // one step; returns true when there is nothing left to do
  auto step = [&](f16v (&accC)[2], f16v (&accP)[2]) -> bool {
    const bool cv = tile < total;  // a current tile exists
    if (!cv && !pv) return true;
    const int64_t t0 = tr * QT;
    const int nv = cv ? (int)min((int64_t)QT, a.n_tokens - t0) : 0;
    const bool more = tile + gridDim.x < total;
    int64_t sn = s + dS, trn = tr + dR;  // the next tile
    if (trn >= tps) {
      trn -= tps;
      ++sn;
    }
    // X to load: the next tile's, else a valid tile's again (not staged)
    const int64_t ls = more ? sn : (cv ? s : sP), lt = more ? trn * QT : (cv ? t0 : t0P);
    __syncthreads();  // the current tile's X and norms are staged
#pragma unroll
    for (int i = 0; i < XG; ++i) xr[i] = x_granule(ls, lt, i * NT + tid);
    // this lane's tokens c32 and 32 + c32 of the current tile: inverse norms and
    // liveness (inside the tile, nonzero); zero vectors get all-zero code bits
    float inv[2];
    bool live[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float ss = ssq[32 * h + c32];
      inv[h] = ss > 0.f ? __builtin_amdgcn_rsqf(ss) : 0.f;
      live[h] = 32 * h + c32 < nv && ss > 0.f;
    }
    const float nrm = sqrtf(ssq[lane]);

    // ---- products of the current tile, interleaved with the codes of the pending
    // one: accC[h][r] = |x| y[coordinate 32 wave + 8 (r / 4) + 4 kh + r % 4][token 32 h + c32].
    // Codes as ballots: row (h, r) of the pending tile's accumulators gives its
    // plane words for coordinates 8 (r / 4) + r % 4 (low dword) and 4 below (high).
    uint32_t w[2][NV];
    uint64_t lvm[2];  // both dwords: live tokens 32h .. 32h + 31 of the pending tile
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      lvm[h] = __builtin_amdgcn_ballot_w64(liveP[h]);
#pragma unroll
      for (int v = 0; v < NV; ++v) w[h][v] = 0u;
    }
    auto codes = [&](int h, int r) {
      const float y = accP[h][r] * invP[h];
      uint64_t c[H > 1 ? H - 1 : 1];
#pragma unroll
      for (int j = 0; j < H - 1; ++j) c[j] = __builtin_amdgcn_ballot_w64(fabsf(y) >= tp[j]);
      const uint64_t sg = __builtin_amdgcn_ballot_w64(y < 0.f);
      const int row = 8 * (r >> 2) + (r & 3);
#pragma unroll
      for (int p = 0; p < B; ++p) {
        uint64_t m = ~sg;
        if (p < B - 1) {
          m = sg;
#pragma unroll
          for (int q = 1 << p; q <= H - 1; q += 1 << p) m ^= c[q - 1];
        }
        const int i0 = row * B + p, i1 = (row + 4) * B + p;
        writelane(w[h][i0 >> 6], (uint32_t)m, i0 & 63);
        writelane(w[h][i1 >> 6], (uint32_t)(m >> 32), i1 & 63);
      }
    };
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 16; ++r) accC[h][r] = 0.f;
    bf16x8 xf[2][2];  // X fragments of k step ks (buffer ks & 1), loaded one step ahead
    auto load_xf = [&](int ks) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int t = 32 * h + c32;
        xf[ks & 1][h] = __builtin_bit_cast(bf16x8, xs[t * 16 + ((2 * ks + kh) ^ (t & 15))]);
      }
    };
    load_xf(0);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (ks < 7) load_xf(ks + 1);
#pragma unroll
      for (int sp = 0; sp < 3; ++sp)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          accC[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf[ks][sp], xf[ks & 1][h], accC[h], 0, 0, 0);
#pragma unroll
      for (int q = 0; q < 4; ++q) codes(ks >> 2, 4 * (ks & 3) + q);
      // issue order within the step: the next fragments' LDS reads, then each
      // MFMA followed by VALU work of the codes, so that the wave keeps issuing
      // VALU instructions while the matrix core runs
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads
#pragma unroll
      for (int i = 0; i < 6; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);  // seven VALU
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // tokens that are not live get zero bits: every plane word of block h has
    // bit t for token 32h + t, as the low dword of the liveness ballot does
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int v = 0; v < NV; ++v) w[h][v] &= (uint32_t)lvm[h];
    if (pv) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (32 * h >= nvP) break;
        const int64_t blk = a.map.rec(sP, t0P + 32 * h) >> 5;  // blocks never straddle pages
        uint32_t *dst = a.bits_out + (blk * QD + 32 * wave) * B;
#pragma unroll
        for (int v = 0; v < NV; ++v)
          if (64 * v + lane < NW) dst[64 * v + lane] = w[h][v];
      }
    }
    if (tid < nv) store_norm(a.norms_out, a.map.rec(s, t0 + tid), nrm, a.nf16);
    __syncthreads();  // every wave is past its reads of the current X and norms
    if (more) stage_x(xr);
    // the current tile becomes the pending one
    pv = cv;
    sP = s;
    t0P = t0;
    nvP = nv;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      invP[h] = inv[h];
      liveP[h] = live[h];
    }
    if (cv) {
      tile += gridDim.x;
      s = sn;
      tr = trn;
    }
    return false;
  };
  for (;;) {
    if (step(accA, accB)) break;
    if (step(accB, accA)) break;
  }
}

// Keys with specialised waves. A work-group of sixteen waves: waves 0..7 (math)
// issue both products on the matrix core, waves 8..15 (epilogue) do the VALU
// work: codes, residual split, packing and the X staging. Each SIMD runs two
// waves of each kind, so the matrix core works through the math waves' MFMAs
// while the epilogue waves issue VALU instructions (the phase-ordered kernel
// runs every wave through the same phase at once, and the two never overlap).
// Math wave m owns the output coordinates (and sketch rows) 16m .. 16m + 15,
// with its rows of the Pi and S parts in registers; epilogue wave m owns the
// same coordinates of y. Tiles go through a pipeline of two phases per step j,
// a barrier after each:
//   phase 1  math: product 1 of tile j (y to LDS)
//            epilogue: pack of tile j - 2, loads of X for tile j + 1
//   phase 2  math: product 2 of tile j - 1 (sign bits into its code fields)
//            epilogue: codes and residual parts of tile j, X of tile j + 1 to LDS
// Buffers written in one step and read two steps on (codes, residual parts,
// norms, |r|^2 partials) alternate by tile parity; y and X are single buffers.
template <int B, bool SK>
__global__ void __launch_bounds__(1024) quant128_keys_kernel(Q128Args a) {
  constexpr int NPL = B + (SK ? 1 : 0);
  constexpr int H = B > 0 ? 1 << (B - 1) : 1;
  constexpr int NE = 512;            // epilogue threads
  constexpr int XG = QT * 16 / NE;   // X granules per epilogue thread
  constexpr int PH0 = (NPL + 1) / 2; // pack: planes per thread (two threads per token and group)
  __shared__ __attribute__((aligned(16))) uint4 xs[QT * 16];    // X tile, swizzled as in quant128_values_kernel
  __shared__ __attribute__((aligned(16))) f4v yb[8 * 4 * 64];   // y: [wave][tb][lane] (|x| y, 4 coordinates)
  __shared__ __attribute__((aligned(16))) uint32_t stage[2][QT * QD / 4];
  __shared__ __attribute__((aligned(16))) uint16_t rt[SK ? 2 : 1][2][SK ? QT * QD : 8];
  __shared__ float ssq[2][QT], nrm[2][QT];
  __shared__ float rho2[2][8][QT];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool math = wave < 8;
  const int m = wave & 7;  // coordinates 16m .. 16m + 15 (either role)
  const int c16 = lane & 15, kq = lane >> 4;
  const int te = tid - NE;  // epilogue thread index
  const int64_t tps = (a.n_tokens + QT - 1) / QT, total = tps * a.n_streams;
  const int64_t tile0 = blockIdx.x;
  if (tile0 >= total) return;
  const int T = (int)((total - 1 - tile0) / gridDim.x) + 1;  // tiles of this work-group
  // (stream, tile in the stream) of tile j: tile0 + j * gridDim.x, advanced by the
  // grid size without a division per step
  const int64_t dS = (int64_t)gridDim.x / tps, dR = (int64_t)gridDim.x % tps;
  struct TilePos {
    int64_t s, tr;
  };
  auto advance = [&](TilePos &p) {
    p.s += dS;
    p.tr += dR;
    if (p.tr >= tps) {
      p.tr -= tps;
      ++p.s;
    }
  };
  if (math) {
    // rows 16m + c16 of the Pi parts and of the S parts
    bf16x8 pf[4][3];
    bf16x8 sf[SK ? 4 : 1][2];
    {
      const int r = 16 * m + c16;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int sp = 0; sp < 3; ++sp) pf[ks][sp] = ld_bf8(a.rot3 + (sp * QD + r) * QD + ks * 32 + kq * 8);
        if constexpr (SK) {
#pragma unroll
          for (int sp = 0; sp < 2; ++sp) sf[ks][sp] = ld_bf8(a.sk2 + (sp * QD + r) * QD + ks * 32 + kq * 8);
        }
      }
    }
    // The two roles run separate loops with the same barriers (one for the first
    // X tile, then two per step), so the register-resident Pi and S parts are not
    // live through the epilogue code.
    __syncthreads();
    for (int j = 0; j < T + 2; ++j) {
      // ---- phase 1: product 1 of tile j
      if (j < T) {
        f4v acc[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) acc[tb] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          bf16x8 xf[4];
#pragma unroll
          for (int tb = 0; tb < 4; ++tb) {
            const int t = tb * 16 + c16;
            xf[tb] = __builtin_bit_cast(bf16x8, xs[t * 16 + ((ks * 4 + kq) ^ (t & 15))]);
          }
#pragma unroll
          for (int sp = 0; sp < 3; ++sp)
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
              acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[ks][sp], xf[tb], acc[tb], 0, 0, 0);
        }
        // acc[tb][r] = |x| y[coordinate 16m + 4kq + r][token tb*16 + c16]
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) yb[(m * 4 + tb) * 64 + lane] = acc[tb];
      }
      __syncthreads();
      // ---- phase 2: product 2 of tile j - 1, z[sketch row][token] = S r; signs into
      // bit 6 of the code fields
      if constexpr (SK) {
        if (j >= 1 && j <= T) {
          const int pb = (j - 1) & 1;
          f4v acc[4];
#pragma unroll
          for (int tb = 0; tb < 4; ++tb) acc[tb] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
              const int g = swz(tb * 16 + c16, 16, ks * 4 + kq, 15) * 8;
              const bf16x8 rh = ld_bf8(&rt[pb][0][g]), rl = ld_bf8(&rt[pb][1][g]);
              acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sf[ks][0], rh, acc[tb], 0, 0, 0);
              acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sf[ks][0], rl, acc[tb], 0, 0, 0);
              acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sf[ks][1], rh, acc[tb], 0, 0, 0);
            }
          }
          const int c0 = 16 * m + 4 * kq;
#pragma unroll
          for (int tb = 0; tb < 4; ++tb) {
            const int tok = tb * 16 + c16;
            uint32_t sg = 0;
#pragma unroll
            for (int r = 0; r < 4; ++r) sg |= (acc[tb][r] >= 0.f ? (1u << QJL_FIELD_BIT) : 0u) << (7 * r);
            atomicOr(&stage[pb][swz(tok, 8, c0 >> 4, 7) * 4 + ((c0 >> 2) & 3)], sg);
          }
        }
      }
      __syncthreads();
    }
    return;
  }
  // positive boundaries t_j (between magnitudes j and j + 1) and the centroid
  // magnitudes, the latter copied into VGPRs once (as select operands they would
  // otherwise be copied from SGPRs at every use). A leaf carries the magnitude
  // index i in its HB lowest mantissa bits, so one select tree gives both the
  // centroid and the code field; the centroid moves by at most 2^HB - 1 ulp
  // (below 10^-6 of it), far inside the tolerances of the residual's norm and of
  // the sketch signs.
  constexpr int HB = B > 1 ? B - 1 : 0;
  constexpr uint32_t HM = (1u << HB) - 1u;
  float tp[H > 1 ? H - 1 : 1];
  uint32_t cvg[H];  // leaves of the select tree (opaque to the compiler, which
                    // otherwise turns the tree into compares of the code)
  if constexpr (B > 0) {
#pragma unroll
    for (int j = 0; j < H - 1; ++j) tp[j] = a.tables->boundary[B][H + j];
#pragma unroll
    for (int i = 0; i < H; ++i) {
      const uint32_t c = (__float_as_uint(a.tables->centroid[B][H + i]) & ~HM) | (uint32_t)i;
      asm("v_mov_b32 %0, %1" : "=v"(cvg[i]) : "s"(c));
    }
  }
  // the magnitude index mag = #{t_j <= |y|} and the signed centroid of y, by a
  // binary tree of selects over the H leaves: node [i, i + 2w) takes its upper
  // half when |y| >= t_(i + w - 1), one compare per boundary and H - 1 selects
  auto code = [&](float y, uint32_t &mag) {
    const float ay = fabsf(y);
    uint32_t c;
    if constexpr (H == 1) {
      c = cvg[0];
    } else if constexpr (H == 2) {
      c = ay >= tp[0] ? cvg[1] : cvg[0];
    } else if constexpr (H == 4) {
      const bool g0 = ay >= tp[0], g1 = ay >= tp[1], g2 = ay >= tp[2];
      const uint32_t cl = g0 ? cvg[1] : cvg[0], ch = g2 ? cvg[3] : cvg[2];
      c = g1 ? ch : cl;
    } else {
      const bool g0 = ay >= tp[0], g1 = ay >= tp[1], g2 = ay >= tp[2], g3 = ay >= tp[3];
      const bool g4 = ay >= tp[4], g5 = ay >= tp[5], g6 = ay >= tp[6];
      const uint32_t c0 = g0 ? cvg[1] : cvg[0], c1 = g2 ? cvg[3] : cvg[2];
      const uint32_t c2 = g4 ? cvg[5] : cvg[4], c3 = g6 ? cvg[7] : cvg[6];
      const uint32_t c01 = g1 ? c1 : c0, c23 = g5 ? c3 : c2;
      c = g3 ? c23 : c01;
    }
    mag = c & HM;
    return __builtin_copysignf(__uint_as_float(c), y);
  };
  // X granule P of tile j (rows past the stream's end re-read its last token),
  // and its staging with the tokens' squared norms (the 16 granules of a token
  // are 16 consecutive threads: a 16-lane shuffle sum)
  auto x_load = [&](const TilePos &p, uint4 (&v)[XG]) {
    const int64_t s = p.s, t0 = p.tr * QT;
    const int last = (int)min((int64_t)QT, a.n_tokens - t0) - 1;
#pragma unroll
    for (int i = 0; i < XG; ++i) {
      const int P = i * NE + te, t = P >> 4, g = (P & 15) ^ (t & 15);
      v[i] = *reinterpret_cast<const uint4 *>(a.x + s * a.xs + (t0 + min(t, last)) * a.xt + g * 8);
    }
  };
  auto x_stage = [&](const uint4 (&v)[XG], int buf) {
#pragma unroll
    for (int i = 0; i < XG; ++i) {
      xs[i * NE + te] = v[i];
      float q = sumsq8(__builtin_bit_cast(bf16x8, v[i]), 0.f);
      q += __shfl_xor(q, 1);
      q += __shfl_xor(q, 2);
      q += __shfl_xor(q, 4);
      q += __shfl_xor(q, 8);
      if ((te & 15) == 0) ssq[buf][(i * NE + te) >> 4] = q;
    }
  };
  uint4 xr[XG];
  TilePos xp = {tile0 / tps, tile0 % tps};  // tile of the next X load
  TilePos pp = xp;                          // tile of the next pack
  x_load(xp, xr);
  x_stage(xr, 0);
  __syncthreads();
  for (int j = 0; j < T + 2; ++j) {
    // ---- phase 1: loads of X for tile j + 1; pack of tile j - 2, thread (token,
    // 32-coordinate group, half) -> half of the NPL words, and the token's norms
    if (j + 1 < T) {
      advance(xp);
      x_load(xp, xr);
    }
    if (j >= 2) {
      const int pb = j & 1;
      const int64_t s = pp.s, t0 = pp.tr * QT;
      advance(pp);
      const int nv = (int)min((int64_t)QT, a.n_tokens - t0);
      const int tok = (te >> 2) & (QT - 1), g = te & 3, h = te >> 8;
      if (tok < nv) {
        const int64_t rec = a.map.rec(s, t0 + tok);
        const float n = nrm[pb][tok];
        uint32_t w[PH0];
        if (n > 0.f) {
          const uint4 q0 = *reinterpret_cast<const uint4 *>(&stage[pb][swz(tok, 8, 2 * g, 7) * 4]);
          const uint4 q1 = *reinterpret_cast<const uint4 *>(&stage[pb][swz(tok, 8, 2 * g + 1, 7) * 4]);
          const uint32_t d8[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
          for (int i = 0; i < PH0; ++i) {
            const int p = PH0 * h + i;
            const int bit = p < B ? p : QJL_FIELD_BIT;
            uint32_t word = 0;
#pragma unroll
            for (int mm = 0; mm < 8; ++mm) word |= gather4(d8[mm], bit) << (4 * mm);
            w[i] = word;
          }
        } else {
#pragma unroll
          for (int i = 0; i < PH0; ++i) w[i] = 0u;
        }
        uint32_t *dst = a.bits_out + (rec * QW + g) * NPL + PH0 * h;
        if constexpr (NPL == 4) {
          *reinterpret_cast<uint2 *>(dst) = make_uint2(w[0], w[1]);
        } else {
#pragma unroll
          for (int i = 0; i < PH0; ++i)
            if (PH0 * h + i < NPL) dst[i] = w[i];
        }
        if (g == 0 && h == 0) {
          if constexpr (SK) {
            float r2 = 0.f;
#pragma unroll
            for (int v = 0; v < 8; ++v) r2 += rho2[pb][v][tok];
            store_norm(a.norms_out, 2 * rec, n, a.nf16);
            store_norm(a.norms_out, 2 * rec + 1, n > 0.f ? sqrtf(r2) : 0.f, a.nf16);
          } else {
            store_norm(a.norms_out, rec, n, a.nf16);
          }
        }
      }
    }
    __syncthreads();
    // ---- phase 2: codes and residual parts of tile j; X of tile j + 1 to LDS
    // (product 1 of tile j is done with the current X)
    if (j < T) {
      const int cb = j & 1;
      float ss[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) ss[tb] = ssq[cb][tb * 16 + c16];
      if (m == 0 && kq == 0) {
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) nrm[cb][tb * 16 + c16] = sqrtf(ss[tb]);
      }
      float rp[4] = {0.f, 0.f, 0.f, 0.f};
      const int c0 = 16 * m + 4 * kq;  // first of the lane's 4 coordinates
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const int tok = tb * 16 + c16;
        // 1/|x| by the hardware reciprocal square root (about 1 ulp: code decisions
        // move only for coordinates far inside the boundary tolerance)
        const float inv = ss[tb] > 0.f ? __builtin_amdgcn_rsqf(ss[tb]) : 0.f;
        const f4v y4 = yb[(m * 4 + tb) * 64 + lane];
        // code fields: H + mag, mirrored to 2H - 1 - (H + mag) for a negative y (the
        // sign's all-ones mask XORs 2H - 1 into the field)
        uint32_t bytes = 0, neg = 0;
        float res[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float y = y4[r] * inv;
          uint32_t mg = 0;
          res[r] = B > 0 ? y - code(y, mg) : y;  // pure QJL keys: the residual is y itself
          bytes |= mg << (7 * r);
          neg |= (uint32_t)(__float_as_int(y) >> 31) & ((uint32_t)(2 * H - 1) << (7 * r));
          if constexpr (SK) rp[tb] = fmaf(res[r], res[r], rp[tb]);
        }
        if constexpr (B > 0) bytes = (bytes | (uint32_t)H * 0x204081u) ^ neg;  // H in every 7-bit field
        stage[cb][swz(tok, 8, c0 >> 4, 7) * 4 + ((c0 >> 2) & 3)] = bytes;
        if constexpr (SK) {
          uint32_t hi2[2], lo2[2];
          split2(res[0], res[1], hi2[0], lo2[0]);
          split2(res[2], res[3], hi2[1], lo2[1]);
          const int gr = swz(tok, 16, c0 >> 3, 15) * 8 + ((c0 >> 2) & 1) * 4;
          *reinterpret_cast<uint2 *>(&rt[cb][0][gr]) = make_uint2(hi2[0], hi2[1]);
          *reinterpret_cast<uint2 *>(&rt[cb][1][gr]) = make_uint2(lo2[0], lo2[1]);
        }
      }
      if constexpr (SK) {
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          rp[tb] += __shfl_xor(rp[tb], 16);
          rp[tb] += __shfl_xor(rp[tb], 32);
        }
        if (kq == 0) {
#pragma unroll
          for (int tb = 0; tb < 4; ++tb) rho2[cb][m][tb * 16 + c16] = rp[tb];
        }
      }
    }
    if (j + 1 < T) x_stage(xr, (j + 1) & 1);
    __syncthreads();
  }
}

// Persistent launch: as many work-groups as fit on the device at once (keys one
// per compute unit, values two), at most one per tile.
template <bool KEYS, int B, bool QJL>
static hipError_t launch_quant128_b(const Q128Args &q, hipStream_t st) {
  const void *fn;
  if constexpr (KEYS) fn = reinterpret_cast<const void *>(&quant128_keys_kernel<B, QJL>);
  else fn = reinterpret_cast<const void *>(&quant128_values_kernel<B>);
  const int nt = KEYS ? 1024 : 256;
  static int resident = 0;  // work-groups resident on the device
  if (resident == 0) {
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e;
    if ((e = hipGetDevice(&dev)) != hipSuccess ||
        (e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess ||
        (e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, nt, 0)) != hipSuccess)
      return e;
    resident = std::max(1, cus * std::max(1, per_cu));
  }
  const int64_t tiles = ((q.n_tokens + QT - 1) / QT) * q.n_streams;
  const unsigned nwg = (unsigned)std::min<int64_t>(tiles, resident);
  if constexpr (KEYS)
    hipLaunchKernelGGL((quant128_keys_kernel<B, QJL>), dim3(nwg), dim3(1024), 0, st, q);
  else
    hipLaunchKernelGGL((quant128_values_kernel<B>), dim3(nwg), dim3(256), 0, st, q);
  return hipGetLastError();
}

// keys: B = 0..4 with the sketch (0 = pure QJL), 1..4 without (MSE-only); values: 1..4
template <bool KEYS>
static hipError_t launch_quant128(const Q128Args &q, int bits, bool qjl, hipStream_t st) {
  if constexpr (KEYS) {
    if (qjl) {
      switch (bits) {
        case 0: return launch_quant128_b<true, 0, true>(q, st);
        case 1: return launch_quant128_b<true, 1, true>(q, st);
        case 2: return launch_quant128_b<true, 2, true>(q, st);
        case 3: return launch_quant128_b<true, 3, true>(q, st);
        case 4: return launch_quant128_b<true, 4, true>(q, st);
        default: return hipErrorInvalidValue;
      }
    }
  }
  (void)qjl;
  switch (bits) {
    case 1: return launch_quant128_b<KEYS, 1, false>(q, st);
    case 2: return launch_quant128_b<KEYS, 2, false>(q, st);
    case 3: return launch_quant128_b<KEYS, 3, false>(q, st);
    case 4: return launch_quant128_b<KEYS, 4, false>(q, st);
    default: return hipErrorInvalidValue;
  }
}

static hipError_t quant128(const tq_ctx *ctx, bool keys, const void *x, int64_t n_streams, int64_t n_tokens,
                           int64_t xs, int64_t xt, const tq_packed *out, const RecMap &map, hipStream_t st) {
  Q128Args q = {};
  q.x = (const uint16_t *)x;
  q.n_streams = n_streams;
  q.n_tokens = n_tokens;
  q.xs = xs;
  q.xt = xt;
  q.rot3 = ctx->d_rot3;
  q.sk2 = ctx->d_sk2;
  q.tables = ctx->d_tables;
  q.bits_out = out->bits;
  q.norms_out = out->norms;
  q.nf16 = out->norm_f16;
  q.map = map;
  return keys ? launch_quant128<true>(q, out->mse_bits, out->qjl != 0, st)
              : launch_quant128<false>(q, out->mse_bits, false, st);
}

hipError_t launch_quantize_keys(const tq_ctx *ctx, const void *x, int is_bf16, int64_t n_streams, int64_t n_tokens,
                                int64_t xs, int64_t xt, const tq_packed *out, const RecMap &map, float *work,
                                hipStream_t st) {
  const int d = ctx->d;
  if (d == QD && is_bf16 && ctx->d_rot3) return quant128(ctx, true, x, n_streams, n_tokens, xs, xt, out, map, st);
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
  g.nf16 = out->norm_f16;
  g.qjl = out->qjl;
  g.resid = work;
  g.n_tokens = n_tokens;
  g.map = map;
  g.rows_on_x = 1;
  dim3 grid((unsigned)((n_tokens + GBM - 1) / GBM), (d + GBN - 1) / GBN, (unsigned)n_streams);
  hipLaunchKernelGGL(gemm_kernel<MODE_KEY_CODES>, grid, dim3(256), 0, st, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !out->qjl) return e;  // MSE-only keys stop after stage 1
  // stage 2: z = S r on the residual rows, sign bits and ||r||
  GemmArgs g2 = g;
  g2.a = {work, d, n_tokens, 0};
  g2.a_stream_stride = n_tokens * (int64_t)d;
  g2.b = {ctx->d_sketch, d, d, 0};
  hipLaunchKernelGGL(gemm_kernel<MODE_KEY_SIGNS>, grid, dim3(256), 0, st, g2);
  return hipGetLastError();
}

hipError_t launch_quantize_values(const tq_ctx *ctx, const void *x, int is_bf16, int64_t n_streams,
                                  int64_t n_tokens, int64_t xs, int64_t xt, const tq_packed *out, const RecMap &map,
                                  hipStream_t st) {
  const int d = ctx->d;
  if (d == QD && is_bf16 && ctx->d_rot3) return quant128(ctx, false, x, n_streams, n_tokens, xs, xt, out, map, st);
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
  g.nf16 = out->norm_f16;
  g.n_tokens = n_tokens;
  g.map = map;
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

hipError_t launch_gemm_store(const void *a, int a_bf16, int64_t lda, int64_t M, const float *b, int64_t ldb,
                             int64_t N, int K, float *c, int64_t ldc, hipStream_t st) {
  GemmArgs g = {};
  g.a = {a, lda, M, a_bf16};
  g.b = {b, ldb, N, 0};
  g.K = K;
  g.M = M;
  g.N = N;
  g.c = c;
  g.ldc = ldc;
  g.rows_on_x = 1;
  dim3 grid((unsigned)((M + GBM - 1) / GBM), (unsigned)((N + GBN - 1) / GBN), 1);
  hipLaunchKernelGGL(gemm_kernel<MODE_STORE>, grid, dim3(256), 0, st, g);
  return hipGetLastError();
}

bool search_supported(const tq_ctx *ctx, int32_t topk);
size_t search_ws_bytes(const tq_ctx *ctx, int64_t nq, int64_t n, int32_t topk, int *splits_out);
hipError_t launch_search(const tq_ctx *ctx, const void *q, int is_bf16, int64_t nq, const tq_packed *keys,
                         float *scores, int32_t topk, int32_t *top_idx, float *top_val, void *ws, hipStream_t st);

size_t scores_ws_bytes(const tq_ctx *ctx, int64_t nq, int64_t n, int32_t topk, int32_t want_scores) {
  if (search_supported(ctx, topk)) return search_ws_bytes(ctx, nq, n, topk, nullptr);
  size_t b = (size_t)nq * 2 * ctx->d * sizeof(float);  // [q_rot | q_s]
  b = (b + 255) & ~(size_t)255;
  if (topk > 0 && !want_scores) b += (size_t)nq * (size_t)n * sizeof(float);
  return b;
}

hipError_t launch_scores(const tq_ctx *ctx, const void *q, int is_bf16, int64_t nq, const tq_packed *keys,
                         float *scores, int32_t topk, int32_t *top_idx, float *top_val, void *ws, hipStream_t st) {
  if (search_supported(ctx, topk)) return launch_search(ctx, q, is_bf16, nq, keys, scores, topk, top_idx, top_val, ws, st);
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
  g3.qjl = keys->qjl;
  g3.d = d;
  g3.kbits = keys->bits;
  g3.knorm = keys->norms;
  g3.knf16 = keys->norm_f16;
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
// and prod_{p in S} s_p = 2 (XOR of planes in S) - 1 = chi_S. Hence
//   sum_j q_j c[idx_j] = sum_S w_S (2 M_S - sum_j q_j),  M_S = sum_j q_j mask_S,j.
//
// Keys (v_mfma_scale_f32_16x16x128_f8f6f4, fp6 A x fp4 B): the query is fixed
// point, split into 8 signed base-8 digits. A row (4*head + slot) carries digit
// slot (first instruction) and slot+4 (second), with e8m0 row scales 2^(3 digit).
// The B operand of a plane word w is four dwords of 0/1 fp4 nibbles, each made
// by one AND (one shift and AND for the last): nibble i of dword q holds bit
// 4i+q of w at nibble bit 0, 1, 2, 2 (values 0.5, 1, 2, 2 for q = 0..3). The A
// digits of element (q, i) are pre-scaled by 1, 1/2, 1/4, 1/4 (all exact in
// e2m3), so every product is d * b / 2; the B scale 2^2 makes each row
// accumulate 2 sum_j Q_j b_j, and the accumulator starts at -sum_j Q_j (per
// slot), so each row ends at sum_j Q_j chi_j of its digit slot, exactly (every
// partial sum is a multiple of 2^(3 slot) below 2^(3 slot + 23)).
//
// Values (v_mfma_i32_16x16x64_i8): token t of a 32-token block sits at bit
// t % 32 of the plane word, bit q + 8 k' for q = t % 8. The B bytes are w AND
// (0x01010101 << q): one AND per four tokens, byte values b * 2^q (q = 7 gives
// -128 b). The A digits compensate per token: the weight p * |v| is fixed point
// at 2^29 (relative to the chunk's largest |v|), divided by 2^q before
// rounding (negated for q = 7), and split into four signed base-256 digits,
// A row = 4*head + digit. Every weight keeps at least 22 bits; the int32 sums
// are exact, and o = unit * sum_S w_S (2 M_S - sum_t E_t) in double.
// ---------------------------------------------------------------------------

constexpr float QMAX = 7190000.f;  // |fixed-point query| bound with 8 signed base-8 digits in [-4, 3]
constexpr float WSCALE = 536870912.f;  // 2^29: fixed point of the value weights
constexpr int KTPW = 2;            // key tiles (16 tokens each) per wave per round (double-buffered)
constexpr int VGPI = 2;            // 128-token value groups per iteration
constexpr int QC = 2;              // per-head query constants: units of the q_rot and q_s digits

struct DecodeArgs {
  const uint32_t *kbits;
  const void *knorm;     // fp32, or fp16 with nf16
  const uint32_t *vbits;
  const void *vnorm;
  const int32_t *seq_len;
  int kbitsB, vbitsB;    // MSE bits of keys / values
  int kqjl;              // keys carry the QJL sign word and |r|
  int kv_heads, capacity, q_heads, group, hgroups;
  int chunk, nchunks;
  int streams_hg;        // KV streams x head groups (decode grid = nchunks x streams_hg)
  int batch;
  // many queries per KV head (prefill): query position i of sequence b and head j
  // of a KV head's group form virtual head i * group + j; head groups are groups
  // of 4 virtual heads. Decode is n_q = 1.
  int n_q, causal;       // causal: position i attends to t < seq_len - n_q + i + 1
  int vgroup;            // n_q * group virtual heads per KV stream
  int kv_streams;        // batch * kv_heads
  RecMap map;            // record of (KV stream, token): contiguous or paged
  const float *ext;      // EXT: logits (log2 units) [stream*hgroups][4][ext_stride], token-indexed
  int64_t ext_stride;
  int span_lg;           // log2 of the runs of consecutive records in a chunk (chunk or page size)
  float scale_log2;      // softmax scale * log2(e)
  float qjl_scale;
  const DeviceTables *tables;
  const void *q;
  int q_bf16;
  const float *rot, *rs_t;  // rs_t: [Pi ; S Pi]^T, 128 x 256 row-major
  uint32_t *qfrag;       // [stream*hgroups][2 (q_rot, q_s)][2 (digits 0-3, 4-7)][64 lanes][8] fp6 fragments
  float *qconst;         // [stream*hgroups][4][QC]: units of the fixed-point q_rot, q_s
  float *partial;        // [batch*q_heads][nchunks][DD + 2]
  float *out;
  // fused step: the prep launch first appends each stream's new K/V token
  const void *ka, *va;   // [batch][kv_heads][DD], the query dtype
  const float *sk;       // S, row-major
  uint32_t *kbits_w, *vbits_w;
  void *knorm_w, *vnorm_w;
  int nf16;              // the cache's norms are fp16
  int32_t *wlen;         // [batch] length after the append; read by decode_kernel instead of seq_len
  int32_t *len_inc;      // lengths the merge kernel advances (fused step only)
  // measurement: the key phase's logits (natural units), [batch][n_q][q_heads][logit_stride]
  float *logit_out;
  int64_t logit_stride;
};


template <typename QT>
__device__ __forceinline__ float qload(const QT *q, int64_t i) {
  if constexpr (sizeof(QT) == 2) return bf16f(q[i]);
  else return q[i];
}

// Fused step, append blocks: a block (512 threads) encodes the new K/V tokens of
// two KV streams, 2 * blk and 2 * blk + 1, each as record seq_len[b] of its
// stream: the record tq_append_token writes (Pi k and Pi v from the Pi rows of
// [Pi ; S Pi]^T, key code, residual, |r|, sign(S r), value code into the
// token-major words). Every global read that does not depend on the tokens (Pi
// rows, S rows, tables, the value words to update) is issued first, so the
// block waits on memory once; the Pi and S rows in registers serve both streams.
struct AppendLds {
  float x[2][2][DD];     // [stream][k, v][coordinate]
  float pp[4][4][DD];    // partial Pi x: [k quarter][stream * 2 + (k, v)][row]
  float res[2][DD];      // key residuals
  float zp[4][2][DD];    // partial S r: [coordinate quarter][stream][row]
  float red[2][8];       // per stream: |k|^2, |v|^2 wave sums (0..3), |r|^2 wave sums (4, 5)
  float tb[48];          // key boundaries, key centroids, value boundaries
};

__device__ __forceinline__ void append_pair(const DecodeArgs &a, int blk, int tid, bool bf16in, AppendLds &L) {
  const int nstreams = a.batch * a.kv_heads;
  const int kB = a.kbitsB, vB = a.vbitsB, kQ = a.kqjl;  // kQ: QJL sign word and |r| (uniform)
  const int lane = tid & 63, w = tid >> 6;
  const int r = tid & (DD - 1), kq = tid >> 7;
  // this thread's stream for the per-coordinate phases: (stream half, key or value)
  const int hs = __builtin_amdgcn_readfirstlane(tid >> 8), kv = (tid >> 7) & 1;  // hs: uniform per wave
  // Loads are issued in the order their values are needed, unconditionally
  // (clamped addresses), so that no wait covers a load it does not need (a wait
  // covers every earlier load): the table entry and the token, the Pi and S rows,
  // and last the value words, whose address needs the length and which are read
  // only at the end.
  int stream[2], pos[2];
  bool on[2];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    stream[s2] = 2 * blk + s2;
    pos[s2] = stream[s2] < nstreams ? a.seq_len[stream[s2] / a.kv_heads] : a.capacity;
  }
  float tbv;
  {
    const int which = min(tid >> 4, 2), i = tid & 15;
    tbv = which == 0 ? a.tables->boundary[kB][i] : which == 1 ? a.tables->centroid[kB][i] : a.tables->boundary[vB][i];
  }
  // thread (stream hs, k or v, coordinate r): its coordinate of the new token
  float xin;
  {
    const int64_t xo = (int64_t)min(stream[hs], nstreams - 1) * DD + r;
    const void *src = kv ? a.va : a.ka;
    xin = bf16in ? __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(src)[xo])
                 : reinterpret_cast<const float *>(src)[xo];
  }
  // thread (row r, quarter kq): 32 entries of row r of Pi (transposed: coalesced
  // over r) and of row r of S
  float prow[32], srow[32];
#pragma unroll
  for (int u = 0; u < 32; ++u) prow[u] = a.rs_t[(kq * 32 + u) * 2 * DD + r];
  if (kQ) {
    const float4 *sr = reinterpret_cast<const float4 *>(a.sk + (int64_t)r * DD + 32 * kq);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float4 v = sr[u];
      srow[4 * u] = v.x; srow[4 * u + 1] = v.y; srow[4 * u + 2] = v.z; srow[4 * u + 3] = v.w;
    }
  }
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
    on[s2] = stream[s2] < nstreams && pos[s2] >= 0 && pos[s2] < a.capacity;  // a full stream gets nothing appended
  // value coordinate threads: the words this token's bits go into (all requested together)
  // (stream hs is uniform per wave: a buffer over the token's 32-token block and
  // four unconditional loads per thread at offsets clamped into the block; words
  // p >= vB are not used)
  const int64_t rec = on[hs] ? a.map.rec(stream[hs], pos[hs]) : 0;
  const int bit_pos = (int)(rec & 31);
  uint32_t vold[4];
  uint32_t *vdst = a.vbits_w + ((rec >> 5) * DD + r) * vB;
  {
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc(a.vbits_w + (rec >> 5) * DD * vB, (short)0, DD * vB * 4, 0x00020000);
#pragma unroll
    for (int p = 0; p < 4; ++p)
      vold[p] = __builtin_amdgcn_raw_buffer_load_b32(vr, (uint32_t)(min(r * vB + p, DD * vB - 1) * 4), 0, 0);
  }
  if (tid < 48) L.tb[tid] = tbv;
  {
    // bf16 input: the 16 loaded bits are the top half of the fp32 value
    const float x = on[hs] ? (bf16in ? __uint_as_float(__float_as_uint(xin) << 16) : xin) : 0.f;
    L.x[hs][kv][r] = x;
    float sq = x * x;
    for (int off = 32; off > 0; off >>= 1) sq += __shfl_xor(sq, off);
    if (lane == 0) L.red[hs][w & 3] = sq;
  }
  __syncthreads();
  {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      const int k = kq * 32 + u;
      acc[0] = fmaf(prow[u], L.x[0][0][k], acc[0]);
      acc[1] = fmaf(prow[u], L.x[0][1][k], acc[1]);
      acc[2] = fmaf(prow[u], L.x[1][0][k], acc[2]);
      acc[3] = fmaf(prow[u], L.x[1][1][k], acc[3]);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) L.pp[kq][v][r] = acc[v];
  }
  __syncthreads();
  const float nk = sqrtf(L.red[hs][0] + L.red[hs][1]), nv = sqrtf(L.red[hs][2] + L.red[hs][3]);
  const int vi = hs * 2 + kv;
  const float yx = (L.pp[0][vi][r] + L.pp[1][vi][r]) + (L.pp[2][vi][r] + L.pp[3][vi][r]);
  int idx = 0;
  if (kv == 0) {
    // key coordinate r: code (threshold count), residual, |r|^2
    const bool live = nk > 0.f;
    const float y = live ? yx / nk : 0.f;
    for (int i = 0; i < (1 << kB) - 1; ++i) idx += (y >= L.tb[i]) ? 1 : 0;
    if (!live) idx = 0;
    const float res = live ? y - (kB > 0 ? L.tb[16 + idx] : 0.f) : 0.f;  // pure QJL keys: r = y
    L.res[hs][r] = res;
    float r2 = res * res;
    for (int off = 32; off > 0; off >>= 1) r2 += __shfl_xor(r2, off);
    if (lane == 0) L.red[hs][4 + (w & 1)] = r2;
  } else if (on[hs]) {
    // value coordinate r: code bits into the token-major words of its 32-token block
    const bool live = nv > 0.f;
    const float y = live ? yx / nv : 0.f;
    int iv = 0;
    for (int i = 0; i < (1 << vB) - 1; ++i) iv += (y >= L.tb[32 + i]) ? 1 : 0;
    if (!live) iv = 0;
    for (int p = 0; p < vB; ++p) {
      const uint32_t bit = (uint32_t)((iv >> p) & 1) << bit_pos;
      vdst[p] = (bit_pos == 0) ? bit : ((vold[p] & ~(1u << bit_pos)) | bit);
    }
  }
  __syncthreads();
  if (kQ) {
    // z = S r for both streams: thread (sketch row r, coordinate quarter kq)
    float z0 = 0.f, z1 = 0.f;
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      z0 = fmaf(srow[u], L.res[0][kq * 32 + u], z0);
      z1 = fmaf(srow[u], L.res[1][kq * 32 + u], z1);
    }
    L.zp[kq][0][r] = z0;
    L.zp[kq][1][r] = z1;
    __syncthreads();
  }
  if (kv == 0 && on[hs]) {
    // waves 0, 1 (stream 0) and 4, 5 (stream 1): key coordinate r
    const bool live = nk > 0.f;
    uint32_t words[5];
    for (int p = 0; p < kB; ++p) {
      const uint64_t bal = __builtin_amdgcn_ballot_w64(((idx >> p) & 1) != 0);
      words[p] = (lane < 32) ? (uint32_t)bal : (uint32_t)(bal >> 32);
    }
    if (kQ) {
      const float z = (L.zp[0][hs][r] + L.zp[1][hs][r]) + (L.zp[2][hs][r] + L.zp[3][hs][r]);
      const uint64_t sbal = __builtin_amdgcn_ballot_w64(live && z >= 0.f);
      words[kB] = (lane < 32) ? (uint32_t)sbal : (uint32_t)(sbal >> 32);
    }
    const int np = kB + kQ;
    if ((lane & 31) == 0) {
      uint32_t *dst = a.kbits_w + (rec * DW + (w & 1) * 2 + (lane >> 5)) * np;
      for (int p = 0; p < np; ++p) dst[p] = words[p];
    }
    if (r == 0) {
      store_norm(a.knorm_w, (1 + kQ) * rec, nk, a.nf16);
      if (kQ) store_norm(a.knorm_w, 2 * rec + 1, live ? sqrtf(L.red[hs][4] + L.red[hs][5]) : 0.f, a.nf16);
      store_norm(a.vnorm_w, rec, nv, a.nf16);
    }
  }
}

// Query blocks: each handles two (stream, head group) units, 2 * blk and
// 2 * blk + 1 (the [Pi ; S Pi] rows in registers serve both): q_rot = Pi q and
// q_s = S q_rot for up to 4 heads per unit, fixed-point split and A-fragment
// layout. With APPEND (fused step) the launch has ceil(batch x kv_heads / 2)
// more blocks, which append the new tokens, and the query blocks publish each
// sequence's length after the append.
struct QueryLds {
  float qk[DD][8];             // the 8 queries [coordinate][unit * 4 + head]
  float part[3][8][2 * DD];    // k quarters 1..3 of every row's sums
  float qv[2][8][DD];          // q_rot, q_s
  float mx[2][8];              // max |q_rot|, max |q_s| per head
  // fixed-point queries offset by QOFF: [type][head][coordinate]
  uint32_t qz[2][8][DD];
};

// Balanced base-8 digits d_k in [-4, 3] of an integer |x| <= QMAX: adding
// QOFF = sum_k 4 * 8^k (k < 8) makes them the plain base-8 digits d_k + 4 of
// x + QOFF, which lies in [0, 8^8).
constexpr int QOFF = 9586980;

// e2m3 codes of the eight digit values v - 4 (v = 0..7) scaled by f = 1, 1/2,
// 1/4 (fi = 0, 1, 2), six bits per value; sign bit 0x20, magnitude m: f = 1:
// 1 -> 0x08, 2 -> 0x10, 3 -> 0x14, 4 -> 0x18; f = 1/2: code 4m; f = 1/4: code 2m
__host__ __device__ constexpr uint64_t digit_code_table(int fi) {
  uint64_t t = 0;
  for (int v = 0; v < 8; ++v) {
    const int dv = v - 4;
    const uint32_t mag = (uint32_t)(dv < 0 ? -dv : dv);
    const uint32_t c1 = mag <= 1u ? (mag << 3) : (8u + (mag << 2));
    const uint32_t c = (fi == 0 ? c1 : (mag << (fi == 1 ? 2 : 1))) | (dv < 0 ? 0x20u : 0u);
    t |= (uint64_t)c << (6 * v);
  }
  return t;
}

template <typename QT, bool APPEND>
__global__ void __launch_bounds__(512) decode_prep_kernel(DecodeArgs a) {
  const int tid = threadIdx.x;
  const int nq = (a.streams_hg + 1) >> 1;  // query blocks
  if constexpr (APPEND) {
    if ((int)blockIdx.x >= nq) {
      __shared__ AppendLds al;
      append_pair(a, (int)blockIdx.x - nq, tid, sizeof(QT) == 2, al);
      return;
    }
  }
  __shared__ __attribute__((aligned(16))) QueryLds ql;
  int sgu[2], nhu[2], bu[2], h0u[2];
#pragma unroll
  for (int u2 = 0; u2 < 2; ++u2) {
    sgu[u2] = 2 * (int)blockIdx.x + u2;
    const int hg = sgu[u2] % a.hgroups, stream = sgu[u2] / a.hgroups;
    bu[u2] = stream / a.kv_heads;
    h0u[u2] = hg * 4;  // first virtual head of the unit
    nhu[u2] = sgu[u2] < a.streams_hg ? min(4, a.vgroup - hg * 4) : 0;
    // fused step: the sequence's length after the append, for the decode launch
    if (APPEND && tid == 0 && nhu[u2] > 0 && stream % a.kv_heads == 0 && hg == 0)
      a.wlen[bu[u2]] = min(a.seq_len[bu[u2]] + 1, a.capacity);
  }
  // thread (r, k quarter kq) owns rows r (q_rot) and r + 128 (q_s) of [Pi ; S Pi]
  // over a quarter of k: its 64 matrix entries (transposed matrix: reads coalesced
  // over r) are all requested before the queries are staged; each query broadcast
  // from LDS then serves both rows
  const int r = tid & (DD - 1), kq = tid >> 7;
  float mrow[2][32];
#pragma unroll
  for (int u = 0; u < 32; ++u) {
    mrow[0][u] = a.rs_t[(kq * 32 + u) * 2 * DD + r];
    mrow[1][u] = a.rs_t[(kq * 32 + u) * 2 * DD + DD + r];
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e = i * 512 + tid, hh = e >> 7, k = e & (DD - 1), u2 = hh >> 2;
    // virtual head vh = position qi x group + head qj of the KV head's group
    const int vh = h0u[u2] + (hh & 3), qi = vh / a.group, qj = vh - qi * a.group;
    const int kvh = (sgu[u2] / a.hgroups) % a.kv_heads;
    const QT *q = reinterpret_cast<const QT *>(a.q) +
                  (((int64_t)bu[u2] * a.n_q + qi) * a.q_heads + kvh * a.group + qj) * DD;
    ql.qk[k][hh] = (hh & 3) < nhu[u2] ? qload(q, k) : 0.f;
  }
  __syncthreads();
  // two 16-byte LDS broadcasts give the eight query entries of a k
  {
    float acc[2][8];
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
      for (int hh = 0; hh < 8; ++hh) acc[T][hh] = 0.f;
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      const float4 q0 = *reinterpret_cast<const float4 *>(&ql.qk[kq * 32 + u][0]);
      const float4 q1 = *reinterpret_cast<const float4 *>(&ql.qk[kq * 32 + u][4]);
      const float qq[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
      for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int hh = 0; hh < 8; ++hh) acc[T][hh] = fmaf(mrow[T][u], qq[hh], acc[T][hh]);
    }
    if (kq > 0) {
#pragma unroll
      for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int hh = 0; hh < 8; ++hh) ql.part[kq - 1][hh][T * DD + r] = acc[T][hh];
    }
    __syncthreads();
    if (kq == 0) {
#pragma unroll
      for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int hh = 0; hh < 8; ++hh)
          ql.qv[T][hh][r] = (acc[T][hh] + ql.part[0][hh][T * DD + r]) + (ql.part[1][hh][T * DD + r] + ql.part[2][hh][T * DD + r]);
    }
  }
  __syncthreads();
  {
    // max |.| per (type, head): wave w reduces rows (T = w >> 2, heads 2 (w & 3), +1)
    const int lane = tid & 63, w = tid >> 6, T = w >> 2;
    for (int hh = (w & 3) * 2; hh < (w & 3) * 2 + 2; ++hh) {
      const float *row = ql.qv[T][hh];
      float m = fmaxf(fabsf(row[lane]), fabsf(row[lane + 64]));
      for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
      if (lane == 0) ql.mx[T][hh] = m;
    }
  }
  __syncthreads();
  // thread (head, coordinate): the fixed-point query of both types, offset so
  // that its digits are plain base-8 digits
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e = i * 512 + tid, hh = e >> 7, j = e & (DD - 1);
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      const float m = ql.mx[T][hh];
      const int qi = m > 0.f ? (int)rintf(ql.qv[T][hh][j] * (QMAX / m)) : 0;
      ql.qz[T][hh][j] = (uint32_t)(qi + QOFF);
    }
  }
  if (tid < 16) {
    const int T = tid >> 3, hh = tid & 7, u2 = hh >> 2;
    const float m = ql.mx[T][hh];
    if (nhu[u2] > 0) a.qconst[((int64_t)sgu[u2] * 4 + (hh & 3)) * QC + T] = m > 0.f ? m / QMAX : 0.f;
  }
  __syncthreads();
  {
    // fragment (unit, T, instr, lane): the 32 codes of row (4*hh + slot), digit
    // 4*instr + slot, packed at 6 bits each (element e at bit 6e); element
    // e = 8q + i holds coordinate 32g + 4i + q, scaled by (1, 1/2, 1/4, 1/4)[q]
    constexpr uint64_t dct[3] = {digit_code_table(0), digit_code_table(1), digit_code_table(2)};
    const int u2 = tid >> 8, T = (tid >> 7) & 1, ins = (tid >> 6) & 1, Ln = tid & 63;
    const int g = Ln >> 4, row = Ln & 15, hh = u2 * 4 + (row >> 2), dig = 4 * ins + (row & 3);
    if (nhu[u2] > 0) {
      const uint4 *src = reinterpret_cast<const uint4 *>(&ql.qz[T][hh][32 * g]);
      const uint32_t sh = 3 * dig;
      uint32_t dw[6] = {0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint4 z4 = src[i];
        const uint32_t zq[4] = {z4.x, z4.y, z4.z, z4.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t v = (zq[q] >> sh) & 7u;
          const uint32_t code = (uint32_t)(dct[q < 2 ? q : 2] >> (6 * v)) & 63u;
          const int bit = 6 * (8 * q + i);
          dw[bit >> 5] |= code << (bit & 31);
          if ((bit & 31) > 26) dw[(bit >> 5) + 1] |= code >> (32 - (bit & 31));
        }
      }
      uint4 *dst = reinterpret_cast<uint4 *>(a.qfrag + ((((int64_t)sgu[u2] * 2 + T) * 2 + ins) * 64 + Ln) * 8);
      dst[0] = make_uint4(dw[0], dw[1], dw[2], dw[3]);
      dst[1] = make_uint4(dw[4], dw[5], 0u, 0u);
    }
  }
}


// Key B operand of a 32-coordinate plane word: element 8q + i (nibble i of
// dword q) is bit 4i + q of w as a 0/1 fp4 value scaled by 0.5, 1, 2, 2 for
// q = 0..3 (the A digits carry the inverse factors).
__device__ __forceinline__ i8v mask_fp4_01(uint32_t w) {
  i8v b;
  b[0] = (int)(w & 0x11111111u);
  b[1] = (int)(w & 0x22222222u);
  b[2] = (int)(w & 0x44444444u);
  b[3] = (int)((w >> 1) & 0x44444444u);
  b[4] = b[5] = b[6] = b[7] = 0;
  return b;
}




// One block of 256 MG threads per (stream, head group): log-sum-exp merge of the
// chunk partials, then o = Pi^T o_rot. The Pi entries of the inverse rotation
// are requested first; the chunks are split over MG thread groups, each of
// which sums its chunks in one pass against its own running maximum, and the
// group sums are combined against the overall maximum. Up to 16 chunks take two
// groups (512 threads: measured 0.7 us faster per serving call than four);
// longer contexts take four, so that each group's pass stays short.
template <int MG>
__global__ void __launch_bounds__(256 * MG) decode_merge_kernel(DecodeArgs a) {
  constexpr int CB = 4, NT = 256 * MG, KS = NT / DD, KR = DD / KS;  // KS slices of KR rows of Pi
  __shared__ float gm[MG][4], gl[MG][4];
  __shared__ float po[MG][4][DD];
  __shared__ float orot[4][DD];
  __shared__ float pk[KS][4][DD];
  const int tid = threadIdx.x, lane = tid & 63;
  const int sg = blockIdx.x;
  const int hg = sg % a.hgroups, stream = sg / a.hgroups;
  const int b = stream / a.kv_heads, kvh = stream % a.kv_heads;
  const int nh = min(4, a.vgroup - hg * 4);
  // fused step: the appended token is now part of every stream of sequence b
  if (a.len_inc && tid == 0 && hg == 0 && stream % a.kv_heads == 0 && a.len_inc[b] < a.capacity) a.len_inc[b] += 1;
  // thread (coordinate j, k slice kg) of the inverse rotation: column j of Pi, rows KR kg .. KR kg + KR - 1
  const int j = tid & (DD - 1), kg = tid >> 7;
  float rk[KR];
#pragma unroll
  for (int u = 0; u < KR; ++u) rk[u] = a.rot[(kg * KR + u) * DD + j];
  const int cg = tid >> 8, hh = (tid >> 6) & 3;  // chunk group, head (one wave per pair)
  const int nc = a.nchunks;
  const float *p = a.partial + ((int64_t)stream * a.vgroup + hg * 4 + min(hh, nh - 1)) * nc * (DD + 2);
  // chunks c = cg (mod MG); lane owns coordinates lane and lane + 64
  float m = -INFINITY, L = 0.f, O0 = 0.f, O1 = 0.f;
  for (int c0 = cg; c0 < nc; c0 += MG * CB) {
    float mv[CB], lv[CB], o0[CB], o1[CB];
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const int c = min(c0 + u * MG, nc - 1);
      const float *pc = p + (int64_t)c * (DD + 2);
      mv[u] = c0 + u * MG < nc ? pc[DD] : -INFINITY;
      lv[u] = pc[DD + 1];
      o0[u] = pc[lane];
      o1[u] = pc[lane + 64];
    }
    float mn = m;
#pragma unroll
    for (int u = 0; u < CB; ++u) mn = fmaxf(mn, mv[u]);
    // what is summed so far moves to the new maximum (nothing is summed while m = -inf)
    const float s = m == -INFINITY ? 0.f : exp2f(m - mn);
    L *= s;
    O0 *= s;
    O1 *= s;
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const float f = mv[u] == -INFINITY ? 0.f : exp2f(mv[u] - mn);
      L = fmaf(f, lv[u], L);
      O0 = fmaf(f, o0[u], O0);
      O1 = fmaf(f, o1[u], O1);
    }
    m = mn;
  }
  po[cg][hh][lane] = O0;
  po[cg][hh][lane + 64] = O1;
  if (lane == 0) {
    gm[cg][hh] = m;
    gl[cg][hh] = L;
  }
  __syncthreads();
  if (tid < 4 * DD) {
    const int h = tid >> 7, jj = tid & (DD - 1);
    float M = gm[0][h];
#pragma unroll
    for (int g = 1; g < MG; ++g) M = fmaxf(M, gm[g][h]);
    float Lh = 0.f, Oh = 0.f;
#pragma unroll
    for (int g = 0; g < MG; ++g) {
      const float w = gm[g][h] == -INFINITY ? 0.f : exp2f(gm[g][h] - M);
      Lh = fmaf(w, gl[g][h], Lh);
      Oh = fmaf(w, po[g][h][jj], Oh);
    }
    orot[h][jj] = (h < nh && Lh > 0.f) ? Oh / Lh : 0.f;
  }
  __syncthreads();
  // o = Pi^T o_rot: k split in KS slices
  {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < KR; ++u) {
#pragma unroll
      for (int h = 0; h < 4; ++h) acc[h] = fmaf(rk[u], orot[h][kg * KR + u], acc[h]);
    }
#pragma unroll
    for (int h = 0; h < 4; ++h) pk[kg][h][j] = acc[h];
  }
  __syncthreads();
  if (tid < 4 * DD) {
    const int h = tid >> 7, jo = tid & (DD - 1);
    if (h < nh) {
      float o = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s) o += pk[s][h][jo];
      // virtual head -> (query position qi, head qj of the group)
      const int vh = hg * 4 + h, qi = vh / a.group, qj = vh - qi * a.group;
      a.out[(((int64_t)b * a.n_q + qi) * a.q_heads + kvh * a.group + qj) * DD + jo] = o;
    }
  }
}

static void launch_decode_merge(const DecodeArgs &a, unsigned blocks, hipStream_t st) {
  if (a.nchunks <= 16) hipLaunchKernelGGL(decode_merge_kernel<2>, dim3(blocks), dim3(512), 0, st, a);
  else hipLaunchKernelGGL(decode_merge_kernel<4>, dim3(blocks), dim3(1024), 0, st, a);
}

// first record of span si (uniform) of a decode chunk
__device__ __forceinline__ int64_t pick_span(int si, int64_t r0, int64_t r1, int64_t r2, int64_t r3) {
  return si == 0 ? r0 : si == 1 ? r1 : si == 2 ? r2 : r3;
}

// KB MSE bits of the keys (0: pure QJL keys), QJL: the keys carry the sign word
// and |r| (false: MSE-only keys)
// SPANS: the chunk's records come in several runs (pages smaller than the chunk);
// NF16: the cache's norms are fp16; EXT: the logits come from a.ext (keys in
// another format, scored beforehand), the values from the cache
// LOGITS (measurement): the work-group writes the logits of its chunk (scale * s,
// natural units) to a.logit_out after the key phase and stops there.
template <int KB, int VB, bool QJL, bool SPANS, bool NF16, bool EXT = false, bool LOGITS = false>
__global__ void __launch_bounds__(256) decode_kernel(DecodeArgs a) {
  constexpr int KM = KB > 0 ? 1 << (KB - 1) : 0;  // key Walsh masks
  constexpr int KQ = QJL ? 1 : 0;
  constexpr int NPL = KB + KQ;  // words per 32-coordinate group of a key record
  constexpr int VM = 1 << (VB - 1);  // value Walsh masks
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float *lg = reinterpret_cast<float *>(smem);                   // [4][chunk] logits (log2 units)
  float *vnl = lg + 4 * a.chunk;                                 // [chunk] value norms
  int8_t *av = reinterpret_cast<int8_t *>(smem + 5 * a.chunk * 4);  // [chunk/128][2][64][16] value A fragments
  __shared__ float red[4], lred[4][4];
  __shared__ float hmax[4], hsum[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar loop control
  // 1-D grid of nchunks x (streams x head groups) work-groups. Work-groups are
  // dealt to the 8 XCDs round-robin by id; when the stream count is a multiple
  // of 8, id -> (stream, chunk) keeps every chunk of a stream on one XCD and
  // close together in time, so its query fragments are fetched into one L2 once
  // (chunk-major order measured 1.085x the algorithmic bytes: the fragments were
  // evicted between a stream's chunks).
  // Many query heads per KV stream: the head groups of one (stream, chunk) are
  // consecutive on one XCD, so its records are read from HBM once and reused
  // from that L2. The last chunk of every stream (usually partial: a few tokens
  // past a multiple of the chunk) is dealt after all the others, on the same XCD
  // as the stream's other chunks, so the launch ends on short work-groups
  // (measured 5% off a decode call whose streams end 64 tokens past a chunk).
  const int HG = a.hgroups;
  int c, hg, stream;
  {
    const int id0 = blockIdx.x;
    const int nf = a.nchunks - 1;  // chunks dealt first; the last chunks go at the end
    const int F = nf * a.streams_hg;
    const bool last = id0 >= F;
    const int id = last ? id0 - F : id0;
    const int ncs = last ? 1 : nf;
    if ((a.kv_streams & 7) == 0) {
      const int k = id >> 3, k2 = k / HG;
      hg = k - k2 * HG;
      c = last ? nf : k2 % ncs;
      stream = (k2 / ncs) * 8 + (id & 7);
    } else {
      const int k2 = id / HG;
      hg = id - k2 * HG;
      c = last ? nf : k2 % ncs;
      stream = k2 / ncs;
    }
  }
  const int sg = stream * HG + hg;
  const int b = stream / a.kv_heads;
  const int nh = min(4, a.vgroup - hg * 4);
  // a length outside [0, capacity] (a caller error) is clamped: no record outside the stream is read;
  // EXT logits exist for the first ext_stride tokens only
  const int len = min(max(a.wlen ? a.wlen[b] : a.seq_len[b], 0), EXT ? min(a.capacity, (int)a.ext_stride) : a.capacity);
  const int t0 = c * a.chunk;
  const int t1 = min(len, t0 + a.chunk);
  // visible tokens of virtual head hh (chunk-relative; causal: up to its position)
  auto vis = [&](int hh) {
    const int qi = (hg * 4 + hh) / a.group;
    const int lim = a.causal ? len - a.n_q + qi + 1 : len;
    return min(max(lim - t0, 0), t1 - t0);
  };
  float *part_base = a.partial;
  auto part = [&](int hh) {
    return part_base + (((int64_t)stream * a.vgroup + hg * 4 + hh) * a.nchunks + c) * (DD + 2);
  };

  if (t0 >= t1) {
    for (int e = tid; e < nh * (DD + 2); e += 256) {
      const int hh = e / (DD + 2), j = e % (DD + 2);
      part(hh)[j] = (j == DD) ? -INFINITY : 0.f;
    }
  } else {
    const int n = t1 - t0;
    // the chunk's records come in spans of 2^span_lg consecutive positions: one
    // span, or (pages smaller than the chunk) up to four pages; rs0..rs3 are the
    // spans' first records, picked per tile or value group by a uniform index
    const int slg = a.span_lg;
    const uint32_t smask = (1u << slg) - 1u;
    const int64_t rs0 = a.map.rec(stream, t0);
    int64_t rs1 = rs0, rs2 = rs0, rs3 = rs0;
    if (SPANS) {
      if ((1 << slg) < n) rs1 = a.map.rec(stream, t0 + (1 << slg));
      if ((2 << slg) < n) rs2 = a.map.rec(stream, t0 + (2 << slg));
      if ((3 << slg) < n) rs3 = a.map.rec(stream, t0 + (3 << slg));
    }
    const float *wk = a.tables->walsh[KB > 0 ? KB : 1];
    const float *wv = a.tables->walsh[VB];
    const int ngrp = (n + 127) >> 7;
    const int tn = lane & 15, G = lane >> 4;  // MFMA column (token), row group (head)
    float vmx = 0.f, lmx = -INFINITY;
    if constexpr (EXT) {
      // ---- phase K from logits computed beforehand (log2 units, [unit][4][ext_stride]) ----
      const float *lgx = a.ext + (int64_t)sg * 4 * a.ext_stride + t0;
      const float *vnx = reinterpret_cast<const float *>(a.vnorm) + rs0;
      const int vis0 = vis(0), vis1 = vis(1), vis2 = vis(2), vis3 = vis(3);
      float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      // a thread's tokens tid + 256 k (k < 4: n <= chunk <= 1024): every load first
      const int vh[4] = {vis0, vis1, vis2, vis3};
      float vv[4], xl[4][4];
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const int tc = tid + 256 * k4;
        vv[k4] = tc < n ? vnx[tc] : 0.f;
#pragma unroll
        for (int h = 0; h < 4; ++h)
          xl[k4][h] = (h < nh && tc < vh[h]) ? lgx[(int64_t)h * a.ext_stride + tc] : -INFINITY;
      }
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const int tc = tid + 256 * k4;
        if (tc < n) {
          vnl[tc] = vv[k4];
          vmx = fmaxf(vmx, vv[k4]);
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            lg[h * a.chunk + tc] = xl[k4][h];
            m4[h] = fmaxf(m4[h], xl[k4][h]);
          }
        }
      }
#pragma unroll
      for (int h = 0; h < 4; ++h)
        for (int off = 32; off > 0; off >>= 1) m4[h] = fmaxf(m4[h], __shfl_xor(m4[h], off));
      lmx = G == 0 ? m4[0] : G == 1 ? m4[1] : G == 2 ? m4[2] : m4[3];  // the row-group layout below
    } else {
      // records of the chunk. Contiguous caches: buffer loads (below). Pages
      // smaller than the chunk: uniform bases (the tile's span) and unsigned 32-bit
      // byte offsets per lane (base + zero-extended offset addressing), key words
      // loaded non-temporally; lanes past the end re-read token n-1. Either way
      // every store below stays unconditional and harmless (tokens past n get -inf
      // logits)
      const uint32_t kgo = (uint32_t)(G * NPL * 4);  // the lane's 32-coordinate group in a record
      struct KBuf {
        uint32_t pl[KTPW][NPL];
        float2 kn[KTPW];  // (|k|, |r|); MSE-only keys: (|k|, 0)
        float vn[KTPW];
        uint32_t tc[KTPW];
      };
      // contiguous records: range-checked buffer loads. Each round builds its
      // descriptors at the round's first token t16 with num_records covering
      // only the chunk's records from there on (max(n - t16, 0)), so the whole
      // offset of a load is its lane offset, which the hardware compares with
      // num_records: a load past the chunk's n records returns zeros and
      // touches no memory (those tokens' logits are masked and their value
      // norms 0). The scalar offset is not range-checked, so it stays 0. The
      // descriptors are scalar work; the lane offsets are loop-invariant. The
      // loads are non-temporal (aux 2: the nt policy): the key records stream
      // through once (measured 0.58 -> 0.63 of HBM peak on the serving step;
      // the value blocks read the same way measured slower, so they keep the
      // default policy)
      constexpr int NB = NF16 ? 2 : 4;  // bytes per norm
      constexpr int RB = DW * NPL * 4;  // bytes per key record
      auto kload = [&](int base, KBuf &bf) {
        if constexpr (!SPANS) {
          const int t16 = __builtin_amdgcn_readfirstlane(base * 16);  // the round's first token (uniform)
          const int rem = max(n - t16, 0);                             // the chunk's records from t16 on
          const int64_t r0 = rs0 + t16;
          const __amdgpu_buffer_rsrc_t rkb = __builtin_amdgcn_make_buffer_rsrc(
              const_cast<uint32_t *>(a.kbits) + r0 * DW * NPL, (short)0, rem * RB, 0x00020000);
          const __amdgpu_buffer_rsrc_t rkn = __builtin_amdgcn_make_buffer_rsrc(
              reinterpret_cast<char *>(const_cast<void *>(a.knorm)) + (1 + KQ) * r0 * NB, (short)0,
              rem * (1 + KQ) * NB, 0x00020000);
          const __amdgpu_buffer_rsrc_t rvn = __builtin_amdgcn_make_buffer_rsrc(
              reinterpret_cast<char *>(const_cast<void *>(a.vnorm)) + r0 * NB, (short)0, rem * NB, 0x00020000);
#pragma unroll
          for (int u = 0; u < KTPW; ++u) {
            const uint32_t tl = (uint32_t)(u * 16 + tn);  // token of the lane, relative to t16
            bf.tc[u] = (uint32_t)t16 + tl;
            buffer_load_words<NPL, 2>(rkb, tl * RB + kgo, bf.pl[u]);
            if constexpr (NF16) {
              if constexpr (QJL) {
                const uint32_t h2 = __builtin_amdgcn_raw_buffer_load_b32(rkn, tl * 4u, 0, 2);
                bf.kn[u] = make_float2(__half2float(__ushort_as_half((unsigned short)(h2 & 0xFFFFu))),
                                       __half2float(__ushort_as_half((unsigned short)(h2 >> 16))));
              } else {
                bf.kn[u] = make_float2(
                    __half2float(__ushort_as_half(__builtin_amdgcn_raw_buffer_load_b16(rkn, tl * 2u, 0, 2))), 0.f);
              }
              bf.vn[u] = __half2float(__ushort_as_half(__builtin_amdgcn_raw_buffer_load_b16(rvn, tl * 2u, 0, 2)));
            } else {
              if constexpr (QJL) {
                const auto k2 = __builtin_amdgcn_raw_buffer_load_b64(rkn, tl * 8u, 0, 2);
                bf.kn[u] = make_float2(__uint_as_float(k2[0]), __uint_as_float(k2[1]));
              } else {
                bf.kn[u] = make_float2(__uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rkn, tl * 4u, 0, 2)), 0.f);
              }
              bf.vn[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rvn, tl * 4u, 0, 2));
            }
          }
          return;
        }
#pragma unroll
        for (int u = 0; u < KTPW; ++u) {
          const uint32_t tc = (uint32_t)min((base + u) * 16 + tn, n - 1);
          bf.tc[u] = tc;
          // a tile lies in one span
          const int64_t rr = SPANS ? pick_span(min((base + u) * 16, n - 1) >> slg, rs0, rs1, rs2, rs3) : rs0;
          const char *kb0 = reinterpret_cast<const char *>(a.kbits + rr * DW * NPL);
          const char *kn0 = reinterpret_cast<const char *>(a.knorm) + (1 + KQ) * rr * NB;
          const char *vn0 = reinterpret_cast<const char *>(a.vnorm) + rr * NB;
          const uint32_t tl = SPANS ? tc & smask : tc;  // position in the span
          const char *src = kb0 + (tl * (uint32_t)(DW * NPL * 4) + kgo);
          if constexpr (NPL == 4) {
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
            const u32x4 w4 = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src));
            bf.pl[u][0] = w4[0]; bf.pl[u][1] = w4[1]; bf.pl[u][2] = w4[2]; bf.pl[u][3] = w4[3];
          } else {
#pragma unroll
            for (int p = 0; p < NPL; ++p) bf.pl[u][p] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(src) + p);
          }
          if constexpr (NF16) {
            if constexpr (QJL) bf.kn[u] = __half22float2(*reinterpret_cast<const __half2 *>(kn0 + (tl << 2)));
            else bf.kn[u] = make_float2(__half2float(*reinterpret_cast<const __half *>(kn0 + (tl << 1))), 0.f);
            bf.vn[u] = __half2float(*reinterpret_cast<const __half *>(vn0 + (tl << 1)));
          } else {
            if constexpr (QJL) bf.kn[u] = *reinterpret_cast<const float2 *>(kn0 + (tl << 3));
            else bf.kn[u] = make_float2(*reinterpret_cast<const float *>(kn0 + (tl << 2)), 0.f);
            bf.vn[u] = *reinterpret_cast<const float *>(vn0 + (tl << 2));
          }
        }
      };
      // the wave's first key tiles are requested before anything else
      KBuf kb_a, kb_b;
      kload(wave * KTPW, kb_a);
      // ---- phase K: logits of all tokens of the chunk (log2 units) ----
      const uint32_t *qf = a.qfrag + (int64_t)sg * 2 * 2 * 64 * 8;
      auto ldfrag = [&](int T, int ins) {
        const uint4 *p = reinterpret_cast<const uint4 *>(qf + ((T * 2 + ins) * 64 + lane) * 8);
        const uint4 x = p[0], y = p[1];
        i8v v;
        v[0] = (int)x.x; v[1] = (int)x.y; v[2] = (int)x.z; v[3] = (int)x.w;
        v[4] = (int)y.x; v[5] = (int)y.y; v[6] = 0; v[7] = 0;
        return v;
      };
      const i8v aqr0 = ldfrag(0, 0), aqr1 = ldfrag(0, 1), aqs0 = ldfrag(1, 0), aqs1 = ldfrag(1, 1);
      const int sc0 = 127 + 3 * (lane & 3), sc1 = sc0 + 12;  // e8m0 row scales 2^(3 digit)
      const float *qc = a.qconst + ((int64_t)sg * 4 + G) * QC;
      // accumulator start -sum_j Q_j per digit slot: the A fragments against an
      // all-ones mask (B scale 2^1 undoes the 1/2 of every product), exact
      f4v init_r = {0.f, 0.f, 0.f, 0.f}, init_s = {0.f, 0.f, 0.f, 0.f};
      {
        const i8v ones = mask_fp4_01(0xFFFFFFFFu);
        const f4v z = {0.f, 0.f, 0.f, 0.f};
        if constexpr (KM > 0) {
          init_r = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aqr0, ones, z, 2, 4, 0, sc0, 0, 128);
          init_r = -__builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aqr1, ones, init_r, 2, 4, 0, sc1, 0, 128);
        }
        if constexpr (QJL) {
          init_s = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aqs0, ones, z, 2, 4, 0, sc0, 0, 128);
          init_s = -__builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aqs1, ones, init_s, 2, 4, 0, sc1, 0, 128);
        }
      }
      // logit (log2 units) = |k| (sum_S wr_S T_S + qs |r| T_QJL) with the query units,
      // the softmax scale and the QJL constant folded into the per-lane weights
      const float sr = qc[0] * a.scale_log2, qs = qc[1] * a.qjl_scale * a.scale_log2;
      float wkr[KM > 0 ? KM : 1];
#pragma unroll
      for (int mi = 0; mi < KM; ++mi) wkr[mi] = wk[mi] * sr;
      const int ntile = (n + 15) >> 4;
      const int visG = vis(G);  // tokens of the chunk this lane's virtual head sees
      auto kcompute = [&](int base, const KBuf &cur) {
        (void)base;
#pragma unroll
        for (int u = 0; u < KTPW; ++u) {
          const int tc = (int)cur.tc[u];
          // all masked sums first (independent accumulators keep the MFMA pipe busy):
          // the KM Walsh masks of the codes, then the sign word's mask
          f4v acc[KM + KQ];
          i8v sm[KB > 0 ? KB : 1];
#pragma unroll
          for (int p = 0; p < KB; ++p) sm[p] = mask_fp4_01(cur.pl[u][p]);
#pragma unroll
          for (int mi = 0; mi < KM + KQ; ++mi) {
            const i8v bm = mi < KM ? walsh_fp4(sm, walsh_mask(KB, mi)) : mask_fp4_01(cur.pl[u][NPL - 1]);
            acc[mi] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(mi < KM ? aqr0 : aqs0, bm, mi < KM ? init_r : init_s,
                                                                       2, 4, 0, sc0, 0, 129);
            acc[mi] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(mi < KM ? aqr1 : aqs1, bm, acc[mi], 2, 4, 0, sc1,
                                                                       0, 129);
          }
          float code = 0.f;
#pragma unroll
          for (int mi = 0; mi < KM; ++mi) code += wkr[mi] * ((acc[mi][0] + acc[mi][1]) + (acc[mi][2] + acc[mi][3]));
          float s;
          if constexpr (QJL) {
            const float Ts = (acc[KM][0] + acc[KM][1]) + (acc[KM][2] + acc[KM][3]);
            s = cur.kn[u].x * fmaf(cur.kn[u].y * Ts, qs, code);
          } else {
            s = cur.kn[u].x * code;
          }
          s = tc < visG ? s : -INFINITY;  // causal mask of this lane's virtual head
          if constexpr (LOGITS) {
            if (tc < visG && G < nh) {
              const int vh = hg * 4 + G, qi = vh / a.group, qj = vh - qi * a.group;
              const int kvh = stream - b * a.kv_heads;
              a.logit_out[(((int64_t)b * a.n_q + qi) * a.q_heads + kvh * a.group + qj) * a.logit_stride + t0 + tc] =
                  s * 0.69314718055994531f;  // log2 units -> natural
            }
          }
          lg[G * a.chunk + tc] = s;
          lmx = fmaxf(lmx, s);
          vnl[tc] = cur.vn[u];
          vmx = fmaxf(vmx, cur.vn[u]);
        }
      };
      // two buffers in turn: the next round's loads are in flight during this one.
      // The loads are unconditional (tiles past the end read zeros, or re-read token
      // n-1 with spans) and pinned ahead of the compute, so their latency overlaps a
      // whole round.
      constexpr int KSTEP = 4 * KTPW;
      int kbase = wave * KTPW;
      while (kbase < ntile) {
        kload(kbase + KSTEP, kb_b);
        __builtin_amdgcn_sched_barrier(0);
        kcompute(kbase, kb_a);
        kbase += KSTEP;
        if (kbase >= ntile) break;
        kload(kbase + KSTEP, kb_a);
        __builtin_amdgcn_sched_barrier(0);
        kcompute(kbase, kb_b);
        kbase += KSTEP;
      }
      if constexpr (LOGITS) return;  // every wave of the work-group, before any barrier
    }
    // the softmax reads rounds of 256 tokens: positions from n to the end of the last
    // round get -inf logits and zero norms (the key phase may write the same values to
    // some of them), so every token's weight comes out of exp2 without a select
    for (int t = n + tid; t < ((n + 255) & ~255); t += 256) {
#pragma unroll
      for (int h = 0; h < 4; ++h) lg[h * a.chunk + t] = -INFINITY;
      vnl[t] = 0.f;
    }
    // the first value blocks are requested before the softmax
    const int vn = lane & 15, vg = lane >> 4;  // coordinate column, token block in the 128-token group
    struct VBuf {
      uint32_t pl[VGPI][2][VB];
    };
    // blocks of the chunk from a uniform base (the group's span); a block past the
    // end re-reads the last one (its tokens carry zero weights)
    const int lastblk = (n - 1) >> 5;
    const uint32_t vco = (uint32_t)((wave * 32 + vn) * VB * 4);  // the lane's coordinate in a block
    auto vload = [&](int grp0, VBuf &bf) {
#pragma unroll
      for (int gi = 0; gi < VGPI; ++gi) {
        // this lane's 32-token block, chunk-relative; a 128-token group lies in one span
        const uint32_t blk = (uint32_t)min((grp0 + gi) * 4 + vg, lastblk);
        const int64_t rr = SPANS ? pick_span((min((grp0 + gi) * 4, lastblk) * 32) >> slg, rs0, rs1, rs2, rs3) : rs0;
        const char *vb0 = reinterpret_cast<const char *>(a.vbits + (rr >> 5) * DD * VB);
        const char *src = vb0 + ((SPANS ? blk & (smask >> 5) : blk) * (uint32_t)(DD * VB * 4) + vco);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int p = 0; p < VB; ++p)
            bf.pl[gi][nt][p] = reinterpret_cast<const uint32_t *>(src + nt * 16 * VB * 4)[p];
      }
    };
    VBuf vb_a, vb_b;
    vload(0, vb_a);
    // chunk maxima: |v| over all lanes; logits per head (lanes of one row group)
    for (int off = 32; off > 0; off >>= 1) vmx = fmaxf(vmx, __shfl_xor(vmx, off));
    for (int off = 8; off > 0; off >>= 1) lmx = fmaxf(lmx, __shfl_xor(lmx, off));
    if (lane == 0) red[wave] = vmx;
    if (tn == 0) lred[wave][G] = lmx;
    __syncthreads();
    const float vmax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    // ---- softmax: wave w owns head w; weights -> fixed-point value digits ----
    // (the wave of an absent head writes zero weights: every value A byte that
    // phase V reads is written here, so the fragments need no clearing)
    {
      // a head that sees no token of the chunk has m = -inf: it is taken as 0 here, so
      // that every exp2 below is 0 rather than NaN (the partial keeps -inf)
      const float mh = fmaxf(fmaxf(lred[0][wave], lred[1][wave]), fmaxf(lred[2][wave], lred[3][wave]));
      const float m = mh == -INFINITY ? 0.f : mh;
      // token t = lane + 64 i: q = t & 7 = lane & 7 is fixed per lane, and so is
      // its weight scale 2^(29 - q) / vmax (negated for q = 7, whose B byte is -128)
      const int qv = lane & 7;
      const float wq = vmax > 0.f ? ldexpf(WSCALE / vmax, -qv) * (qv == 7 ? -1.f : 1.f) : 0.f;
      // token t lands in fragment byte
      //   (i>>1)*2048 + ins*1024 + gg*256 + head*64 + qq*4 + bb, with q = t&7, ins = q>>2,
      //   qq = q&3, bb = (t>>3)&3, gg = (t>>5)&3: the lane-dependent part is fixed.
      const int lbase = (((lane >> 2) & 1) << 10) | (((lane >> 5) & 1) << 8) | (wave << 6) | ((lane & 3) << 2) |
                        ((lane >> 3) & 3);
      // four independent iterations per round (tokens t = lane + 64 i); rounds run to
      // a multiple of 256 tokens, inside the chunk's LDS. Tokens past n and tokens the
      // head does not see (causal mask) hold -inf logits, so p = W = 0 for them. The
      // rows of an absent head (wave >= nh) get weights that nothing reads.
      float l = 0.f;
      const float *lgw = lg + wave * a.chunk + lane;
      const float *vnw = vnl + lane;
      const int nit = (n + 63) >> 6;
      for (int i0 = 0; i0 < nit; i0 += 4) {
        // the round's LDS reads first, then branch-free arithmetic
        float lv[4], nv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          lv[j] = lgw[64 * (i0 + j)];
          nv[j] = vnw[64 * (i0 + j)];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float e = __builtin_amdgcn_exp2f(lv[j] - m);  // <= 1; 0 for a -inf logit
          l += e;
          // fixed point by truncation: an error below one unit of 2^-29 of the largest weight
          const int W = (int)(e * nv[j] * wq);
          const uint32_t x = ((uint32_t)W + 0x80808080u) ^ 0x80808080u;  // four signed base-256 digits
          int8_t *dst = av + lbase + ((i0 >> 1) << 11) + ((j >> 1) << 11) + ((j & 1) << 9);
          dst[0] = (int8_t)x;
          dst[16] = (int8_t)(x >> 8);
          dst[32] = (int8_t)(x >> 16);
          dst[48] = (int8_t)(x >> 24);
        }
      }
      for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off);
      if (lane == 0) {
        hmax[wave] = mh;
        hsum[wave] = l;
      }
    }
    __syncthreads();

    // ---- phase V: value sums on MFMA; wave w owns coordinates 32w .. 32w+31 ----
    i4v accv[2][VM];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int mi = 0; mi < VM; ++mi) accv[nt][mi] = i4v{0, 0, 0, 0};
    // the same sums against an all-ones mask: per (head, digit) the effective weight
    // total sum_t W_t 2^q (the -sum_t term of every Walsh mask), exact in int32
    i4v accw = i4v{0, 0, 0, 0};
    i4v ones_lo, ones_hi;
    mask_bytes_pow2(0xFFFFFFFFu, ones_lo, ones_hi);
    auto vcompute = [&](int grp0, const VBuf &vcur) {
#pragma unroll
      for (int gi = 0; gi < VGPI; ++gi) {
        const int grp = grp0 + gi;
        if (grp >= ngrp) break;
        const i4v a0 = *reinterpret_cast<const i4v *>(av + ((grp * 2 + 0) * 64 + lane) * 16);
        const i4v a1 = *reinterpret_cast<const i4v *>(av + ((grp * 2 + 1) * 64 + lane) * 16);
        accw = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, ones_lo, accw, 0, 0, 0);
        accw = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, ones_hi, accw, 0, 0, 0);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
          for (int mi = 0; mi < VM; ++mi) {
            i4v lo, hi;
            mask_bytes_pow2(xor_planes(vcur.pl[gi][nt], walsh_mask(VB, mi)), lo, hi);
            accv[nt][mi] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, lo, accv[nt][mi], 0, 0, 0);
            accv[nt][mi] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, hi, accv[nt][mi], 0, 0, 0);
          }
        }
      }
    };
    // two buffers in turn, unconditional loads pinned ahead of the compute (blocks
    // past the end re-read the last one)
    int vbase = 0;
    while (vbase < ngrp) {
      vload(vbase + VGPI, vb_b);
      __builtin_amdgcn_sched_barrier(0);
      vcompute(vbase, vb_a);
      vbase += VGPI;
      if (vbase >= ngrp) break;
      vload(vbase + VGPI, vb_a);
      __builtin_amdgcn_sched_barrier(0);
      vcompute(vbase, vb_b);
      vbase += VGPI;
    }
    // flush: lane (coordinate vn, head vg) holds digits 0..3 of every mask sum.
    // The digit sums (|x| < 2^24) convert exactly; the base-256 combination and
    // 2 M - W are rounded in fp32: the error of a partial is a few units of 2^-24
    // of sum_t p_t |v_t| (relative to the partial's own sum l, at most 2^-22 of the
    // chunk's largest |v|), far below the attention tolerance
    if (vg < nh) {
      auto digits = [](const i4v &x) {
        return fmaf(16777216.f, (float)x[3], fmaf(65536.f, (float)x[2], fmaf(256.f, (float)x[1], (float)x[0])));
      };
      const float W = digits(accw);
      const float unit = vmax * (1.f / WSCALE);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        float o = 0.f;
#pragma unroll
        for (int mi = 0; mi < VM; ++mi) o = fmaf(wv[mi], fmaf(2.f, digits(accv[nt][mi]), -W), o);
        part(vg)[wave * 32 + nt * 16 + vn] = o * unit;
      }
    }
    if (tid < nh) {
      part(tid)[DD] = hmax[tid];
      part(tid)[DD + 1] = hsum[tid];
    }
  }
}

RecMap cache_map(const tq_kv_cache *cache, int64_t oo) {
  RecMap m;
  m.oo = oo;
  if (cache->d_block_table == nullptr) {
    m.os = cache->capacity;
    return m;
  }
  m.table = cache->d_block_table;
  m.page_tokens = cache->page_tokens;
  m.heads = cache->kv_heads;
  m.cols = cache->capacity / cache->page_tokens;
  m.npages = (int32_t)(cache->k.n / ((int64_t)cache->kv_heads * cache->page_tokens));
  return m;
}

size_t decode_ws_bytes(const tq_ctx *ctx, const tq_kv_cache *cache, int32_t q_heads, int *chunk_out,
                       int *nchunks_out, int n_q) {
  const int group = q_heads / cache->kv_heads;
  const int hgroups = (group * n_q + 3) / 4;
  const int maxlen = cache->host_max_len > 0 ? cache->host_max_len : cache->capacity;
  const int64_t streams = (int64_t)cache->batch * cache->kv_heads * hgroups;
  int chunk = 1024;
  while (chunk > 256 && streams * ((maxlen + chunk - 1) / chunk) < 2048) chunk >>= 1;
  // paged cache: pages either hold whole chunks or tile them (a chunk spans at
  // most four pages of 256 or 512 tokens); other page sizes take the largest
  // chunk that divides the page
  if (cache->d_block_table)
    while ((cache->page_tokens % chunk) != 0 && (chunk % cache->page_tokens) != 0) chunk >>= 1;
  const int nchunks = std::max(1, (maxlen + chunk - 1) / chunk);
  if (chunk_out) *chunk_out = chunk;
  if (nchunks_out) *nchunks_out = nchunks;
  size_t b = 0;
  b += (size_t)streams * 2 * 2 * 64 * 32;  // qfrag (fp6 fragments, 8 dwords per lane)
  b = (b + 255) & ~(size_t)255;
  b += (size_t)streams * 4 * QC * sizeof(float);  // qconst
  b = (b + 255) & ~(size_t)255;
  b += (size_t)cache->batch * q_heads * n_q * nchunks * (DD + 2) * sizeof(float);  // partials
  b = (b + 255) & ~(size_t)255;
  b += (size_t)cache->batch * sizeof(int32_t);  // fused step: lengths after the append
  (void)ctx;
  return b;
}

template <int KB, int VB, bool QJL>
static hipError_t launch_decode_kv(const DecodeArgs &a, dim3 grid, size_t shm, hipStream_t st) {
  const bool spans = a.chunk > (1 << a.span_lg);
  if (a.logit_out) {  // measurement: logits only (contiguous caches)
    if (spans) return hipErrorInvalidValue;
    if (a.nf16) hipLaunchKernelGGL((decode_kernel<KB, 1, QJL, false, true, false, true>), grid, dim3(256), shm, st, a);
    else hipLaunchKernelGGL((decode_kernel<KB, 1, QJL, false, false, false, true>), grid, dim3(256), shm, st, a);
    return hipGetLastError();
  }
  if (a.nf16) {
    if (spans) hipLaunchKernelGGL((decode_kernel<KB, VB, QJL, true, true>), grid, dim3(256), shm, st, a);
    else hipLaunchKernelGGL((decode_kernel<KB, VB, QJL, false, true>), grid, dim3(256), shm, st, a);
  } else {
    if (spans) hipLaunchKernelGGL((decode_kernel<KB, VB, QJL, true, false>), grid, dim3(256), shm, st, a);
    else hipLaunchKernelGGL((decode_kernel<KB, VB, QJL, false, false>), grid, dim3(256), shm, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_decode(const tq_ctx *ctx, const tq_kv_cache *cache, const void *q, int is_bf16, int32_t q_heads,
                         float scale, float *out, void *ws, hipStream_t st, const void *k_new, const void *v_new,
                         hipEvent_t ev0, hipEvent_t ev1, int n_q, int causal, const float *ext, int64_t ext_stride,
                         float *logits) {
  int chunk = 0, nchunks = 0;
  decode_ws_bytes(ctx, cache, q_heads, &chunk, &nchunks, n_q);
  DecodeArgs a = {};
  a.kbits = cache->k.bits;
  a.knorm = cache->k.norms;
  a.vbits = cache->v.bits;
  a.vnorm = cache->v.norms;
  a.nf16 = cache->k.norm_f16;
  a.seq_len = cache->d_seq_len;
  a.kbitsB = cache->k.mse_bits;
  a.kqjl = cache->k.qjl;
  a.vbitsB = cache->v.mse_bits;
  a.kv_heads = cache->kv_heads;
  a.capacity = cache->capacity;
  a.q_heads = q_heads;
  a.group = q_heads / cache->kv_heads;
  a.n_q = n_q;
  a.causal = causal;
  a.vgroup = a.group * n_q;
  a.kv_streams = cache->batch * cache->kv_heads;
  a.map = cache_map(cache, 0);
  {
    const int span = cache->d_block_table ? std::min(cache->page_tokens, chunk) : chunk;
    a.span_lg = 0;
    while ((1 << a.span_lg) < span) ++a.span_lg;
  }
  a.hgroups = (a.vgroup + 3) / 4;
  a.chunk = chunk;
  a.nchunks = nchunks;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.qjl_scale = (float)(std::sqrt(M_PI / 2.0) / DD);
  a.tables = ctx->d_tables;
  a.q = q;
  a.q_bf16 = is_bf16;
  a.rot = ctx->d_rot;
  a.rs_t = ctx->d_rs_t;
  const int streams = cache->batch * cache->kv_heads * a.hgroups;
  char *p = (char *)ws;
  a.qfrag = (uint32_t *)p;
  p += (((size_t)streams * 2 * 2 * 64 * 32) + 255) & ~(size_t)255;
  a.qconst = (float *)p;
  p += (((size_t)streams * 4 * QC * sizeof(float)) + 255) & ~(size_t)255;
  a.partial = (float *)p;
  p += (((size_t)cache->batch * q_heads * n_q * nchunks * (DD + 2) * sizeof(float)) + 255) & ~(size_t)255;
  a.out = out;
  const bool step = k_new != nullptr;
  if (step) {
    // fused step: the prep launch appends the new token; decode reads the new
    // lengths from the workspace and the merge launch advances seq_len
    a.ka = k_new;
    a.va = v_new;
    a.sk = ctx->d_sketch;
    a.kbits_w = cache->k.bits;
    a.vbits_w = cache->v.bits;
    a.knorm_w = cache->k.norms;
    a.vnorm_w = cache->v.norms;
    a.wlen = (int32_t *)p;
    a.len_inc = cache->d_seq_len;
  }
  a.streams_hg = streams;
  a.ext = ext;
  a.ext_stride = ext_stride;
  a.logit_out = logits;
  a.logit_stride = cache->capacity;
  // two (stream, head group) units per query block; fused step: one more block
  // per two KV streams appends their new tokens
  a.batch = cache->batch;
  if (ext) {
    // logits computed beforehand: no query preparation, the values from the cache
    const size_t shm = (size_t)5 * chunk * sizeof(float) + (size_t)(chunk / 128) * 2 * 64 * 16;
    const dim3 grid(nchunks * streams);
    hipError_t e = hipSuccess;
    if (ev0 && (e = hipEventRecord(ev0, st)) != hipSuccess) return e;
    switch (cache->v.mse_bits) {
      case 1: hipLaunchKernelGGL((decode_kernel<1, 1, false, false, false, true>), grid, dim3(256), shm, st, a); break;
      case 2: hipLaunchKernelGGL((decode_kernel<1, 2, false, false, false, true>), grid, dim3(256), shm, st, a); break;
      case 3: hipLaunchKernelGGL((decode_kernel<1, 3, false, false, false, true>), grid, dim3(256), shm, st, a); break;
      case 4: hipLaunchKernelGGL((decode_kernel<1, 4, false, false, false, true>), grid, dim3(256), shm, st, a); break;
      default: return hipErrorInvalidValue;
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (ev1 && (e = hipEventRecord(ev1, st)) != hipSuccess) return e;
    launch_decode_merge(a, (unsigned)streams, st);
    return hipGetLastError();
  }
  const dim3 pgrid((streams + 1) / 2 + (step ? (cache->batch * cache->kv_heads + 1) / 2 : 0));
  if (is_bf16)
    hipLaunchKernelGGL((step ? decode_prep_kernel<uint16_t, true> : decode_prep_kernel<uint16_t, false>), pgrid,
                       dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL((step ? decode_prep_kernel<float, true> : decode_prep_kernel<float, false>), pgrid,
                       dim3(512), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t shm = (size_t)5 * chunk * sizeof(float) + (size_t)(chunk / 128) * 2 * 64 * 16;
  dim3 grid(nchunks * streams);
  const int kb = cache->k.mse_bits, vb = cache->v.mse_bits;
  const bool kq = cache->k.qjl != 0;
  if (ev0 && (e = hipEventRecord(ev0, st)) != hipSuccess) return e;
#define TQ_DEC(K_, V_, Q_) else if (kb == K_ && vb == V_ && kq == Q_) e = launch_decode_kv<K_, V_, Q_>(a, grid, shm, st);
#define TQ_DEC4(K_, Q_) TQ_DEC(K_, 1, Q_) TQ_DEC(K_, 2, Q_) TQ_DEC(K_, 3, Q_) TQ_DEC(K_, 4, Q_)
  if (false) {
  }
  TQ_DEC4(1, true) TQ_DEC4(2, true) TQ_DEC4(3, true) TQ_DEC4(4, true)
  TQ_DEC4(0, true)
  TQ_DEC4(1, false) TQ_DEC4(2, false) TQ_DEC4(3, false) TQ_DEC4(4, false)
  else return hipErrorInvalidValue;
#undef TQ_DEC4
#undef TQ_DEC
  if (e != hipSuccess) return e;
  if (ev1 && (e = hipEventRecord(ev1, st)) != hipSuccess) return e;
  if (logits) return hipSuccess;  // measurement: no softmax, no merge
  launch_decode_merge(a, (unsigned)streams, st);
  return hipGetLastError();
}

hipError_t launch_merge_partials(const tq_ctx *ctx, const tq_kv_cache *cache, int32_t q_heads, int n_q,
                                 float *partial, int nchunks, float *out, hipStream_t st) {
  DecodeArgs a = {};
  a.kv_heads = cache->kv_heads;
  a.capacity = cache->capacity;
  a.q_heads = q_heads;
  a.group = q_heads / cache->kv_heads;
  a.n_q = n_q;
  a.vgroup = a.group * n_q;
  a.hgroups = (a.vgroup + 3) / 4;
  a.nchunks = nchunks;
  a.batch = cache->batch;
  a.kv_streams = cache->batch * cache->kv_heads;
  a.rot = ctx->d_rot;
  a.partial = partial;
  a.out = out;
  launch_decode_merge(a, (unsigned)(a.kv_streams * a.hgroups), st);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Vector search (tq_scores, d a multiple of 128): the decode scheme on blocks of
// 128 coordinates. Query side: q_rot = Pi q and q_s = S q_rot (fp32 GEMMs), then
// fixed point relative to each query's largest |q_rot| and |q_s|, split into
// eight balanced base-8 fp6 digits in the MFMA A layout of every block
// (search_prep_kernel). Key side: a block's plane words become 0/1 fp4 B
// operands (one AND each) and the Walsh masks their XORs, and
// v_mfma_scale_f32_16x16x128_f8f6f4 gives sum_j Q_j chi_j of the block per digit
// slot exactly. Each block's sums are folded into an fp32 score partial (the
// Walsh weights, the query units, the QJL constant and |r|), so one block's
// query fragments stay in registers for a whole block of keys. The top-k is
// fused: every wave keeps the best k (score, index) of each of its queries in
// LDS, and a merge kernel combines the key ranges; the score matrix is written
// only when the caller asks for it.
// ---------------------------------------------------------------------------

constexpr int SW = 8;       // waves per search work-group
constexpr int SQW = 2;      // query groups (of 4 queries) per wave
constexpr int STB = 8;      // 16-key tiles per wave step (128 keys)
constexpr int STS = 4;      // tiles whose key words are loaded together
constexpr int SK_MAX = 64;  // largest fused k

struct SearchArgs {
  const float *qa;          // [nq][2d]: q_rot | q_s
  int64_t nq, n;
  int d, nb;                // nb = d / 128 coordinate blocks
  uint32_t *qfrag;          // [ceil(nq/4)][nb][2 T][2 ins][64][8]: fp6 digit fragments
  float *qunit;             // [nq][2]: units of the fixed-point q_rot, q_s
  const uint32_t *kbits;
  const void *knorm;
  int nf16;
  float qjl_scale;          // sqrt(pi/2)/m
  const DeviceTables *tables;
  float *scores;            // [nq][n] or NULL
  int topk;                 // 0: no top-k
  int splits;               // key ranges (grid y)
  int64_t keys_per_split;   // a multiple of 16 * STB
  float *cand_val;          // [nq][splits][topk]
  int32_t *cand_idx;
  int32_t *top_idx;         // [nq][topk]
  float *top_val;
};

// One block of 256 threads per query group (4 queries): maxima, units, and the
// digit fragments of every block of 128 coordinates, in the layout
// decode_prep_kernel writes for d = 128: fragment (T, ins, lane) holds the 32
// codes of row 4 * query + slot, digit 4 * ins + slot; element 8q + i (bits
// 6(8q + i)) is coordinate 32 g + 4 i + q of the block, g = lane >> 4, scaled by
// (1, 1/2, 1/4, 1/4)[q].
__global__ void __launch_bounds__(256) search_prep_kernel(SearchArgs a) {
  __shared__ float mq[2][4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t qg = blockIdx.x;
  const int d = a.d;
  {
    // wave w: query 4 qg + w
    const int64_t q = qg * 4 + w;
    float m0 = 0.f, m1 = 0.f;
    if (q < a.nq) {
      const float *row = a.qa + q * 2 * d;
      for (int j = lane; j < d; j += 64) {
        m0 = fmaxf(m0, fabsf(row[j]));
        m1 = fmaxf(m1, fabsf(row[d + j]));
      }
    }
    for (int off = 32; off > 0; off >>= 1) {
      m0 = fmaxf(m0, __shfl_xor(m0, off));
      m1 = fmaxf(m1, __shfl_xor(m1, off));
    }
    if (lane == 0) {
      mq[0][w] = m0;
      mq[1][w] = m1;
      if (q < a.nq) {
        a.qunit[q * 2 + 0] = m0 > 0.f ? m0 / QMAX : 0.f;
        a.qunit[q * 2 + 1] = m1 > 0.f ? m1 / QMAX : 0.f;
      }
    }
  }
  __syncthreads();
  constexpr uint64_t dct[3] = {digit_code_table(0), digit_code_table(1), digit_code_table(2)};
  const int nfl = a.nb * 256;  // fragment lanes of the group: (block, T, ins, lane)
  for (int f = tid; f < nfl; f += 256) {
    const int cb = f >> 8, T = (f >> 7) & 1, ins = (f >> 6) & 1, Ln = f & 63;
    const int g = Ln >> 4, row = Ln & 15, hh = row >> 2, dig = 4 * ins + (row & 3);
    const int64_t q = qg * 4 + hh;
    const float m = mq[T][hh];
    const bool live = q < a.nq && m > 0.f;
    const float sc = live ? QMAX / m : 0.f;
    const float *src = a.qa + (live ? q : 0) * 2 * d + T * d + cb * 128 + 32 * g;
    const uint32_t sh = 3 * dig;
    uint32_t dw[6] = {0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 x4 = *reinterpret_cast<const float4 *>(src + 4 * i);
      const float xq[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const uint32_t z = (uint32_t)((int)rintf(xq[qq] * sc) + QOFF);
        const uint32_t v = (z >> sh) & 7u;
        const uint32_t code = (uint32_t)(dct[qq < 2 ? qq : 2] >> (6 * v)) & 63u;
        const int bit = 6 * (8 * qq + i);
        dw[bit >> 5] |= code << (bit & 31);
        if ((bit & 31) > 26) dw[(bit >> 5) + 1] |= code >> (32 - (bit & 31));
      }
    }
    uint4 *dst = reinterpret_cast<uint4 *>(a.qfrag + ((((qg * a.nb + cb) * 2 + T) * 2 + ins) * 64 + Ln) * 8);
    dst[0] = make_uint4(dw[0], dw[1], dw[2], dw[3]);
    dst[1] = make_uint4(dw[4], dw[5], 0u, 0u);
  }
}

// (score, index) order of the results: the higher score first, ties to the lower index
__device__ __forceinline__ bool sbetter(float v, int i, float w, int j) { return v > w || (v == w && i < j); }

__device__ __forceinline__ int64_t uniform64(int64_t x) {
  return (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(x >> 32)) << 32) |
                   (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x));
}

// KB MSE bits of the keys (0: pure QJL keys), QJL: the keys carry the sign word.
// Grid (query sets of SW * SQW groups, key ranges). Wave w of a work-group takes
// query groups SQW (SW blockIdx.x + w) + i, i < SQW, and the work-group's key
// range in steps of STB 16-key tiles; every wave of a work-group reads the same
// keys at about the same time (L1 and L2 hits after the first). Per step and
// block: the block's query fragments (registers), then per tile its key words,
// its masks, and per query group the MFMAs and the fold into the score partial.
// Lane (tn, G): key tn of a tile for query G of a group.
template <int KB, bool QJL>
__global__ void __launch_bounds__(64 * SW) search_kernel(SearchArgs a) {
  constexpr int KM = KB > 0 ? 1 << (KB - 1) : 0;
  constexpr int KQ = QJL ? 1 : 0;
  constexpr int NPL = KB + KQ;
  constexpr int NA = KM + KQ;  // masked sums per (tile, group)
  __shared__ float lv[SW][SQW * 4][SK_MAX];
  __shared__ int li[SW][SQW * 4][SK_MAX];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int tn = lane & 15, G = lane >> 4;
  const int64_t nqg = (a.nq + 3) >> 2;
  const int64_t qg0 = ((int64_t)blockIdx.x * SW + w) * SQW;
  if (qg0 >= nqg) return;  // no barriers below: every wave works alone
  const int K = a.topk;
  for (int i = lane; i < SQW * 4 * SK_MAX; i += 64) {
    lv[w][i / SK_MAX][i % SK_MAX] = -INFINITY;
    li[w][i / SK_MAX][i % SK_MAX] = INT_MAX;
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  // per group i: this lane's query, its units, the Walsh weights in query units
  bool qlive[SQW];
  float qs[SQW], wr[SQW][KM > 0 ? KM : 1], thr[SQW];
  const float *wk = a.tables->walsh[KB > 0 ? KB : 1];
#pragma unroll
  for (int i = 0; i < SQW; ++i) {
    const int64_t q = (qg0 + i) * 4 + G;
    qlive[i] = qg0 + i < nqg && q < a.nq;
    const float ur = qlive[i] ? a.qunit[q * 2] : 0.f, us = qlive[i] ? a.qunit[q * 2 + 1] : 0.f;
    qs[i] = us * a.qjl_scale;
#pragma unroll
    for (int mi = 0; mi < KM; ++mi) wr[i][mi] = wk[mi] * ur;
    thr[i] = -INFINITY;
  }
  const int sc0 = 127 + 3 * (lane & 3), sc1 = sc0 + 12;  // e8m0 row scales 2^(3 digit)
  auto ldfrag = [&](int64_t qg, int cb, int T, int ins) {
    if (qg >= nqg) qg = nqg - 1;  // an absent group repeats the last one (its scores are not used)
    const uint4 *p = reinterpret_cast<const uint4 *>(a.qfrag + ((((qg * a.nb + cb) * 2 + T) * 2 + ins) * 64 + lane) * 8);
    const uint4 x = p[0], y = p[1];
    i8v v;
    v[0] = (int)x.x; v[1] = (int)x.y; v[2] = (int)x.z; v[3] = (int)x.w;
    v[4] = (int)y.x; v[5] = (int)y.y; v[6] = 0; v[7] = 0;
    return v;
  };
  // accumulator start of every block: -sum_j Q_j per digit slot over the block (A
  // against an all-ones mask, B scale 2^1 undoes the 1/2 of every product); the
  // block's partial is then sum_j Q_j chi_j
  const int W = a.d >> 5;                       // 32-coordinate groups per key
  const uint32_t RBY = (uint32_t)(W * NPL * 4); // bytes per key record
  const int64_t k_begin = (int64_t)blockIdx.y * a.keys_per_split;
  const int64_t k_end = min(a.n, k_begin + a.keys_per_split);
  for (int64_t k0 = k_begin; k0 < k_end; k0 += 16 * STB) {
    const int64_t ku = uniform64(k0);
    const int rem = (int)min((int64_t)16 * STB, a.n - ku);  // keys of this step (range-checked loads)
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t *>(a.kbits) + ku * (W * NPL), (short)0, (int)(rem * RBY), 0x00020000);
    float part[SQW][STB];
#pragma unroll
    for (int i = 0; i < SQW; ++i)
#pragma unroll
      for (int t = 0; t < STB; ++t) part[i][t] = 0.f;
    // |r| of the lane's key in every tile (QJL keys)
    float rho[STB];
#pragma unroll
    for (int t = 0; t < STB; ++t) {
      const int64_t key = min(ku + 16 * t + tn, a.n - 1);
      rho[t] = QJL ? load_norm(a.knorm, 2 * key + 1, a.nf16) : 0.f;
    }
    for (int cb = 0; cb < a.nb; ++cb) {
      i8v ar[SQW][2], as[SQW][2];
      f4v ir[SQW], is[SQW];
#pragma unroll
      for (int i = 0; i < SQW; ++i) {
        const i8v ones = mask_fp4_01(0xFFFFFFFFu);
        const f4v z = {0.f, 0.f, 0.f, 0.f};
        ir[i] = z;
        is[i] = z;
#pragma unroll
        for (int ins = 0; ins < 2; ++ins) {
          ar[i][ins] = KM > 0 ? ldfrag(qg0 + i, cb, 0, ins) : i8v{};
          as[i][ins] = QJL ? ldfrag(qg0 + i, cb, 1, ins) : i8v{};
        }
        if constexpr (KM > 0) {
          ir[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ar[i][0], ones, z, 2, 4, 0, sc0, 0, 128);
          ir[i] = -__builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ar[i][1], ones, ir[i], 2, 4, 0, sc1, 0, 128);
        }
        if constexpr (QJL) {
          is[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(as[i][0], ones, z, 2, 4, 0, sc0, 0, 128);
          is[i] = -__builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(as[i][1], ones, is[i], 2, 4, 0, sc1, 0, 128);
        }
      }
#pragma unroll
      for (int t0 = 0; t0 < STB; t0 += STS) {
        // key words of block cb for tiles t0 .. t0 + STS - 1: group 4 cb + G of key 16 t + tn
        uint32_t pw[STS][NPL];
#pragma unroll
        for (int u = 0; u < STS; ++u) {
          const uint32_t off = (uint32_t)(16 * (t0 + u) + tn) * RBY + (uint32_t)((4 * cb + G) * NPL * 4);
          buffer_load_words<NPL, 0>(rk, off, pw[u]);
        }
#pragma unroll
        for (int u = 0; u < STS; ++u) {
          const int t = t0 + u;
          i8v sm[KB > 0 ? KB : 1];
#pragma unroll
          for (int p = 0; p < KB; ++p) sm[p] = mask_fp4_01(pw[u][p]);
          i8v bm[NA > 0 ? NA : 1];
#pragma unroll
          for (int mi = 0; mi < NA; ++mi) bm[mi] = mi < KM ? walsh_fp4(sm, walsh_mask(KB, mi)) : mask_fp4_01(pw[u][NPL - 1]);
#pragma unroll
          for (int i = 0; i < SQW; ++i) {
            f4v acc[NA > 0 ? NA : 1];
#pragma unroll
            for (int mi = 0; mi < NA; ++mi) {
              const bool cm = mi < KM;
              acc[mi] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(cm ? ar[i][0] : as[i][0], bm[mi],
                                                                         cm ? ir[i] : is[i], 2, 4, 0, sc0, 0, 129);
              acc[mi] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(cm ? ar[i][1] : as[i][1], bm[mi], acc[mi], 2,
                                                                         4, 0, sc1, 0, 129);
            }
            float c = part[i][t];
#pragma unroll
            for (int mi = 0; mi < KM; ++mi) c = fmaf(wr[i][mi], (acc[mi][0] + acc[mi][1]) + (acc[mi][2] + acc[mi][3]), c);
            if constexpr (QJL) c = fmaf(rho[t] * qs[i], (acc[KM][0] + acc[KM][1]) + (acc[KM][2] + acc[KM][3]), c);
            part[i][t] = c;
          }
        }
      }
    }
    // the step's scores: s = |k| * partial; the fused top-k
#pragma unroll
    for (int t = 0; t < STB; ++t) {
      const int64_t key = ku + 16 * t + tn;
      const bool kl = key < k_end;
      const float nk = load_norm(a.knorm, (1 + KQ) * (kl ? key : a.n - 1), a.nf16);
#pragma unroll
      for (int i = 0; i < SQW; ++i) {
        const float s = nk * part[i][t];
        const bool ok = kl && qlive[i];
        const int64_t q = (qg0 + i) * 4 + G;
        if (a.scores && ok) a.scores[q * a.n + key] = s;
        if (K > 0) {
          // candidates beat their query's k-th best; the wave inserts them one at
          // a time into the query's sorted list (keys arrive in increasing index
          // order, so a tie with the k-th best is not a candidate)
          uint64_t m = __builtin_amdgcn_ballot_w64(ok && s > thr[i]);
          while (m) {
            const int l = __builtin_ctzll(m);
            m &= m - 1;
            const float sv = __shfl(s, l);
            const int ki = __shfl((int)key, l);
            const int qq = i * 4 + (l >> 4);
            const float ev = lane < K ? lv[w][qq][lane] : -INFINITY;
            const int ei = lane < K ? li[w][qq][lane] : INT_MAX;
            const int pos = __builtin_popcountll(__builtin_amdgcn_ballot_w64(lane < K && sbetter(ev, ei, sv, ki)));
            const float e2 = __shfl(ev, K >= 2 ? K - 2 : 0);
            // every lane takes part in the shuffles (no lane reads an inactive one)
            const float evp = __shfl_up(ev, 1);
            const int eip = __shfl_up(ei, 1);
            if (pos < K) {
              if (lane > pos && lane < K) {
                lv[w][qq][lane] = evp;
                li[w][qq][lane] = eip;
              }
              if (lane == pos) {
                lv[w][qq][lane] = sv;
                li[w][qq][lane] = ki;
              }
              const float kth = (pos == K - 1 || K < 2) ? sv : e2;  // the k-th best now
              if (G == (l >> 4)) thr[i] = kth;
            }
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
          }
        }
      }
    }
  }
  if (K > 0) {
    // this range's best k of each of the wave's queries
    for (int e = lane; e < SQW * 4 * K; e += 64) {
      const int qq = e / K, j = e - qq * K;
      const int64_t q = qg0 * 4 + qq;
      if (q < a.nq) {
        const int64_t o = (q * a.splits + blockIdx.y) * K + j;
        a.cand_val[o] = lv[w][qq][j];
        a.cand_idx[o] = li[w][qq][j];
      }
    }
  }
}

// One wave per query: the best k of its splits * k candidates by (-score, index).
__global__ void __launch_bounds__(64) search_merge_kernel(SearchArgs a) {
  extern __shared__ unsigned char sm_raw[];
  const int lane = threadIdx.x;
  const int64_t q = blockIdx.x;
  const int K = a.topk, C = a.splits * K;
  float *vv = reinterpret_cast<float *>(sm_raw);
  int *ii = reinterpret_cast<int *>(vv + C);
  for (int i = lane; i < C; i += 64) {
    vv[i] = a.cand_val[q * C + i];
    ii[i] = a.cand_idx[q * C + i];
  }
  __syncthreads();
  for (int k = 0; k < K; ++k) {
    float bv = -INFINITY;
    int bi = INT_MAX, bp = -1;
    for (int i = lane; i < C; i += 64)
      if (ii[i] != INT_MAX && sbetter(vv[i], ii[i], bv, bi)) {
        bv = vv[i];
        bi = ii[i];
        bp = i;
      }
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off), op = __shfl_xor(bp, off);
      if (sbetter(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
        bp = op;
      }
    }
    if (lane == 0) {
      a.top_val[q * K + k] = bv;
      a.top_idx[q * K + k] = bi;
      if (bp >= 0) ii[bp] = INT_MAX;  // taken
    }
    __syncthreads();
  }
}

bool search_supported(const tq_ctx *ctx, int32_t topk) { return (ctx->d % 128) == 0 && topk <= SK_MAX; }

size_t search_ws_bytes(const tq_ctx *ctx, int64_t nq, int64_t n, int32_t topk, int *splits_out) {
  const int d = ctx->d;
  const int64_t nqg = (nq + 3) / 4;
  // key ranges: about two work-groups per compute unit in all, each range at
  // least 16 steps of 256 keys; the merge keeps at most 4096 candidates a query
  const int64_t sets = (nqg + SW * SQW - 1) / (SW * SQW);
  const int64_t steps = (n + 16 * STB - 1) / (16 * STB);
  int64_t splits = std::max<int64_t>(1, std::min<int64_t>((512 + sets - 1) / sets, steps / 16));
  if (topk > 0) splits = std::min<int64_t>(splits, 4096 / topk);
  if (splits_out) *splits_out = (int)splits;
  size_t b = (size_t)nq * 2 * d * sizeof(float);  // [q_rot | q_s]
  b = (b + 255) & ~(size_t)255;
  b += (size_t)nqg * (d / 128) * 2 * 2 * 64 * 32;  // digit fragments
  b = (b + 255) & ~(size_t)255;
  b += (size_t)nq * 2 * sizeof(float);  // units
  b = (b + 255) & ~(size_t)255;
  if (topk > 0) {
    b += (size_t)nq * splits * topk * sizeof(float);
    b = (b + 255) & ~(size_t)255;
    b += (size_t)nq * splits * topk * sizeof(int32_t);
    b = (b + 255) & ~(size_t)255;
  }
  return b;
}

template <int KB, bool QJL>
static void launch_search_kernel(const SearchArgs &a, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((search_kernel<KB, QJL>), grid, dim3(64 * SW), 0, st, a);
}

hipError_t launch_search(const tq_ctx *ctx, const void *q, int is_bf16, int64_t nq, const tq_packed *keys,
                         float *scores, int32_t topk, int32_t *top_idx, float *top_val, void *ws, hipStream_t st) {
  const int d = ctx->d;
  int splits = 1;
  search_ws_bytes(ctx, nq, keys->n, topk, &splits);
  const int64_t nqg = (nq + 3) / 4;
  char *p = (char *)ws;
  SearchArgs a = {};
  a.qa = (const float *)p;
  float *qa = (float *)p;
  p += ((size_t)nq * 2 * d * sizeof(float) + 255) & ~(size_t)255;
  a.nq = nq;
  a.n = keys->n;
  a.d = d;
  a.nb = d / 128;
  a.qfrag = (uint32_t *)p;
  p += ((size_t)nqg * a.nb * 2 * 2 * 64 * 32 + 255) & ~(size_t)255;
  a.qunit = (float *)p;
  p += ((size_t)nq * 2 * sizeof(float) + 255) & ~(size_t)255;
  if (topk > 0) {
    a.cand_val = (float *)p;
    p += ((size_t)nq * splits * topk * sizeof(float) + 255) & ~(size_t)255;
    a.cand_idx = (int32_t *)p;
  }
  a.kbits = keys->bits;
  a.knorm = keys->norms;
  a.nf16 = keys->norm_f16;
  a.qjl_scale = (float)(std::sqrt(M_PI / 2.0) / d);
  a.tables = ctx->d_tables;
  a.scores = scores;
  a.topk = topk;
  a.splits = splits;
  const int64_t steps = (keys->n + 16 * STB - 1) / (16 * STB);
  a.keys_per_split = ((steps + splits - 1) / splits) * 16 * STB;
  a.top_idx = top_idx;
  a.top_val = top_val;
  if (nq == 0 || keys->n == 0) return hipSuccess;
  // q_rot = Pi q, q_s = S q_rot (fp32 MFMA GEMMs)
  hipError_t e = launch_gemm_store(q, is_bf16, d, nq, ctx->d_rot, d, d, d, qa, 2 * d, st);
  if (e != hipSuccess) return e;
  if ((e = launch_gemm_store(qa, 0, 2 * d, nq, ctx->d_sketch, d, d, d, qa + d, 2 * d, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(search_prep_kernel, dim3((unsigned)nqg), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const dim3 grid((unsigned)((nqg + SW * SQW - 1) / (SW * SQW)), (unsigned)splits);
  const int kb = keys->mse_bits;
  if (keys->qjl) {
    switch (kb) {
      case 0: launch_search_kernel<0, true>(a, grid, st); break;
      case 1: launch_search_kernel<1, true>(a, grid, st); break;
      case 2: launch_search_kernel<2, true>(a, grid, st); break;
      case 3: launch_search_kernel<3, true>(a, grid, st); break;
      case 4: launch_search_kernel<4, true>(a, grid, st); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (kb) {
      case 1: launch_search_kernel<1, false>(a, grid, st); break;
      case 2: launch_search_kernel<2, false>(a, grid, st); break;
      case 3: launch_search_kernel<3, false>(a, grid, st); break;
      case 4: launch_search_kernel<4, false>(a, grid, st); break;
      default: return hipErrorInvalidValue;
    }
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (topk > 0) {
    const size_t shm = (size_t)splits * topk * (sizeof(float) + sizeof(int));
    hipLaunchKernelGGL(search_merge_kernel, dim3((unsigned)nq), dim3(64), shm, st, a);
    e = hipGetLastError();
  }
  return e;
}

// ---------------------------------------------------------------------------
// Read-bandwidth probe: each work-group streams its own contiguous slice with
// 16-byte non-temporal buffer loads, four in flight per thread, and writes an
// XOR fold of what it read. (Grid-strided loads of the default policy reached
// 5.5-6.0 TB/s; non-temporal loads of contiguous slices 6.9 TB/s.)
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(256) read_probe_kernel(const uint4 *__restrict__ p, int64_t n16, uint32_t *sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = min((int64_t)blockIdx.x * per, n16), b1 = min(b0 + per, n16);
  constexpr int64_t WIN = (int64_t)1 << 26;  // 16-byte granules per descriptor (1 GiB)
  uint32_t acc = 0;
  for (int64_t w0 = b0; w0 < b1; w0 += WIN) {
    const int64_t cnt = min(WIN, b1 - w0);
    // range-checked: a load past the window's cnt granules returns zeros
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4 *>(p + w0), (short)0, (int)(cnt * 16), 0x00020000);
    for (int64_t i = threadIdx.x; i < cnt; i += 1024) {
      uint32_t f[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)((i + 256 * u) * 16), 0, 2);
        f[u] = v[0] ^ v[1] ^ v[2] ^ v[3];
      }
      acc ^= (f[0] ^ f[1]) ^ (f[2] ^ f[3]);
    }
  }
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

hipError_t launch_read_probe(const void *src, size_t bytes, int grid, uint32_t *sink, hipStream_t st) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(256), 0, st, reinterpret_cast<const uint4 *>(src),
                     (int64_t)(bytes / 16), sink);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Append: one block of 128 threads (thread = coordinate) per (b, h) stream; a
// second launch advances the sequence lengths once every stream has read them.
// ---------------------------------------------------------------------------

struct AppendArgs {
  const void *k, *v;
  int bf16;
  const float *rot_t, *sketch_t;
  const DeviceTables *tables;
  uint32_t *kbits;
  void *knorm;
  uint32_t *vbits;
  void *vnorm;
  int32_t *seq_len;
  int nf16;  // fp16 norms
  int kB, vB, kv_heads, capacity;
  int kQ;  // keys carry the QJL sign word and |r|
  RecMap map;
};

__device__ __forceinline__ float block_sum128(float v, float *red) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = red[0] + red[1];
  __syncthreads();
  return r;
}

__global__ void __launch_bounds__(DD) append_kernel(AppendArgs a) {
  __shared__ float xs[DD], rs[DD], vs[DD];
  __shared__ float red[2];
  const int stream = blockIdx.x, j = threadIdx.x, lane = j & 63, wv = j >> 6;
  const int b = stream / a.kv_heads;
  const int t = a.seq_len[b];
  if (t < 0 || t >= a.capacity) return;  // full stream (or an invalid length): nothing is written
  const int64_t rec = a.map.rec(stream, t);
  const int64_t off = (int64_t)stream * DD + j;
  const float x = a.bf16 ? bf16f(((const uint16_t *)a.k)[off]) : ((const float *)a.k)[off];
  const float xv = a.bf16 ? bf16f(((const uint16_t *)a.v)[off]) : ((const float *)a.v)[off];
  xs[j] = x;
  vs[j] = xv;
  const float nrm = sqrtf(block_sum128(x * x, red));  // also orders the xs / vs writes
  const float nv = sqrtf(block_sum128(xv * xv, red));
  float y = 0.f, yv = 0.f;
#pragma unroll 16
  for (int k = 0; k < DD; ++k) {
    const float p = a.rot_t[k * DD + j];  // Pi[j][k], coalesced over j
    y += p * xs[k];
    yv += p * vs[k];
  }
  // ---- key: codes, residual, sketch signs (kQ; pure QJL keys: kB = 0, r = y) ----
  const bool live = nrm > 0.f;
  y = live ? y / nrm : 0.f;
  int idx = 0;
  for (int i = 0; i < (1 << a.kB) - 1; ++i) idx += (y >= a.tables->boundary[a.kB][i]) ? 1 : 0;
  if (!live) idx = 0;
  uint32_t words[5];
  for (int p = 0; p < a.kB; ++p) {
    const uint64_t bal = __builtin_amdgcn_ballot_w64(((idx >> p) & 1) != 0);
    words[p] = (lane < 32) ? (uint32_t)bal : (uint32_t)(bal >> 32);
  }
  float rho = 0.f;
  if (a.kQ) {  // uniform over the block
    const float r = live ? y - (a.kB > 0 ? a.tables->centroid[a.kB][idx] : 0.f) : 0.f;
    rs[j] = r;
    rho = sqrtf(block_sum128(r * r, red));
    float z = 0.f;
#pragma unroll 16
    for (int k = 0; k < DD; ++k) z += a.sketch_t[k * DD + j] * rs[k];
    const uint64_t bal = __builtin_amdgcn_ballot_w64(live && z >= 0.f);
    words[a.kB] = (lane < 32) ? (uint32_t)bal : (uint32_t)(bal >> 32);
  }
  const int np = a.kB + a.kQ;
  if ((lane & 31) == 0) {
    const int w = wv * 2 + (lane >> 5);
    uint32_t *dst = a.kbits + (rec * DW + w) * np;
    for (int p = 0; p < np; ++p) dst[p] = words[p];
  }
  if (j == 0) {
    store_norm(a.knorm, (1 + a.kQ) * rec, nrm, a.nf16);
    if (a.kQ) store_norm(a.knorm, 2 * rec + 1, live ? rho : 0.f, a.nf16);
    store_norm(a.vnorm, rec, nv, a.nf16);
  }
  // ---- value: codes into the token-major word of this coordinate ----
  const bool livev = nv > 0.f;
  yv = livev ? yv / nv : 0.f;
  int iv = 0;
  for (int i = 0; i < (1 << a.vB) - 1; ++i) iv += (yv >= a.tables->boundary[a.vB][i]) ? 1 : 0;
  if (!livev) iv = 0;
  const int64_t blk = rec >> 5;
  const int pos = (int)(rec & 31);
  uint32_t *dst = a.vbits + (blk * DD + j) * a.vB;
  for (int p = 0; p < a.vB; ++p) {
    const uint32_t bit = (uint32_t)((iv >> p) & 1) << pos;
    dst[p] = (pos == 0) ? bit : ((dst[p] & ~(1u << pos)) | bit);
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
  a.rot_t = ctx->d_rot_t;
  a.sketch_t = ctx->d_sketch_t;
  a.tables = ctx->d_tables;
  a.kbits = cache->k.bits;
  a.knorm = cache->k.norms;
  a.vbits = cache->v.bits;
  a.vnorm = cache->v.norms;
  a.nf16 = cache->k.norm_f16;
  a.seq_len = cache->d_seq_len;
  a.kB = cache->k.mse_bits;
  a.kQ = cache->k.qjl;
  a.vB = cache->v.mse_bits;
  a.kv_heads = cache->kv_heads;
  a.capacity = cache->capacity;
  a.map = cache_map(cache, 0);
  hipLaunchKernelGGL(append_kernel, dim3(cache->batch * cache->kv_heads), dim3(DD), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(append_len_kernel, dim3((cache->batch + 255) / 256), dim3(256), 0, st, cache->d_seq_len,
                     cache->batch, cache->capacity);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Library-held scratch for callers that cannot allocate (tq_attention_decode_noalloc):
// one array per device, alive until the process ends. Host code never uses the
// array's name as an address (on the host it is only a stand-in for the symbol):
// its device address comes from hipGetSymbolAddress, taken once per device with
// that device current (at context creation) and kept per device.
// ---------------------------------------------------------------------------

static __device__ __align__(256) unsigned char scratch[TQ_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_init(int device) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[device]) return hipSuccess;
  void *ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (ptr == nullptr) return hipErrorInvalidSymbol;
  g_scratch_ptr[device] = ptr;
  return hipSuccess;
}

void *scratch_ptr(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  return g_scratch_ptr[device];
}

}  // namespace tq
