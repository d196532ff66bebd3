// PolarQuant keys on gfx950, d = 128.
//
// Pages cited by title and section:
//  [arxiv-summary] PolarQuant summary page, section 3.中核となる技術的要素:
//            random preconditioning, a recursive polar transformation, angle
//            codebooks designed from the angle distribution, the radius kept
//            apart.
//  [gemilab] TurboQuant PolarQuant/QJL technical deep dive, section
//            PolarQuant：極座標変換による根本的削減 (v = r u).
//
// Layout (the pages fix none): level-1 angle codes (b1 bits each, pair i of
// y = Pi x) little-endian in a bit stream of w1 words, then the higher-level
// codes (b2 bits each; level 2 nodes first, each level in node order) in w2
// words; the radius ||x|| as fp32 in a separate array.
//
//  polar_encode_kernel   one wave per vector: lane l owns coordinate pair l;
//                        level l >= 2 combines the radii of lanes l and
//                        l + 2^(l-2) (a shuffle), so the owner lanes of level l
//                        are the multiples of 2^(l-1). Codes go to LDS, then
//                        one lane per record word assembles the bit streams.
//  polar_rebuild_kernel  one wave per record: lane l multiplies the radius by
//                        the cos or sin of its six ancestors' angles, top-down,
//                        then splits the result by its pair's angle: y_hat rows
//                        for the fp32 scores GEMM.
#include <hip/hip_runtime.h>

#include "tq_internal.h"

namespace tq {

constexpr int PD = 128;  // vector dimension of the polar path
constexpr int PL = 7;    // levels: log2(PD)

struct PolarArgs {
  const float *y;       // encode: [n][PD] rotated vectors
  float *yh;            // rebuild: [n][PD]
  uint32_t *bits;       // records [rec][w1 + w2]
  float *norms;         // [rec]
  int64_t n, rec0;
  int b1, b2, w1, w2;
  const DeviceTables *tables;
};

// first index of a level's codes in the higher-level stream
__device__ __forceinline__ int level_offset(int lv) { return 64 - (128 >> (lv - 1)); }

__device__ __forceinline__ uint32_t angle_code(float psi, const float *bnd) {
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < 15; ++i) c += psi >= bnd[i] ? 1u : 0u;  // boundaries past the last are +inf
  return c;
}

// word `wi` of a bit stream of `count` codes of `bits` bits (codes[i] at bit i * bits)
__device__ __forceinline__ uint32_t assemble_word(const uint8_t *codes, int count, int bits, int wi) {
  uint32_t w = 0;
  const int lo = wi * 32;
  for (int i = lo / bits; i < count && i * bits < lo + 32; ++i) {
    const int o = i * bits - lo;
    const uint32_t c = codes[i];
    w |= o >= 0 ? c << o : c >> (-o);
  }
  return w;
}

__global__ void __launch_bounds__(256) polar_encode_kernel(PolarArgs a) {
  __shared__ uint8_t codes[4][128];  // per wave: [0, 64) level 1, [64, 127) higher levels
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t v = (int64_t)blockIdx.x * 4 + w;
  const bool live = v < a.n;  // uniform per wave
  float r = 0.f;
  if (live) {
    const float2 p = reinterpret_cast<const float2 *>(a.y + v * PD)[lane];
    r = sqrtf(fmaf(p.x, p.x, p.y * p.y));
    codes[w][lane] = (uint8_t)angle_code(atan2f(p.y, p.x), a.tables->pbound[1][a.b1]);
#pragma unroll
    for (int lv = 2; lv <= PL; ++lv) {
      const int step = 1 << (lv - 2);
      const float rr = __shfl_down(r, step);  // the right child's radius
      const float psi = atan2f(rr, r);
      const float rn = sqrtf(fmaf(r, r, rr * rr));
      if ((lane & (2 * step - 1)) == 0)
        codes[w][64 + level_offset(lv) + (lane >> (lv - 1))] = (uint8_t)angle_code(psi, a.tables->pbound[lv][a.b2]);
      r = rn;  // an owner carries its node's radius to the next level
    }
  }
  __syncthreads();
  if (live) {
    const int W = a.w1 + a.w2;
    if (lane < W) {
      const uint32_t word = lane < a.w1 ? assemble_word(codes[w], 64, a.b1, lane)
                                        : assemble_word(codes[w] + 64, 63, a.b2, lane - a.w1);
      a.bits[(a.rec0 + v) * W + lane] = word;
    }
    if (lane == 0) a.norms[a.rec0 + v] = r;  // lane 0 owns the root: ||y|| = ||x||
  }
}

// `bits` bits at bit position `pos` of the stream whose first word is held by lane `base`
__device__ __forceinline__ uint32_t stream_bits(uint32_t wreg, int base, int pos, int bits) {
  const int j = base + (pos >> 5), sh = pos & 31;
  const uint32_t lo = __shfl(wreg, j), hi = __shfl(wreg, min(j + 1, 63));
  const uint64_t v = ((uint64_t)hi << 32 | lo) >> sh;
  return (uint32_t)v & ((1u << bits) - 1u);
}

__global__ void __launch_bounds__(256) polar_rebuild_kernel(PolarArgs a) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t v = (int64_t)blockIdx.x * 4 + w;
  if (v >= a.n) return;  // uniform per wave; no barrier below
  const int W = a.w1 + a.w2;
  const uint32_t wreg = lane < W ? a.bits[(a.rec0 + v) * W + lane] : 0u;
  float r = a.norms[a.rec0 + v];
  // top-down: the radius of this lane's pair is ||x|| times the cos (left child)
  // or sin (right child) of each ancestor's angle
#pragma unroll
  for (int lv = PL; lv >= 2; --lv) {
    const int node = lane >> (lv - 1), side = (lane >> (lv - 2)) & 1;
    const uint32_t c = stream_bits(wreg, a.w1, (level_offset(lv) + node) * a.b2, a.b2);
    r *= side ? a.tables->psin[lv][a.b2][c] : a.tables->pcos[lv][a.b2][c];
  }
  const uint32_t c1 = stream_bits(wreg, 0, lane * a.b1, a.b1);
  float2 o;
  o.x = r * a.tables->pcos[1][a.b1][c1];
  o.y = r * a.tables->psin[1][a.b1][c1];
  reinterpret_cast<float2 *>(a.yh + v * PD)[lane] = o;
}

static PolarArgs polar_args(const tq_ctx *ctx, const tq_polar_packed *p) {
  PolarArgs a = {};
  a.bits = p->bits;
  a.norms = p->norms;
  a.b1 = p->b1;
  a.b2 = p->b2;
  a.w1 = (p->b1 * (PD / 2) + 31) / 32;
  a.w2 = (p->b2 * (PD / 2 - 1) + 31) / 32;
  a.tables = ctx->d_tables;
  return a;
}

hipError_t launch_polar_quantize(const tq_ctx *ctx, const void *x, int is_bf16, int64_t n, int64_t xs,
                                 const tq_polar_packed *out, int64_t out_offset, void *ws, hipStream_t st) {
  float *y = (float *)ws;
  // preconditioning: y = Pi x on the fp32 MFMA GEMM
  hipError_t e = launch_gemm_store(x, is_bf16, xs, n, ctx->d_rot, PD, PD, PD, y, PD, st);
  if (e != hipSuccess) return e;
  PolarArgs a = polar_args(ctx, out);
  a.y = y;
  a.n = n;
  a.rec0 = out_offset;
  hipLaunchKernelGGL(polar_encode_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_polar_scores(const tq_ctx *ctx, const void *q, int is_bf16, int64_t nq, const tq_polar_packed *keys,
                               float *scores, void *ws, hipStream_t st) {
  float *qr = (float *)ws;
  float *yh = (float *)((char *)ws + (((size_t)nq * PD * sizeof(float) + 255) & ~(size_t)255));
  hipError_t e = launch_gemm_store(q, is_bf16, PD, nq, ctx->d_rot, PD, PD, PD, qr, PD, st);  // q_rot = Pi q
  if (e != hipSuccess) return e;
  PolarArgs a = polar_args(ctx, keys);
  a.yh = yh;
  a.n = keys->n;
  a.rec0 = 0;
  hipLaunchKernelGGL(polar_rebuild_kernel, dim3((unsigned)((keys->n + 3) / 4)), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return launch_gemm_store(qr, 0, PD, nq, yh, PD, keys->n, PD, scores, keys->n, st);  // <q_rot, y_hat>
}

}  // namespace tq
