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
//  polar_encode_kernel   a wave per vector (grid-strided): lane l owns pair l;
//                        the radii of level l >= 2 combine lanes l and
//                        l + 2^(l-2) (a shuffle; owners are the multiples of
//                        2^(l-1)), then the 63 higher angles are taken one per
//                        lane. Codes go to LDS, then one lane per record word
//                        assembles the bit streams.
//  polar_rebuild_kernel  one wave per record: lane l multiplies the radius by
//                        the cos or sin of its six ancestors' angles, top-down,
//                        then splits the result by its pair's angle: y_hat rows
//                        for the fp32 scores GEMM.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "tq_internal.h"

namespace tq {

constexpr int PD = 128;  // vector dimension of the polar path
constexpr int PL = 7;    // levels: log2(PD)

struct PolarArgs {
  const float *y;       // encode: [n][PD] rotated vectors
  float *yh;            // rebuild: [n][PD]
  uint32_t *bits;       // records [rec][w1 + w2]
  float *norms;         // [rec]
  int64_t n, rec0;      // vectors; rebuild: first record
  int64_t n_tokens, os; // encode: vector v = (stream v / n_tokens, token v % n_tokens) -> record
                        // stream * os + rec0 + token
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

// LDS ordering among the lanes of one wave (its LDS operations run in order):
// a compiler barrier plus a wave-scope fence
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Each wave encodes vectors v = wave id, + total waves, ... (a grid-strided loop:
// one short wave per vector spent its time being dispatched).
__global__ void __launch_bounds__(256) polar_encode_kernel(PolarArgs a) {
  __shared__ uint8_t codes[4][128];  // per wave: [0, 64) level 1, [64, 127) higher levels
  __shared__ float hb[PL + 1][16];   // the higher levels' boundaries (a lane's level varies with the lane)
  // w read through readfirstlane: v, and the record index divided out of it,
  // are wave-uniform (scalar arithmetic, not a per-lane 64-bit division)
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  const int W = a.w1 + a.w2;
  if (threadIdx.x < (PL + 1) * 16) {
    const int lv = threadIdx.x >> 4, i = threadIdx.x & 15;
    hb[lv][i] = lv >= 2 ? a.tables->pbound[lv][a.b2][i] : INFINITY;
  }
  __syncthreads();  // once, before the loop (every thread reaches it)
  const int nb2 = (1 << a.b2) - 1;  // boundaries of a higher-level code
  for (int64_t v = (int64_t)blockIdx.x * 4 + w; v < a.n; v += nwaves) {  // uniform per wave
    const float2 p = reinterpret_cast<const float2 *>(a.y + v * PD)[lane];
    codes[w][lane] = (uint8_t)angle_code(atan2f(p.y, p.x), a.tables->pbound[1][a.b1]);
    // radii of every level first (a shuffle and a hypot per level): rl[k] is the
    // radius of the level-(k+1) node this lane owns (owners: multiples of 2^k)
    float rl[PL];
    rl[0] = sqrtf(fmaf(p.x, p.x, p.y * p.y));
#pragma unroll
    for (int k = 1; k < PL; ++k) {
      const float rr = __shfl_down(rl[k - 1], 1 << (k - 1));  // the right child's radius
      rl[k] = sqrtf(fmaf(rl[k - 1], rl[k - 1], rr * rr));
    }
    const float r = rl[PL - 1];  // lane 0: the root, ||y|| = ||x||
    // then the 63 higher angles at once, one per lane: lane j < 63 takes code j of
    // the higher stream, node i of level lv, whose children are the level-(lv-1)
    // nodes 2i and 2i + 1, owned by lanes 2i * 2^(lv-2) and (2i + 1) * 2^(lv-2)
    const int j = lane;
    const int lv = j < 32 ? 2 : j < 48 ? 3 : j < 56 ? 4 : j < 60 ? 5 : j < 62 ? 6 : 7;
    const int i = j - level_offset(lv), sh = lv - 2;
    float left = 0.f, right = 0.f;
#pragma unroll
    for (int k = 0; k < PL - 1; ++k) {  // child level k + 1 = lv - 1: the shuffle source is per lane
      const float l_ = __shfl(rl[k], (2 * i) << k), r_ = __shfl(rl[k], (2 * i + 1) << k);
      left = k == sh ? l_ : left;
      right = k == sh ? r_ : right;
    }
    if (j < 63) {
      const float psi = atan2f(right, left);
      uint32_t c = 0;
      for (int q = 0; q < nb2; ++q) c += psi >= hb[lv][q] ? 1u : 0u;
      codes[w][64 + j] = (uint8_t)c;
    }
    wave_lds_sync();  // this wave's codes written
    const int64_t st = v / a.n_tokens, rec = st * a.os + a.rec0 + (v - st * a.n_tokens);
    if (lane < W) {
      const uint32_t word = lane < a.w1 ? assemble_word(codes[w], 64, a.b1, lane)
                                        : assemble_word(codes[w] + 64, 63, a.b2, lane - a.w1);
      a.bits[rec * W + lane] = word;
    }
    if (lane == 0) a.norms[rec] = r;  // lane 0 owns the root: ||y|| = ||x||
    wave_lds_sync();  // read back before the next vector's codes
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

hipError_t launch_polar_quantize(const tq_ctx *ctx, const void *x, int is_bf16, int64_t n_streams, int64_t n_tokens,
                                 int64_t xs, const tq_polar_packed *out, int64_t out_stream_stride, int64_t out_offset,
                                 void *ws, hipStream_t st) {
  const int64_t n = n_streams * n_tokens;
  float *y = (float *)ws;
  // preconditioning: y = Pi x on the fp32 MFMA GEMM
  hipError_t e = launch_gemm_store(x, is_bf16, xs, n, ctx->d_rot, PD, PD, PD, y, PD, st);
  if (e != hipSuccess) return e;
  PolarArgs a = polar_args(ctx, out);
  a.y = y;
  a.n = n;
  a.rec0 = out_offset;
  a.n_tokens = n_tokens;
  a.os = out_stream_stride;
  // enough waves to fill the GPU several times over; each loops over its vectors
  const int64_t blocks = std::min<int64_t>((n + 3) / 4, 8192);
  if (blocks > 0) hipLaunchKernelGGL(polar_encode_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
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

// ---------------------------------------------------------------------------
// Decode attention with PolarQuant keys. polar_logits_kernel scores every
// cached token against the 4 query heads of a (KV stream, head group): one
// thread per token evaluates <q, y_hat> on the transform's tree without
// rebuilding y_hat: a leaf (coordinate pair) gives q[2i] cos + q[2i+1] sin of
// its angle, a node combines its children as cos * left + sin * right, and the
// root is scaled by ||x||, evaluated per level-4 subtree (see the kernel). The
// logits (log2 units) feed
// decode_kernel's softmax and stage-1 value sums (EXT variant).
// ---------------------------------------------------------------------------

struct PolarLogitArgs {
  const uint32_t *bits;
  const float *norms;
  int b1, b2, w1, w2;
  const float *qrot;        // [batch * q_heads][PD]
  const int32_t *seq_len;
  float *out;               // [stream * hgroups + hg][4][stride]
  int64_t stride;
  int kv_heads, capacity, q_heads, group, hgroups;
  float scale_log2;
  const DeviceTables *tables;
};

__device__ __forceinline__ float4 fma4(float a, const float4 &x, float b, const float4 &y) {
  return make_float4(fmaf(a, x.x, b * y.x), fmaf(a, x.y, b * y.y), fmaf(a, x.z, b * y.z), fmaf(a, x.w, b * y.w));
}

// One thread per cached token: <q, u_hat> for the 4 heads of a head group. B1,
// B2: bits of the level-1 and higher angle codes, so that every code's bit
// position in the record is a constant (one bit-field extract from the record
// words held in registers). The block's 256 tokens share the queries, so the
// value of every leaf (coordinate pair l, level-1 code c):
// cos c * q[2l] + sin c * q[2l+1], is tabulated once per block in LDS.
template <int B1, int B2>
__global__ void __launch_bounds__(256) polar_logits_kernel(PolarLogitArgs a) {
  constexpr int W1 = (B1 * (PD / 2) + 31) / 32, W2 = (B2 * (PD / 2 - 1) + 31) / 32, W = W1 + W2;
  constexpr int NC1 = 1 << B1, HI0 = W1 * 32;
  __shared__ float4 lt[PD / 2][NC1];    // leaf values of the 4 heads per (pair, level-1 code)
  __shared__ float2 tab[PL + 1][16];    // (cos, sin) of each level's centroids
  __shared__ float4 qs[PD];             // coordinate -> the 4 heads
  const int tid = threadIdx.x;
  const int sg = blockIdx.y, hg = sg % a.hgroups, stream = sg / a.hgroups;
  const int b = stream / a.kv_heads, kvh = stream - b * a.kv_heads;
  const int nh = min(4, a.group - hg * 4);
  // a length past the logit rows (a caller error) is clamped: every write stays in its row
  const int len = min(max(a.seq_len[b], 0), (int)min(a.stride, (int64_t)a.capacity));
  if ((int)blockIdx.x * 256 >= len) return;  // the whole block (before any barrier)
  const int t = blockIdx.x * 256 + tid;
  const bool live = t < len;
  // this thread's record (a dead thread re-reads the last one)
  uint32_t rec[W];
  {
    const uint32_t *src = a.bits + ((int64_t)stream * a.capacity + min(t, len - 1)) * W;
#pragma unroll
    for (int k = 0; k < W; ++k) rec[k] = src[k];
  }
  for (int e = tid; e < 4 * PD; e += 256) {
    const int h = e >> 7, j = e & (PD - 1);
    reinterpret_cast<float *>(qs)[j * 4 + h] =
        h < nh ? a.qrot[((int64_t)b * a.q_heads + kvh * a.group + hg * 4 + h) * PD + j] : 0.f;
  }
  if (tid < (PL + 1) * 16) {
    const int lv = tid >> 4, i = tid & 15;
    const int bb = lv == 1 ? B1 : B2;
    tab[lv][i] = lv >= 1 ? make_float2(a.tables->pcos[lv][bb][i], a.tables->psin[lv][bb][i]) : make_float2(0.f, 0.f);
  }
  __syncthreads();
  for (int e = tid; e < (PD / 2) * NC1; e += 256) {
    const int l = e >> B1, c = e & (NC1 - 1);
    const float2 cs = tab[1][c];
    lt[l][c] = fma4(cs.x, qs[2 * l], cs.y, qs[2 * l + 1]);
  }
  __syncthreads();
  if (!live) return;  // past the barriers
  // code of nb bits at bit pos of the record (pos, nb constant after unrolling)
  auto code = [&](int pos, int nb) -> uint32_t {
    const int j = pos >> 5, sh = pos & 31;
    uint32_t v = rec[j] >> sh;
    if (sh + nb > 32) v |= rec[j + 1] << (32 - sh);
    return v & ((1u << nb) - 1u);
  };
  // node i of level lv (2..7): its angle's (cos, sin)
  auto ang = [&](int lv, int i) { return tab[lv][code(HI0 + (64 - (128 >> (lv - 1)) + i) * B2, B2)]; };
  auto node = [&](int lv, int i, const float4 &L, const float4 &R) {
    const float2 cs = ang(lv, i);
    return fma4(cs.x, L, cs.y, R);
  };
  auto leaf = [&](int l) { return lt[l][code(l * B1, B1)]; };
  // The tree's dot product is linear in each subtree: <q, u_hat> = sum over the
  // 8 level-4 nodes of (the cos / sin product along its 3 ancestors) x (its
  // subtree's value); a node's value is cos * left + sin * right of its angle.
  float4 T = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int n4 = 0; n4 < 8; ++n4) {
    float P = 1.f;
#pragma unroll
    for (int lv = 5; lv <= PL; ++lv) {
      const float2 cs = ang(lv, n4 >> (lv - 4));
      P *= ((n4 >> (lv - 5)) & 1) ? cs.y : cs.x;
    }
    const int l0 = 8 * n4;
    const float4 a3 = node(3, 2 * n4, node(2, 4 * n4, leaf(l0), leaf(l0 + 1)), node(2, 4 * n4 + 1, leaf(l0 + 2), leaf(l0 + 3)));
    const float4 b3 = node(3, 2 * n4 + 1, node(2, 4 * n4 + 2, leaf(l0 + 4), leaf(l0 + 5)),
                           node(2, 4 * n4 + 3, leaf(l0 + 6), leaf(l0 + 7)));
    T = fma4(1.f, T, P, node(4, n4, a3, b3));
    // one subtree at a time: T is final here and no LDS read moves across (an
    // empty asm statement, no instruction), so the live set stays one subtree's
    asm volatile("" : "+v"(T.x), "+v"(T.y), "+v"(T.z), "+v"(T.w) : : "memory");
  }
  // s = ||x|| <q, u_hat>, in log2 units of the softmax
  const float R = a.norms[(int64_t)stream * a.capacity + t] * a.scale_log2;
  float *o = a.out + (int64_t)sg * 4 * a.stride + t;
  const float v[4] = {T.x, T.y, T.z, T.w};
#pragma unroll
  for (int h = 0; h < 4; ++h)
    if (h < nh) o[(int64_t)h * a.stride] = R * v[h];
}

// q_rot = Pi q for the decode queries: a block of 256 threads takes 8 query
// rows; thread (coordinate j, half h) forms output j of rows 4h .. 4h + 3 from
// the columns of Pi^T (coalesced over j) against the rows staged in LDS.
__global__ void __launch_bounds__(256) polar_qrot_kernel(const void *q, int is_bf16, int64_t nq, const float *rot_t,
                                                         float *out) {
  __shared__ float qs[8][PD];
  const int tid = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * 8;
  for (int e = tid; e < 8 * PD; e += 256) {
    const int64_t r = r0 + (e >> 7);
    const int64_t i = r * PD + (e & (PD - 1));
    float x = 0.f;
    if (r < nq)
      x = is_bf16 ? __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(q)[i] << 16)
                  : reinterpret_cast<const float *>(q)[i];
    qs[e >> 7][e & (PD - 1)] = x;
  }
  __syncthreads();
  const int j = tid & (PD - 1), h = tid >> 7;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 16
  for (int kk = 0; kk < PD; ++kk) {
    const float r = rot_t[kk * PD + j];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = fmaf(r, qs[4 * h + u][kk], acc[u]);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t row = r0 + 4 * h + u;
    if (row < nq) out[row * PD + j] = acc[u];
  }
}

size_t polar_attention_ws_bytes(const tq_ctx *ctx, const tq_kv_cache *values, int32_t q_heads) {
  const int group = q_heads / values->kv_heads, hgroups = (group + 3) / 4;
  const int maxlen = values->host_max_len > 0 ? values->host_max_len : values->capacity;
  size_t b = decode_ws_bytes(ctx, values, q_heads, nullptr, nullptr, 1);
  b = (b + 255) & ~(size_t)255;
  b += (size_t)values->batch * q_heads * PD * sizeof(float);  // rotated queries
  b = (b + 255) & ~(size_t)255;
  b += (size_t)values->batch * values->kv_heads * hgroups * 4 * maxlen * sizeof(float);  // logits
  return b;
}

hipError_t launch_polar_attention(const tq_ctx *ctx, const tq_polar_packed *keys, const tq_kv_cache *values,
                                  const void *q, int is_bf16, int32_t q_heads, float scale, float *out, void *ws,
                                  hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  const int group = q_heads / values->kv_heads, hgroups = (group + 3) / 4;
  const int maxlen = values->host_max_len > 0 ? values->host_max_len : values->capacity;
  char *p = (char *)ws + ((decode_ws_bytes(ctx, values, q_heads, nullptr, nullptr, 1) + 255) & ~(size_t)255);
  float *qrot = (float *)p;
  p += ((size_t)values->batch * q_heads * PD * sizeof(float) + 255) & ~(size_t)255;
  float *lg = (float *)p;
  const int64_t nqr = (int64_t)values->batch * q_heads;
  hipLaunchKernelGGL(polar_qrot_kernel, dim3((unsigned)((nqr + 7) / 8)), dim3(256), 0, st, q, is_bf16, nqr,
                     ctx->d_rot_t, qrot);  // Pi q
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  PolarLogitArgs a = {};
  a.bits = keys->bits;
  a.norms = keys->norms;
  a.b1 = keys->b1;
  a.b2 = keys->b2;
  a.w1 = (keys->b1 * (PD / 2) + 31) / 32;
  a.w2 = (keys->b2 * (PD / 2 - 1) + 31) / 32;
  a.qrot = qrot;
  a.seq_len = values->d_seq_len;
  a.out = lg;
  a.stride = maxlen;
  a.kv_heads = values->kv_heads;
  a.capacity = values->capacity;
  a.q_heads = q_heads;
  a.group = group;
  a.hgroups = hgroups;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.tables = ctx->d_tables;
  const dim3 grid((unsigned)((maxlen + 255) / 256), (unsigned)(values->batch * values->kv_heads * hgroups));
  if (ev0 && (e = hipEventRecord(ev0, st)) != hipSuccess) return e;  // timing: the scoring kernel
#define TQ_PL(B1_, B2_) \
  case B1_ * 8 + B2_: hipLaunchKernelGGL((polar_logits_kernel<B1_, B2_>), grid, dim3(256), 0, st, a); break;
  switch (keys->b1 * 8 + keys->b2) {
    TQ_PL(1, 1) TQ_PL(1, 2) TQ_PL(1, 3) TQ_PL(1, 4) TQ_PL(2, 1) TQ_PL(2, 2) TQ_PL(2, 3) TQ_PL(2, 4)
    TQ_PL(3, 1) TQ_PL(3, 2) TQ_PL(3, 3) TQ_PL(3, 4) TQ_PL(4, 1) TQ_PL(4, 2) TQ_PL(4, 3) TQ_PL(4, 4)
    default: return hipErrorInvalidValue;
  }
#undef TQ_PL
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev1 && (e = hipEventRecord(ev1, st)) != hipSuccess) return e;
  return launch_decode(ctx, values, nullptr, 0, q_heads, scale, out, ws, st, nullptr, nullptr, nullptr, nullptr, 1, 0,
                       lg, maxlen);
}

}  // namespace tq
