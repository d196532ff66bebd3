// Prefill attention kernels of libtq for CDNA4 (gfx950), wave64: the query
// positions of a prompt chunk attend to the packed cache, sixteen virtual heads
// (query position x head of a KV head's group) per work-group.
//
// Pages cited by title and section:
//  [ebisuda] "TurboQuant: Google's 6x KV Cache Compression Algorithm Gains
//            Open-Source Momentum", sections 第1段階 (rotation, codebook) and
//            第2段階 (the QJL residual term of the inner-product estimator).
//  [gemilab] TurboQuant technical deep dive, section Attention機構 (softmax
//            attention over the cached keys and values).
//
// Kernels
//  prefill_prep_kernel  q_rot = Pi q and q_s = S q_rot of the sixteen virtual
//                       heads of a unit, fixed point relative to each head's
//                       largest |entry|, six balanced base-16 digits per entry
//                       as fp6 MFMA A fragments (one digit per fragment).
//  prefill_kernel       one pass over a chunk of the context in blocks of 512
//                       tokens: key scores of 16 heads x 16 tokens per fp6 x fp4
//                       MFMA chain, online softmax, value sums on int8 MFMA over
//                       the value bit masks. When one chunk covers the context
//                       the work-group finishes the output (o = Pi^T o_rot / l);
//                       otherwise the chunk partials (rotated output, max logit,
//                       weight sum) go through the decode merge.
//
// Arithmetic (the decode kernels' scheme, regrouped for many heads per KV head):
//  scores   A rows are the 16 heads, B columns 16 tokens; the six digit
//           fragments of a head are chained into one fp32 accumulator with the
//           e8m0 A scale 2^(4k+1), so the matrix core adds the digits and every
//           lane ends with finished sums sum_j Q_j (2 m_j - 1) of 4 heads x 1
//           token per Walsh mask (accumulator start -sum_j Q_j). The B values
//           are 0/1 scaled by 1, 1, 2, 2 in the four coordinate groups q of a
//           32-bit plane word; the A digits d/2, d/2, d/4, d/4 undo it (all
//           exact fp6 e2m3 values for d in [-8, 7]).
//  softmax  each block's logits (log2 units) against the block's own maximum;
//           the weight e_t |v_t| becomes a 29-bit fixed point relative to the
//           block's largest |v| (2^(29 - q') / vmax for token byte position q'),
//           four signed base-256 digits (int8 A fragments, one per digit).
//  values   B bytes are the value plane bits in place (2^q'); every block's
//           integer sums are flushed into an fp32 running output rescaled by
//           the running maximum (online softmax), o = unit sum_S w_S (2 M_S - W).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <type_traits>

#include "tq_device.h"
#include "tq_internal.h"
#include <hip/hip_fp16.h>

namespace tq {

constexpr int PH = 16;               // virtual heads per work-group (MFMA rows)
constexpr int PB = 512;              // tokens per block
constexpr int PLS = PB + 4;          // LDS row stride of the logits (floats)
constexpr int PDIG = 6;              // query digits, balanced base 16
constexpr float PQMAX = 7800000.f;   // |fixed-point query| bound: below 7 * (16^6 - 1) / 15
constexpr int PQOFF = 8947848;       // sum_k 8 * 16^k (k < 6): the digits of x + PQOFF are d_k + 8
constexpr int PCHUNK_MAX = 32768;    // tokens per work-group at most (int32 digit sums stay exact)
constexpr uint32_t PFRAG_WORDS = 2 * PDIG * 64 * 6;  // query fragment dwords per unit

struct PrefillArgs {
  const uint32_t *kbits;
  const void *knorm;
  const uint32_t *vbits;
  const void *vnorm;
  const int32_t *seq_len;
  RecMap map;              // record of (KV stream, token): contiguous, or pages of a multiple of 512 tokens
  int nf16;
  int kv_heads, capacity, q_heads, group, n_q, causal, vgroup;
  int hb;                  // units (of 16 virtual heads) per KV stream
  int kv_streams;
  int chunk, nchunks;      // tokens per work-group, chunks per unit
  const void *q;
  int q_bf16;
  const float *rs_t;       // [Pi ; S Pi]^T, 128 x 256 row-major
  const DeviceTables *tables;
  float scale_log2, qjl_scale;
  uint32_t *qfrag;         // [unit][2 (q_rot, q_s)][6 digits][64 lanes][6 dwords]
  float *qconst;           // [unit][16][4]: q_rot unit x scale, q_s unit x QJL constant x scale, -sum Q_rot, -sum Q_s
  float *partial;          // [stream][vgroup][nchunks][DD + 2]
  const float *rot;        // Pi, row-major (the output's inverse rotation when one chunk covers the context)
  float *out;              // [batch][n_q][q_heads][DD]
};

// e2m3 code of x, a multiple of 1/8 with |x| <= 7.5: sign 0x20, exponent field
// e (bias 1; 0 = subnormal m/8), mantissa m.
__host__ __device__ constexpr uint32_t e2m3_code(double x) {
  const uint32_t s = x < 0 ? 0x20u : 0u;
  const double a = x < 0 ? -x : x;
  if (a < 1.0) return s | (uint32_t)(a * 8.0);
  const int e = a < 2.0 ? 0 : (a < 4.0 ? 1 : 2);
  const uint32_t m = (uint32_t)((a / (double)(1 << e) - 1.0) * 8.0);
  return s | ((uint32_t)(e + 1) << 3) | m;
}

// Magnitude codes of |d| / 2^f for |d| = 0 .. 8, six bits each (f = 1: the
// digits of coordinate groups 0, 1; f = 2: groups 2, 3); the sign is bit 0x20.
__host__ __device__ constexpr uint64_t digit_mag_table(int f) {
  uint64_t t = 0;
  for (int m = 0; m <= 8; ++m) t |= (uint64_t)e2m3_code((double)m / (1 << f)) << (6 * m);
  return t;
}

// Key B operand of a 32-coordinate plane word: element 8q + i (nibble i of dword
// q) is bit 4i + q of w as an fp4 value 0/1 (q = 0, 1) or 0/2 (q = 2, 3).
__device__ __forceinline__ i8v mask_fp4_1122(uint32_t w) {
  i8v b;
  b[0] = (int)((w << 1) & 0x22222222u);
  b[1] = (int)(w & 0x22222222u);
  b[2] = (int)(w & 0x44444444u);
  b[3] = (int)((w >> 1) & 0x44444444u);
  b[4] = b[5] = b[6] = b[7] = 0;
  return b;
}

// A wave-uniform 64-bit value in scalar registers (buffer descriptors built from
// it stay scalar: no per-lane loop over distinct descriptors).
__device__ __forceinline__ int64_t uniform_i64(int64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Maximum over the 16 lanes of a row (DPP row rotations: no lane addresses).
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false)));
  return x;
}

// One work-group (256 threads) per unit of 16 virtual heads: the rotated and
// sketched queries, their fixed point and the A fragments of every digit.
__global__ void __launch_bounds__(256) prefill_prep_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) float qk[DD][PH];  // queries [coordinate][head]
  __shared__ float qv[2][PH][DD];                            // q_rot, q_s
  __shared__ __attribute__((aligned(16))) int qz[2][PH][DD];  // fixed point + PQOFF
  __shared__ float mx[2][PH];
  __shared__ int qsum[2][PH];
  const int unit = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int stream = unit / a.hb, hb = unit - stream * a.hb;
  const int b = stream / a.kv_heads, kvh = stream - b * a.kv_heads;
  const int vh0 = hb * PH, nh = min(PH, a.vgroup - vh0);
  for (int e = tid; e < PH * DD; e += 256) {
    const int h = e >> 7, k = e & (DD - 1);
    float x = 0.f;
    if (h < nh) {
      const int vh = vh0 + h, qi = vh / a.group, qj = vh - qi * a.group;
      const int64_t off = (((int64_t)b * a.n_q + qi) * a.q_heads + kvh * a.group + qj) * DD + k;
      x = a.q_bf16 ? bf16f(reinterpret_cast<const uint16_t *>(a.q)[off]) : reinterpret_cast<const float *>(a.q)[off];
    }
    qk[k][h] = x;
  }
  __syncthreads();
  {
    // thread r: row r of [Pi ; S Pi] against the sixteen queries
    float acc[PH];
#pragma unroll
    for (int h = 0; h < PH; ++h) acc[h] = 0.f;
    for (int k = 0; k < DD; ++k) {
      const float m = a.rs_t[k * 2 * DD + tid];
      const float4 *x = reinterpret_cast<const float4 *>(qk[k]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float4 v = x[u];
        acc[4 * u] = fmaf(m, v.x, acc[4 * u]);
        acc[4 * u + 1] = fmaf(m, v.y, acc[4 * u + 1]);
        acc[4 * u + 2] = fmaf(m, v.z, acc[4 * u + 2]);
        acc[4 * u + 3] = fmaf(m, v.w, acc[4 * u + 3]);
      }
    }
    const int T = tid >> 7, row = tid & (DD - 1);
#pragma unroll
    for (int h = 0; h < PH; ++h) qv[T][h][row] = acc[h];
  }
  __syncthreads();
  for (int p = wave; p < 2 * PH; p += 4) {
    const int T = p >> 4, h = p & (PH - 1);
    float m = fmaxf(fabsf(qv[T][h][lane]), fabsf(qv[T][h][lane + 64]));
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if (lane == 0) mx[T][h] = m;
  }
  __syncthreads();
  {
    // thread (type, head, 16 rows): fixed point and the sum over its rows
    const int T = tid >> 7, h = (tid >> 3) & (PH - 1), r0 = (tid & 7) * 16;
    const float m = mx[T][h];
    const float f = m > 0.f ? PQMAX / m : 0.f;
    int s = 0;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int Q = (int)rintf(qv[T][h][r0 + u] * f);
      qz[T][h][r0 + u] = Q + PQOFF;
      s += Q;
    }
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 4);
    if ((tid & 7) == 0) qsum[T][h] = s;
  }
  __syncthreads();
  if (tid < PH) {
    float *qc = a.qconst + ((int64_t)unit * PH + tid) * 4;
    qc[0] = mx[0][tid] / PQMAX * a.scale_log2;
    qc[1] = mx[1][tid] / PQMAX * a.qjl_scale * a.scale_log2;
    qc[2] = -(float)qsum[0][tid];
    qc[3] = -(float)qsum[1][tid];
  }
  // fragment (type T, digit k, lane l): row l & 15 (head), coordinates
  // 32 (l >> 4) + 4i + q as element 8q + i at 6 bits each; digit d scaled by
  // 1/2 (q = 0, 1) or 1/4 (q = 2, 3)
  for (int it = 0; it < 3; ++it) {
    const int item = it * 256 + tid;
    const int T = item / (PDIG * 64), k = (item >> 6) % PDIG, l = item & 63;
    const int h = l & (PH - 1), g = l >> 4;
    constexpr uint64_t mag1 = digit_mag_table(1), mag2 = digit_mag_table(2);
    uint32_t dw[6] = {0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int4 z4 = *reinterpret_cast<const int4 *>(&qz[T][h][32 * g + 4 * i]);
      const int zq[4] = {z4.x, z4.y, z4.z, z4.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d = ((zq[q] >> (4 * k)) & 15) - 8;
        const uint32_t mag = (uint32_t)((q < 2 ? mag1 : mag2) >> (6 * (d < 0 ? -d : d))) & 63u;
        const uint32_t code = mag | (d < 0 ? 0x20u : 0u);
        const int bit = 6 * (8 * q + i);
        dw[bit >> 5] |= code << (bit & 31);
        if ((bit & 31) > 26) dw[(bit >> 5) + 1] |= code >> (32 - (bit & 31));
      }
    }
    uint32_t *dst = a.qfrag + (int64_t)unit * PFRAG_WORDS + ((T * PDIG + k) * 64 + l) * 6;
#pragma unroll
    for (int j = 0; j < 6; ++j) dst[j] = dw[j];
  }
}

// KB MSE bits of the keys (0: pure QJL keys), VB value bits (<= 3), QJL: the keys
// carry the sign word and |r|; NF16: the cache's norms are fp16 (compile-time, so
// that the tile loop has no branch and its loads stay in flight across tiles).
// Work-group: 4 waves over one chunk of one unit (stream, 16 virtual heads).
// Per block of 512 tokens: phase K (wave w scores tokens 128 w .. 128 w + 127 of
// all 16 heads), phase S (thread (head, 32 tokens): softmax weights to value
// digits), phase V (wave w sums coordinates 32 w .. 32 w + 31 of all heads).
template <int KB, int VB, bool QJL, bool NF16>
__global__ void __launch_bounds__(256, 2) prefill_kernel(PrefillArgs a) {
  constexpr int KM = KB > 0 ? 1 << (KB - 1) : 0;  // key Walsh masks
  constexpr int KQ = QJL ? 1 : 0;
  constexpr int NA = KM + KQ;                      // key masks per tile
  constexpr int NPL = KB + KQ;                     // words per 32-coordinate group of a key record
  constexpr int RB = DW * NPL * 4;                 // bytes per key record
  constexpr int VM = 1 << (VB - 1);                // value Walsh masks
  constexpr int VWB = DD * VB * 4;                 // bytes per 32-token value block
  __shared__ __attribute__((aligned(16))) float lg[PH * PLS];          // logits (log2 units) [head][token]
  __shared__ __attribute__((aligned(16))) float vnl[PB];               // value norms
  __shared__ __attribute__((aligned(16))) uint4 av[4 * 2 * 4 * 64];    // [group][lo, hi][digit][lane] int8 A
  __shared__ __attribute__((aligned(16))) float sred[4][PH];           // block max logit per wave and head
  __shared__ float svm[4];                                            // block max |v| per wave
  __shared__ __attribute__((aligned(16))) long long wtp[4][PH];       // weight totals per wave and head
  __shared__ float lred[4][PH];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // work-group -> (stream, unit of the stream, chunk). Work-groups are dealt to
  // the 8 XCDs round-robin by id: with a multiple of 8 streams all work-groups of
  // a stream land on one XCD, whose L2 then holds that stream's records for all
  // its units. Units of later query positions (the most visible tokens) first.
  int stream, hb, c;
  {
    const int id = blockIdx.x, per = a.hb * a.nchunks;
    int rem;
    if ((a.kv_streams & 7) == 0) {
      const int k = id >> 3, s8 = k / per;
      rem = k - s8 * per;
      stream = s8 * 8 + (id & 7);
    } else {
      stream = id / per;
      rem = id - stream * per;
    }
    const int hr = rem / a.nchunks;
    c = rem - hr * a.nchunks;
    hb = a.hb - 1 - hr;
  }
  const int unit = stream * a.hb + hb;
  const int b = stream / a.kv_heads;
  // a length outside [0, capacity] (a caller error) is clamped
  const int len = min(max(a.seq_len[b], 0), a.capacity);
  const int vh0 = hb * PH, nh = min(PH, a.vgroup - vh0);
  auto vis = [&](int h) {  // tokens virtual head vh0 + h sees; grows with h
    if (h >= nh) return 0;
    const int qi = (vh0 + h) / a.group;
    return min(max(a.causal ? len - a.n_q + qi + 1 : len, 0), len);
  };
  const int vis_lo = vis(0), vis_hi = vis(nh - 1);
  const int t_begin = c * a.chunk;
  const int t_end = min(min(len, t_begin + a.chunk), vis_hi);
  const int64_t pstride = (int64_t)a.nchunks * (DD + 2);
  float *pbase = a.partial + ((int64_t)stream * a.vgroup + vh0) * pstride + (int64_t)c * (DD + 2);
  if (t_begin >= t_end) {
    if (a.nchunks == 1) {
      // no visible token for any head of the unit: zero outputs
      const int b2 = stream / a.kv_heads, kvh = stream - b2 * a.kv_heads;
      for (int e = tid; e < nh * DD; e += 256) {
        const int h = e / DD, j = e - h * DD;
        const int vh = vh0 + h, qi = vh / a.group, qj = vh - qi * a.group;
        a.out[(((int64_t)b2 * a.n_q + qi) * a.q_heads + kvh * a.group + qj) * DD + j] = 0.f;
      }
      return;
    }
    for (int e = tid; e < nh * (DD + 2); e += 256) {
      const int h = e / (DD + 2), j = e - h * (DD + 2);
      pbase[h * pstride + j] = j == DD ? -INFINITY : 0.f;
    }
    return;
  }

  // phase K lane: token column tn, heads 4G .. 4G + 3
  const int tn = lane & 15, G = lane >> 4;
  float sr[4], qs[4];
  int visk[4];
  f4v init_r, init_s;
  {
    const float4 *qc = reinterpret_cast<const float4 *>(a.qconst + (int64_t)unit * PH * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 v = qc[4 * G + i];
      sr[i] = v.x;
      qs[i] = v.y;
      init_r[i] = v.z;
      init_s[i] = v.w;
      visk[i] = vis(4 * G + i);
    }
  }
  float wk[KM > 0 ? KM : 1];
#pragma unroll
  for (int mi = 0; mi < KM; ++mi) wk[mi] = a.tables->walsh[KB > 0 ? KB : 1][mi];
  float wv[VM];
#pragma unroll
  for (int mi = 0; mi < VM; ++mi) wv[mi] = a.tables->walsh[VB][mi];
  // phase S thread: head hs, 32-token block vgb of the block
  const int hs = tid & 15, vgb = tid >> 4;
  float mrs = -INFINITY, lsum = 0.f;  // running max and weight sum of head hs
  // phase V lane: coordinate column vn, heads 4 vgl .. 4 vgl + 3
  const int vn = lane & 15, vgl = lane >> 4;
  float mrv[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  float O[2][4];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) O[nt][i] = 0.f;

  const __amdgpu_buffer_rsrc_t rqf = __builtin_amdgcn_make_buffer_rsrc(a.qfrag + (int64_t)unit * PFRAG_WORDS, (short)0,
                                                                       PFRAG_WORDS * 4, 0x00020000);
  constexpr int NB = 4;                               // fp32 norms (fp16: 2, below)
  for (int T0 = t_begin; T0 < t_end; T0 += PB) {
    const int n = __builtin_amdgcn_readfirstlane(min(PB, t_end - T0));
    const bool full = n == PB && T0 + PB <= vis_lo;  // no token of the block is masked
    // ---- phase K ----
    {
      float lmx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      float vmx = 0.f;
      const int nw = __builtin_amdgcn_readfirstlane(min(max(n - 128 * wave, 0), 128));  // tokens of this wave
      if (nw > 0) {
        // range-checked descriptors over the wave's records only: loads past
        // them return zeros; the scalar offset (not range-checked) stays 0
        const int64_t r0 = uniform_i64(a.map.rec(stream, T0) + 128 * wave);
        constexpr int nb = NF16 ? 2 : NB;
        const __amdgpu_buffer_rsrc_t rkb = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint32_t *>(a.kbits) + r0 * DW * NPL, (short)0, nw * RB, 0x00020000);
        const __amdgpu_buffer_rsrc_t rkn = __builtin_amdgcn_make_buffer_rsrc(
            reinterpret_cast<char *>(const_cast<void *>(a.knorm)) + (1 + KQ) * r0 * nb, (short)0, nw * (1 + KQ) * nb,
            0x00020000);
        const __amdgpu_buffer_rsrc_t rvn = __builtin_amdgcn_make_buffer_rsrc(
            reinterpret_cast<char *>(const_cast<void *>(a.vnorm)) + r0 * nb, (short)0, nw * nb, 0x00020000);
        struct KT {
          uint32_t pl[NPL];
          float2 kn;  // (|k|, |r|)
          float vn;
        };
        auto kload = [&](int u, KT &t) {
          const uint32_t tl = (uint32_t)(16 * u + tn);
          const uint32_t off = tl * RB + (uint32_t)(G * NPL * 4);
          buffer_load_words<NPL, 2>(rkb, off, t.pl);
          if constexpr (NF16) {
            if constexpr (QJL) {
              const uint32_t h2 = __builtin_amdgcn_raw_buffer_load_b32(rkn, tl * 4u, 0, 2);
              t.kn = make_float2(__half2float(__ushort_as_half((unsigned short)(h2 & 0xFFFFu))),
                                 __half2float(__ushort_as_half((unsigned short)(h2 >> 16))));
            } else {
              t.kn = make_float2(__half2float(__ushort_as_half(__builtin_amdgcn_raw_buffer_load_b16(rkn, tl * 2u, 0, 2))),
                                 0.f);
            }
            t.vn = __half2float(__ushort_as_half(__builtin_amdgcn_raw_buffer_load_b16(rvn, tl * 2u, 0, 2)));
          } else {
            if constexpr (QJL) {
              const auto k2 = __builtin_amdgcn_raw_buffer_load_b64(rkn, tl * 8u, 0, 2);
              t.kn = make_float2(__uint_as_float(k2[0]), __uint_as_float(k2[1]));
            } else {
              t.kn = make_float2(__uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rkn, tl * 4u, 0, 2)), 0.f);
            }
            t.vn = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rvn, tl * 4u, 0, 2));
          }
        };
        KT ka, kb;
        kload(0, ka);
        // the query fragments (an L2 hit after the work-group's first block):
        // one lane offset, the fragment offsets in the scalar offset field
        i8v aq[2][PDIG];
#pragma unroll
        for (int T = 0; T < 2; ++T) {
          if ((T == 0 && KM == 0) || (T == 1 && !QJL)) continue;
#pragma unroll
          for (int k = 0; k < PDIG; ++k) {
            const int fo = (T * PDIG + k) * 64 * 24;
            const auto x0 = __builtin_amdgcn_raw_buffer_load_b64(rqf, (uint32_t)lane * 24u, fo, 0);
            const auto x1 = __builtin_amdgcn_raw_buffer_load_b64(rqf, (uint32_t)lane * 24u + 8u, fo, 0);
            const auto x2 = __builtin_amdgcn_raw_buffer_load_b64(rqf, (uint32_t)lane * 24u + 16u, fo, 0);
            i8v v;
            v[0] = (int)x0[0]; v[1] = (int)x0[1]; v[2] = (int)x1[0]; v[3] = (int)x1[1];
            v[4] = (int)x2[0]; v[5] = (int)x2[1]; v[6] = 0; v[7] = 0;
            aq[T][k] = v;
          }
        }
        int lim[4];  // block-relative visibility of the lane's heads
#pragma unroll
        for (int i = 0; i < 4; ++i) lim[i] = min(visk[i] - T0, n);
        auto kcompute = [&](int u, const KT &t, auto masked) {
          i8v bm[NA > 0 ? NA : 1];
          {
            i8v sm[KB > 0 ? KB : 1];
#pragma unroll
            for (int p = 0; p < KB; ++p) sm[p] = mask_fp4_1122(t.pl[p]);
#pragma unroll
            for (int mi = 0; mi < KM; ++mi) bm[mi] = walsh_fp4(sm, walsh_mask(KB, mi));
            if constexpr (QJL) bm[KM] = mask_fp4_1122(t.pl[NPL - 1]);
          }
          f4v acc[NA > 0 ? NA : 1];
#pragma unroll
          for (int mi = 0; mi < NA; ++mi) acc[mi] = mi < KM ? init_r : init_s;
          // digit-major: the NA accumulators are independent within a digit. The
          // wave's priority is raised while it issues MFMAs, so that of two waves
          // on a SIMD the one with matrix work goes first and the other's VALU
          // work fills the gaps
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int k = 0; k < PDIG; ++k)
#pragma unroll
            for (int mi = 0; mi < NA; ++mi)
              acc[mi] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aq[mi < KM ? 0 : 1][k], bm[mi], acc[mi], 2, 4,
                                                                         0, 128 + 4 * k, 0, 128);
          __builtin_amdgcn_s_setprio(0);
          const int tc = 128 * wave + 16 * u + tn;  // block-relative token
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float code = 0.f;
#pragma unroll
            for (int mi = 0; mi < KM; ++mi) code = fmaf(wk[mi], acc[mi][i], code);
            float s;
            if constexpr (QJL) s = t.kn.x * fmaf(sr[i], code, qs[i] * (t.kn.y * acc[KM][i]));
            else s = t.kn.x * (sr[i] * code);
            if constexpr (decltype(masked)::value) s = tc < lim[i] ? s : -INFINITY;
            lg[(4 * G + i) * PLS + tc] = s;
            lmx[i] = fmaxf(lmx[i], s);
          }
          vnl[tc] = t.vn;
          vmx = fmaxf(vmx, t.vn);
        };
        const int ntl = (nw + 15) >> 4;
        auto tiles = [&](auto masked) {
          for (int u = 0; u < ntl; u += 2) {
            kload(u + 1, kb);  // past the wave's tokens: zeros
            __builtin_amdgcn_sched_barrier(0);
            kcompute(u, ka, masked);
            if (u + 1 >= ntl) break;
            kload(u + 2, ka);
            __builtin_amdgcn_sched_barrier(0);
            kcompute(u + 1, kb, masked);
          }
        };
        // blocks inside every head's visible range skip the per-token mask
        if (full) tiles(std::false_type{});
        else tiles(std::true_type{});
      }
      // the block's tokens past its end (the chunk's last block): masked logits
      // and zero norms, so phase S needs no per-token test
      if (nw < 128) {
        for (int u = (nw + 15) >> 4; u < 8; ++u) {
          const int tc = 128 * wave + 16 * u + tn;
#pragma unroll
          for (int i = 0; i < 4; ++i) lg[(4 * G + i) * PLS + tc] = -INFINITY;
          vnl[tc] = 0.f;
        }
      }
      // per-head maxima over the wave's tokens: the 16 lanes of a row group
#pragma unroll
      for (int i = 0; i < 4; ++i) lmx[i] = row_max16(lmx[i]);
      vmx = row_max16(vmx);
      if (tn == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sred[wave][4 * G + i] = lmx[i];
      }
      if (lane == 0) {
        const float v1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vmx), 16));
        const float v2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vmx), 32));
        const float v3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vmx), 48));
        svm[wave] = fmaxf(fmaxf(vmx, v1), fmaxf(v2, v3));
      }
    }
    __syncthreads();
    // the block's value words (all four 128-token groups), requested before phase S;
    // blocks past the chunk's end read zeros (range-checked descriptor). A block's
    // records are consecutive (one page holds whole blocks)
    const __amdgpu_buffer_rsrc_t rvb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t *>(a.vbits) + (uniform_i64(a.map.rec(stream, T0)) >> 5) * DD * VB, (short)0,
        ((n + 31) >> 5) * VWB, 0x00020000);
    const uint32_t vlo = (uint32_t)((vgl * DD + 32 * wave + vn) * VB * 4);
    uint32_t vw[4][2][VB];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int p = 0; p < VB; ++p)
          vw[g][nt][p] = __builtin_amdgcn_raw_buffer_load_b32(rvb, g * 4 * VWB + vlo + nt * 16 * VB * 4 + 4 * p, 0, 0);
    const float bv = fmaxf(fmaxf(svm[0], svm[1]), fmaxf(svm[2], svm[3]));
    // the block maxima of the phase V lane's heads, read before the next block's
    // phase K can overwrite them
    float bmv[4];
    {
      float4 bq[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) bq[w] = reinterpret_cast<const float4 *>(sred[w])[vgl];
      bmv[0] = fmaxf(fmaxf(bq[0].x, bq[1].x), fmaxf(bq[2].x, bq[3].x));
      bmv[1] = fmaxf(fmaxf(bq[0].y, bq[1].y), fmaxf(bq[2].y, bq[3].y));
      bmv[2] = fmaxf(fmaxf(bq[0].z, bq[1].z), fmaxf(bq[2].z, bq[3].z));
      bmv[3] = fmaxf(fmaxf(bq[0].w, bq[1].w), fmaxf(bq[2].w, bq[3].w));
    }
    // ---- phase S: thread (head hs, tokens 32 vgb .. 32 vgb + 31) ----
    {
      const float bm = fmaxf(fmaxf(sred[0][hs], sred[1][hs]), fmaxf(sred[2][hs], sred[3][hs]));
      const float ref = bm == -INFINITY ? 0.f : bm;  // weights against the block's own maximum
      // token byte position q' = t & 7: weight scale 2^(29 - q') / bv (the B byte is 2^q' b)
      const float cv = bv > 0.f ? 536870912.f / bv : 0.f;
      const float *lrow = lg + hs * PLS + 32 * vgb;
      const float *vrow = vnl + 32 * vgb;
      float le = 0.f;
      long long wt = 0;  // sum_t W_t 2^q' (exact)
      uint4 *dst = av + ((vgb >> 2) * 8) * 64 + 16 * (vgb & 3) + hs;
#pragma unroll
      for (int lohi = 0; lohi < 2; ++lohi) {
        uint32_t x[4][4];
#pragma unroll
        for (int kp = 0; kp < 4; ++kp) {
          const float4 l4 = *reinterpret_cast<const float4 *>(lrow + 8 * kp + 4 * lohi);
          const float4 v4 = *reinterpret_cast<const float4 *>(vrow + 8 * kp + 4 * lohi);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, nv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int qq = 4 * lohi + q;
            const float e = __builtin_amdgcn_exp2f(lv[q] - ref);  // <= 1
            // rounding by truncation of W + 1/2 (W >= 0)
            uint32_t W = (uint32_t)fmaf(e, nv[q] * (cv * (1.f / (float)(1 << qq))), 0.5f);
            le += e;
            wt += (long long)((unsigned long long)W << qq);
            // four signed base-256 digits; the B byte of q' = 7 is -128 b, so its weight is negated
            x[kp][q] = (qq == 7 ? 0x80808080u - W : W + 0x80808080u) ^ 0x80808080u;
          }
        }
        // digit words: dword q of digit k holds byte k of tokens 8 kp + 4 lohi + q, kp = 0..3
        uint32_t d[4][4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t p01 = __builtin_amdgcn_perm(x[1][q], x[0][q], 0x05010400u);
          const uint32_t p23 = __builtin_amdgcn_perm(x[3][q], x[2][q], 0x05010400u);
          const uint32_t q01 = __builtin_amdgcn_perm(x[1][q], x[0][q], 0x07030602u);
          const uint32_t q23 = __builtin_amdgcn_perm(x[3][q], x[2][q], 0x07030602u);
          d[0][q] = __builtin_amdgcn_perm(p23, p01, 0x05040100u);
          d[1][q] = __builtin_amdgcn_perm(p23, p01, 0x07060302u);
          d[2][q] = __builtin_amdgcn_perm(q23, q01, 0x05040100u);
          d[3][q] = __builtin_amdgcn_perm(q23, q01, 0x07060302u);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) dst[(lohi * 4 + k) * 64] = make_uint4(d[k][0], d[k][1], d[k][2], d[k][3]);
      }
      // weight totals per head: lanes hs, hs + 16, hs + 32, hs + 48 of the wave
      wt += __shfl_xor(wt, 16);
      wt += __shfl_xor(wt, 32);
      if (lane < 16) wtp[wave][hs] = wt;
      // online softmax: the running sum moves to the new maximum
      const float mn = fmaxf(mrs, bm);
      const float rh = mrs == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrs - mn);
      const float fh = bm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(bm - mn);
      lsum = fmaf(lsum, rh, le * fh);
      mrs = mn;
    }
    __syncthreads();
    // ---- phase V: wave w sums coordinates 32 w .. 32 w + 31 of the 16 heads ----
    {
      // the block's online-softmax factors of the lane's heads
      const float unit = bv * (1.f / 536870912.f);
      float rhv[4], scv[4], wtv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = 4 * vgl + i;
        const float bm = bmv[i];
        const float mn = fmaxf(mrv[i], bm);
        rhv[i] = mrv[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrv[i] - mn);
        scv[i] = (bm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(bm - mn)) * unit;
        mrv[i] = mn;
        wtv[i] = (float)(wtp[0][hh] + wtp[1][hh] + wtp[2][hh] + wtp[3][hh]);
      }
      // one 16-coordinate half (nt) at a time: its integer sums over the block's
      // groups, then the flush o_rot = unit sum_S w_S (2 M_S - W) into the
      // running output
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        i4v acc[VM][4];
        auto vgroup = [&](auto gc, auto first) {
          constexpr int g = decltype(gc)::value;
          // one group's fragments at a time (no hoisting of later groups' LDS reads)
          __builtin_amdgcn_sched_barrier(0);
          const uint4 *ag = av + (g * 8) * 64 + lane;
          i4v alo[4], ahi[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint4 x0 = ag[k * 64], x1 = ag[(4 + k) * 64];
            alo[k] = i4v{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w};
            ahi[k] = i4v{(int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
          }
#pragma unroll
          for (int mi = 0; mi < VM; ++mi) {
            i4v lo, hi;
            mask_bytes_pow2(xor_planes(vw[g][nt], walsh_mask(VB, mi)), lo, hi);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              if constexpr (decltype(first)::value)
                acc[mi][k] = __builtin_amdgcn_mfma_i32_16x16x64_i8(alo[k], lo, i4v{0, 0, 0, 0}, 0, 0, 0);
              else
                acc[mi][k] = __builtin_amdgcn_mfma_i32_16x16x64_i8(alo[k], lo, acc[mi][k], 0, 0, 0);
              acc[mi][k] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ahi[k], hi, acc[mi][k], 0, 0, 0);
            }
          }
        };
        // all four groups, also past the block's end: their weights are zero
        // (branch-free, so the accumulators stay in one set of registers)
        __builtin_amdgcn_s_setprio(1);
        vgroup(std::integral_constant<int, 0>{}, std::true_type{});
        vgroup(std::integral_constant<int, 1>{}, std::false_type{});
        vgroup(std::integral_constant<int, 2>{}, std::false_type{});
        vgroup(std::integral_constant<int, 3>{}, std::false_type{});
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float o = 0.f;
#pragma unroll
          for (int mi = 0; mi < VM; ++mi) {
            const float M = fmaf(fmaf(fmaf((float)acc[mi][3][i], 256.f, (float)acc[mi][2][i]), 256.f,
                                      (float)acc[mi][1][i]),
                                 256.f, (float)acc[mi][0][i]);
            o = fmaf(wv[mi], fmaf(2.f, M, -wtv[i]), o);
          }
          O[nt][i] = fmaf(O[nt][i], rhv[i], scv[i] * o);
        }
      }
    }
  }
  // weight sums per head: lanes hs, hs + 16, hs + 32, hs + 48 of each wave, then the waves
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (lane < 16) lred[wave][lane] = lsum;
  __syncthreads();
  if (a.nchunks == 1) {
    // one chunk covers the whole context: the output is finished here,
    // o = Pi^T o_rot / l (no partials, no merge launch). o_rot goes through LDS
    // (the logits' space, unused past the last block)
    float *orot = lg;  // [16][DD]
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) orot[(4 * vgl + i) * DD + 32 * wave + 16 * nt + vn] = O[nt][i];
    __syncthreads();
    // thread (coordinate j, heads h0 .. h0 + 7): column j of Pi against o_rot
    const int j = tid & (DD - 1), h0 = (tid >> 7) * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < DD; ++k) {
      const float p = a.rot[k * DD + j];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] = fmaf(p, orot[(h0 + u) * DD + k], acc[u]);
    }
    const int b2 = stream / a.kv_heads, kvh = stream - b2 * a.kv_heads;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int h = h0 + u;
      if (h < nh) {
        const float l = (lred[0][h] + lred[1][h]) + (lred[2][h] + lred[3][h]);
        const int vh = vh0 + h, qi = vh / a.group, qj = vh - qi * a.group;
        a.out[(((int64_t)b2 * a.n_q + qi) * a.q_heads + kvh * a.group + qj) * DD + j] = l > 0.f ? acc[u] / l : 0.f;
      }
    }
    return;
  }
  if (tid < nh) {
    pbase[tid * pstride + DD] = mrs;
    pbase[tid * pstride + DD + 1] = (lred[0][tid] + lred[1][tid]) + (lred[2][tid] + lred[3][tid]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hh = 4 * vgl + i;
    if (hh < nh) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) pbase[hh * pstride + 32 * wave + 16 * nt + vn] = O[nt][i];
    }
  }
}

bool prefill_supported(const tq_ctx *ctx, const tq_kv_cache *cache, int32_t q_heads, int n_q) {
  if (!ctx || !cache || ctx->d != DD) return false;
  if (cache->d_block_table != nullptr && (cache->page_tokens % PB) != 0) return false;
  if (cache->v.mse_bits < 1 || cache->v.mse_bits > 3) return false;
  if (cache->k.mse_bits < (cache->k.qjl ? 0 : 1) || cache->k.mse_bits > 4) return false;
  if (n_q < 2 || q_heads <= 0 || cache->kv_heads <= 0 || (q_heads % cache->kv_heads) != 0) return false;
  return (int64_t)n_q * (q_heads / cache->kv_heads) >= PH;
}

namespace {
struct PrefillShape {
  int hb, nchunks, chunk;
  int64_t units;
};
PrefillShape prefill_shape(const tq_kv_cache *cache, int32_t q_heads, int n_q) {
  PrefillShape s;
  const int vgroup = (q_heads / cache->kv_heads) * n_q;
  s.hb = (vgroup + PH - 1) / PH;
  s.units = (int64_t)cache->batch * cache->kv_heads * s.hb;
  const int maxlen = std::max(1, cache->host_max_len > 0 ? cache->host_max_len : cache->capacity);
  const int blocks = (maxlen + PB - 1) / PB;
  // split the context when the units alone give under ~1024 work-groups;
  // a work-group covers at most PCHUNK_MAX tokens
  int nch = (int)std::max<int64_t>(1, (1024 + s.units - 1) / s.units);
  nch = std::max(nch, (maxlen + PCHUNK_MAX - 1) / PCHUNK_MAX);
  nch = std::min(nch, blocks);
  s.chunk = ((blocks + nch - 1) / nch) * PB;
  s.nchunks = (maxlen + s.chunk - 1) / s.chunk;
  return s;
}
}  // namespace

size_t prefill_ws_bytes(const tq_kv_cache *cache, int32_t q_heads, int n_q) {
  const PrefillShape s = prefill_shape(cache, q_heads, n_q);
  const int vgroup = (q_heads / cache->kv_heads) * n_q;
  size_t b = (size_t)s.units * PFRAG_WORDS * 4;
  b = (b + 255) & ~(size_t)255;
  b += (size_t)s.units * PH * 4 * sizeof(float);
  b = (b + 255) & ~(size_t)255;
  b += (size_t)cache->batch * cache->kv_heads * vgroup * s.nchunks * (DD + 2) * sizeof(float);
  return b;
}

template <int KB, bool QJL, bool NF16>
static hipError_t launch_prefill_kn(const PrefillArgs &a, int vb, dim3 grid, hipStream_t st) {
  switch (vb) {
    case 1: hipLaunchKernelGGL((prefill_kernel<KB, 1, QJL, NF16>), grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<KB, 2, QJL, NF16>), grid, dim3(256), 0, st, a); break;
    case 3: hipLaunchKernelGGL((prefill_kernel<KB, 3, QJL, NF16>), grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KB, bool QJL>
static hipError_t launch_prefill_k(const PrefillArgs &a, int vb, dim3 grid, hipStream_t st) {
  return a.nf16 ? launch_prefill_kn<KB, QJL, true>(a, vb, grid, st) : launch_prefill_kn<KB, QJL, false>(a, vb, grid, st);
}

hipError_t launch_prefill(const tq_ctx *ctx, const tq_kv_cache *cache, const void *q, int is_bf16, int32_t q_heads,
                          int n_q, int causal, float scale, float *out, void *ws, hipStream_t st, hipEvent_t ev0,
                          hipEvent_t ev1) {
  const PrefillShape s = prefill_shape(cache, q_heads, n_q);
  PrefillArgs a = {};
  a.kbits = cache->k.bits;
  a.knorm = cache->k.norms;
  a.vbits = cache->v.bits;
  a.vnorm = cache->v.norms;
  a.seq_len = cache->d_seq_len;
  a.map = cache_map(cache, 0);
  a.nf16 = cache->k.norm_f16;
  a.kv_heads = cache->kv_heads;
  a.capacity = cache->capacity;
  a.q_heads = q_heads;
  a.group = q_heads / cache->kv_heads;
  a.n_q = n_q;
  a.causal = causal;
  a.vgroup = a.group * n_q;
  a.hb = s.hb;
  a.kv_streams = cache->batch * cache->kv_heads;
  a.chunk = s.chunk;
  a.nchunks = s.nchunks;
  a.q = q;
  a.q_bf16 = is_bf16;
  a.rs_t = ctx->d_rs_t;
  a.tables = ctx->d_tables;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.qjl_scale = (float)(std::sqrt(M_PI / 2.0) / DD);
  char *p = (char *)ws;
  a.qfrag = (uint32_t *)p;
  p += ((size_t)s.units * PFRAG_WORDS * 4 + 255) & ~(size_t)255;
  a.qconst = (float *)p;
  p += ((size_t)s.units * PH * 4 * sizeof(float) + 255) & ~(size_t)255;
  a.partial = (float *)p;
  a.rot = ctx->d_rot;
  a.out = out;
  hipLaunchKernelGGL(prefill_prep_kernel, dim3((unsigned)s.units), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)(s.units * s.nchunks));
  const int kb = cache->k.mse_bits, vb = cache->v.mse_bits;
  if (ev0 && (e = hipEventRecord(ev0, st)) != hipSuccess) return e;
  if (cache->k.qjl) {
    switch (kb) {
      case 0: e = launch_prefill_k<0, true>(a, vb, grid, st); break;
      case 1: e = launch_prefill_k<1, true>(a, vb, grid, st); break;
      case 2: e = launch_prefill_k<2, true>(a, vb, grid, st); break;
      case 3: e = launch_prefill_k<3, true>(a, vb, grid, st); break;
      case 4: e = launch_prefill_k<4, true>(a, vb, grid, st); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (kb) {
      case 1: e = launch_prefill_k<1, false>(a, vb, grid, st); break;
      case 2: e = launch_prefill_k<2, false>(a, vb, grid, st); break;
      case 3: e = launch_prefill_k<3, false>(a, vb, grid, st); break;
      case 4: e = launch_prefill_k<4, false>(a, vb, grid, st); break;
      default: return hipErrorInvalidValue;
    }
  }
  if (e != hipSuccess) return e;
  if (ev1 && (e = hipEventRecord(ev1, st)) != hipSuccess) return e;
  if (s.nchunks == 1) return hipSuccess;  // the kernel wrote the output
  return launch_merge_partials(ctx, cache, q_heads, n_q, a.partial, s.nchunks, out, st);
}

}  // namespace tq
