// Device-side definitions shared by the kernel sources of libtq (gfx950, wave64):
// MFMA operand vector types, the Walsh subsets of the bit planes, and the bit
// mask operands built from plane words.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace tq {

constexpr int DD = 128;            // head dim
constexpr int DW = DD / 32;        // 32-coordinate groups

typedef int i4v __attribute__((ext_vector_type(4)));
typedef float f4v __attribute__((ext_vector_type(4)));
typedef int i8v __attribute__((ext_vector_type(8)));

// bf16 bits (low 16 of b16) to fp32
__device__ __forceinline__ float bf16f(uint32_t b16) { return __uint_as_float(b16 << 16); }

// The i-th odd-cardinality subset of the B planes, ordered by (popcount, value).
__host__ __device__ constexpr int walsh_mask(int B, int i) {
  return i < B ? (1 << i) : (B == 3 ? 7 : (i == 4 ? 7 : i == 5 ? 11 : i == 6 ? 13 : 14));
}

// Plane index of the k-th member of the plane subset S.
__host__ __device__ constexpr int nth_plane(int S, int k) {
  for (int p = 0; p < 4; ++p)
    if (S & (1 << p)) {
      if (k == 0) return p;
      --k;
    }
  return 0;
}

// XOR of the plane words of subset S (one plane, or three in one bitop3).
template <int NP>
__device__ __forceinline__ uint32_t xor_planes(const uint32_t (&pl)[NP], int S) {
  if (__builtin_popcount(S) == 1) return pl[nth_plane(S, 0)];
  return __builtin_amdgcn_bitop3_b32(pl[nth_plane(S, 0)], pl[nth_plane(S, 1)], pl[nth_plane(S, 2)], 0x96);
}

// fp4 B operand of a Walsh mask from the B operands of the single planes: the AND
// masks commute with XOR, so each dword is the XOR of the planes' dwords
// (S is one of the odd subsets of at most four planes that walsh_mask lists:
// one plane or three; three take one three-input XOR per dword)
template <int NP>
__device__ __forceinline__ i8v walsh_fp4(const i8v (&sm)[NP], int S) {
  if (__builtin_popcount(S) == 1) return sm[nth_plane(S, 0)];
  const i8v &x = sm[nth_plane(S, 0)], &y = sm[nth_plane(S, 1)], &z = sm[nth_plane(S, 2)];
  i8v r = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int q = 0; q < 4; ++q)
    r[q] = (int)__builtin_amdgcn_bitop3_b32((uint32_t)x[q], (uint32_t)y[q], (uint32_t)z[q], 0x96);
  return r;
}

// Value B bytes of a token-major plane word: byte k' of dword q is bit q + 8k'
// of m, left in place (value b * 2^q; -128 b for q = 7).
__device__ __forceinline__ void mask_bytes_pow2(uint32_t m, i4v &lo, i4v &hi) {
  lo[0] = (int)(m & 0x01010101u);
  lo[1] = (int)(m & 0x02020202u);
  lo[2] = (int)(m & 0x04040404u);
  lo[3] = (int)(m & 0x08080808u);
  hi[0] = (int)(m & 0x10101010u);
  hi[1] = (int)(m & 0x20202020u);
  hi[2] = (int)(m & 0x40404040u);
  hi[3] = (int)(m & 0x80808080u);
}

// NPL consecutive dwords at byte offset off of a buffer resource, with the
// widest loads (dword alignment suffices for buffer loads); AUX is the cache
// policy field (2: non-temporal).
template <int NPL, int AUX>
__device__ __forceinline__ void buffer_load_words(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t (&w)[NPL]) {
  if constexpr (NPL == 1) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX);
  } else if constexpr (NPL == 2) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX);
    w[0] = x[0]; w[1] = x[1];
  } else if constexpr (NPL == 3) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, AUX);
    w[0] = x[0]; w[1] = x[1]; w[2] = x[2];
  } else {
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
    w[0] = x[0]; w[1] = x[1]; w[2] = x[2]; w[3] = x[3];
    if constexpr (NPL == 5) w[4] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 16u, 0, AUX);
  }
}

}  // namespace tq
