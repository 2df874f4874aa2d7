// Device-side helpers shared by the gfx950 attention kernels.
//
// Register layouts of the two bf16 MFMA shapes used here (64-lane wave,
// lane l, operand element j, accumulator register i):
//   v_mfma_f32_32x32x16_bf16: A[m = l%32][k = 8*(l/32) + j],
//                             B[k = 8*(l/32) + j][n = l%32],
//                             D[m = 8*(i/4) + 4*(l/32) + i%4][n = l%32]
//   v_mfma_f32_16x16x32_bf16: A[m = l%16][k = 8*(l/16) + j],
//                             B[k = 8*(l/16) + j][n = l%16],
//                             D[m = 4*(l/16) + i][n = l%16]
// ds_read_tr16_b64 (transposing LDS read): inside each 16-lane group, lane i
// receives as element j the (i%4)-th 16-bit value of the 8-byte chunk that
// lane 4*j + i/4 of the group addresses.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kBlockTokens = 16;  // tokens per physical block of a paged cache

#define ATTN_LDS __attribute__((address_space(3)))

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Two fp32 values -> two bf16 (round to nearest even) in one dword, a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t v = {a, b};
  bf16x2_t h = __builtin_convertvector(v, bf16x2_t);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// max over the two 32-lane halves of the wave (lanes l and l^32); NaN-propagating.
__device__ __forceinline__ float max_across_halves(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float sum_across_halves(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
// the same over lanes l and l^16.
__device__ __forceinline__ float max_across_rows16(float x) {
  auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float sum_across_rows16(float x) {
  auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Where logical token t of sequence b lives in a K/V cache, as an element
// offset of its (kv head 0) row; -1 when the token has no valid storage.
// Paged: block_table[b][t / 16], slot t % 16 of a [num_blocks, 16, Hkv, D]
// pool. Contiguous (table == nullptr): row t of sequence b of a
// [B, max_len, Hkv, D] cache.
struct CacheView {
  const int32_t* table;  // [B, max_blocks] or nullptr
  int max_blocks;
  int num_blocks;
  int max_len;
  int hkv;
  int d;
};

__device__ __forceinline__ long long cache_row(const CacheView& c, int b, int t) {
  if (t < 0 || t >= c.max_len) return -1;
  if (c.table == nullptr) {
    return ((long long)b * c.max_len + t) * c.hkv * c.d;
  }
  const int i = t / kBlockTokens;
  if (i >= c.max_blocks) return -1;
  const int blk = c.table[(long long)b * c.max_blocks + i];
  if (blk < 0 || blk >= c.num_blocks) return -1;
  return ((long long)blk * kBlockTokens + (t % kBlockTokens)) * c.hkv * c.d;
}

// Keys of sequence b that exist in the cache: seq_len clamped to the capacity.
__device__ __forceinline__ int cache_len_clamped(const CacheView& c, int seq_len) {
  int cap = c.max_len;
  if (c.table != nullptr) {
    const long long tcap = (long long)c.max_blocks * kBlockTokens;
    if (tcap < cap) cap = (int)tcap;
  }
  return seq_len < 0 ? 0 : (seq_len > cap ? cap : seq_len);
}

}  // namespace attn
