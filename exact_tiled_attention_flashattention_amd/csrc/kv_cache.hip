// Cache writes and reads that move stored bits only.
//
// kv_append: the decode step grows each layer's cache by the new tokens' K
// and V ("大模型面试笔记——Attention篇" §4: x_K <- Concat(x_K, t·W_K);
// "Phase 07 · 12: KV cache, Flash Attention and inference optimisation",
// "Build it, step 1"). Row r of sequence b goes to logical position
// cache_lens[b] + r, which the page table maps to block table[b][pos / 16],
// slot pos % 16 ("Paged attention" section of the same page).
// gather: the inverse walk, used to check the page-table addressing bit for
// bit. Both use cache_row(), the helper the decode kernel uses.
// One thread moves 16 bytes; a K/V row of d elements is d*elem/16 threads,
// so a wave writes whole rows.
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

struct CopyParams {
  const float* k_scale;
  const float* v_scale;
  const char* src_k;
  const char* src_v;
  char* dst_k;
  char* dst_v;
  CacheView cv;
  const int32_t* lens;
  int eb;  // element bytes
  int B, Hkv, Nnew, d;
  long long total;
};

__global__ __launch_bounds__(256) void kv_append_kernel(CopyParams p) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= p.total) return;
  const int cpr = p.d * p.eb / 16;
  const int ch = (int)(idx % cpr);
  long long rr = idx / cpr;
  const int kvh = (int)(rr % p.Hkv);
  rr /= p.Hkv;
  const int r = (int)(rr % p.Nnew);
  const int b = (int)(rr / p.Nnew);
  const long long t = (long long)p.lens[b] + r;
  if (t < 0 || t > 0x7fffffffLL) return;
  const long long row = cache_row(p.cv, b, (int)t);
  if (row < 0) return;
  const long long src = (((long long)b * p.Nnew + r) * p.Hkv + kvh) * p.d * p.eb + ch * 16;
  const long long dst = (row + (long long)kvh * p.d) * p.eb + ch * 16;
  *reinterpret_cast<u32x4_t*>(p.dst_k + dst) = *reinterpret_cast<const u32x4_t*>(p.src_k + src);
  *reinterpret_cast<u32x4_t*>(p.dst_v + dst) = *reinterpret_cast<const u32x4_t*>(p.src_v + src);
}

// kv_append into an E4M3 cache: one thread turns 8 bf16 elements of a new
// row into 8 codes. code = nearest-even(clamp(x / scale, -448, 448)): one
// IEEE fp32 division, a NaN-preserving clamp (the conversion itself turns
// magnitudes past 464 into NaN), then the hardware conversion, which rounds
// to nearest even.
__global__ __launch_bounds__(256) void kv_append_fp8_kernel(CopyParams p) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= p.total) return;
  const int cpr = p.d / 8;
  const int ch = (int)(idx % cpr);
  long long rr = idx / cpr;
  const int kvh = (int)(rr % p.Hkv);
  rr /= p.Hkv;
  const int r = (int)(rr % p.Nnew);
  const int b = (int)(rr / p.Nnew);
  const long long t = (long long)p.lens[b] + r;
  if (t < 0 || t > 0x7fffffffLL) return;
  const long long row = cache_row(p.cv, b, (int)t);
  if (row < 0) return;
  const long long src = ((((long long)b * p.Nnew + r) * p.Hkv + kvh) * p.d + ch * 8) * 2;
  const long long dst = row + (long long)kvh * p.d + ch * 8;
  const float sk = p.k_scale[kvh];
  const float sv = p.v_scale[kvh];
  // the two elements of bf16 pair w, divided by s and clamped
  auto pair = [](uint32_t w, float s, float& y0, float& y1) {
    y0 = __uint_as_float(w << 16) / s;  // bf16 -> fp32 is exact
    y1 = __uint_as_float(w & 0xffff0000u) / s;
    y0 = __builtin_elementwise_minimum(__builtin_elementwise_maximum(y0, -448.f), 448.f);
    y1 = __builtin_elementwise_minimum(__builtin_elementwise_maximum(y1, -448.f), 448.f);
  };
  auto encode8 = [&](u32x4_t x, float s) {
    float a0, a1, b0, b1, c0, c1, d0, d1;
    pair(x[0], s, a0, a1);
    pair(x[1], s, b0, b1);
    pair(x[2], s, c0, c1);
    pair(x[3], s, d0, d1);
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);  // bytes 0, 1
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(b0, b1, lo, true);       // bytes 2, 3
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(d0, d1, hi, true);
    return u32x2_t{(uint32_t)lo, (uint32_t)hi};
  };
  const u32x4_t xk = *reinterpret_cast<const u32x4_t*>(p.src_k + src);
  const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(p.src_v + src);
  *reinterpret_cast<u32x2_t*>(p.dst_k + dst) = encode8(xk, sk);
  *reinterpret_cast<u32x2_t*>(p.dst_v + dst) = encode8(xv, sv);
}

// out [B, max_len, Hkv, d]; one thread per 16 bytes of every output row.
__global__ __launch_bounds__(256) void gather_kernel(CopyParams p) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= p.total) return;
  const int cpr = p.d * p.eb / 16;
  const int ch = (int)(idx % cpr);
  long long rr = idx / cpr;
  const int kvh = (int)(rr % p.Hkv);
  rr /= p.Hkv;
  const int t = (int)(rr % p.cv.max_len);
  const int b = (int)(rr / p.cv.max_len);
  const int n = cache_len_clamped(p.cv, p.lens[b]);
  if (t >= n) return;
  const long long row = cache_row(p.cv, b, t);
  if (row < 0) return;
  const long long src = (row + (long long)kvh * p.d) * p.eb + ch * 16;
  const long long dst = (((long long)b * p.cv.max_len + t) * p.Hkv + kvh) * p.d * p.eb + ch * 16;
  *reinterpret_cast<u32x4_t*>(p.dst_k + dst) = *reinterpret_cast<const u32x4_t*>(p.src_k + src);
}

CopyParams make_params(const CacheCopyArgs& a) {
  CopyParams p;
  p.src_k = static_cast<const char*>(a.src_k);
  p.src_v = static_cast<const char*>(a.src_v);
  p.dst_k = static_cast<char*>(a.dst_k);
  p.dst_v = static_cast<char*>(a.dst_v);
  p.cv.table = a.block_table;
  p.cv.max_blocks = a.max_blocks;
  p.cv.num_blocks = a.num_blocks;
  p.cv.max_len = a.max_seq_len;
  p.cv.hkv = a.Hkv;
  p.cv.d = a.d;
  p.lens = a.lens;
  p.eb = a.elem_bytes;
  p.B = a.B;
  p.Hkv = a.Hkv;
  p.Nnew = a.Nnew;
  p.d = a.d;
  p.k_scale = a.k_scale;
  p.v_scale = a.v_scale;
  p.total = 0;
  return p;
}

hipError_t launch_copy(void (*kern)(CopyParams), CopyParams p, hipStream_t s) {
  if (p.total <= 0) return hipSuccess;
  const long long blocks = (p.total + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(kern, dim3((int)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_append(const CacheCopyArgs& a, hipStream_t s) {
  CopyParams p = make_params(a);
  p.total = (long long)a.B * a.Nnew * a.Hkv * (a.d * a.elem_bytes / 16);
  return launch_copy(kv_append_kernel, p, s);
}

hipError_t launch_kv_append_fp8(const CacheCopyArgs& a, hipStream_t s) {
  CopyParams p = make_params(a);
  p.total = (long long)a.B * a.Nnew * a.Hkv * (a.d / 8);
  return launch_copy(kv_append_fp8_kernel, p, s);
}

hipError_t launch_gather(const CacheCopyArgs& a, hipStream_t s) {
  CopyParams p = make_params(a);
  p.total = (long long)a.B * a.max_seq_len * a.Hkv * (a.d * a.elem_bytes / 16);
  return launch_copy(gather_kernel, p, s);
}

}  // namespace attn
