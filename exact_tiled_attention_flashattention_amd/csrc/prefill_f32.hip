// fp32 prefill: the same tiled online-softmax method in full fp32 on the
// vector ALUs ("Phase 07 · 12: KV cache, Flash Attention and inference
// optimisation", sections "tiling trick" and "Build it, step 2").
//
// The fp32 path exists for exactness checks at fp32 tolerance and for small
// single-head problems; it is latency-bound, not a throughput path. A
// workgroup of 256 threads owns 64 query rows of one head; 4 lanes share a
// row, each holding a quarter of q and of the output (interleaved 16-byte
// chunks so the 4 lanes read adjacent LDS words). K/V tiles of 32 keys are
// staged in LDS and broadcast to all rows. A row's dot product is finished
// with two lane exchanges; the running max/sum update is the same as in the
// bf16 kernel.
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kRows = 64;
constexpr int kKeys = 32;

struct F32Params {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int B, Hq, Hkv, Nq, Nk, G, n_qblk;
  float c;  // scale * log2(e)
  int causal;
  int q_offset;
};

template <int D>
__global__ __launch_bounds__(256) void prefill_f32_kernel(F32Params p) {
  constexpr int NE = D / 16;  // float4 chunks per lane
  __shared__ __attribute__((aligned(16))) float kt[kKeys * D];
  __shared__ __attribute__((aligned(16))) float vt[kKeys * D];

  const int tid = threadIdx.x;
  const int part = tid & 3;
  const int row = tid >> 2;
  const int qblk = blockIdx.x % p.n_qblk;
  const int bh = blockIdx.x / p.n_qblk;
  const int hq = bh % p.Hq;
  const int b = bh / p.Hq;
  const int kvh = hq / p.G;
  const int my_q = qblk * kRows + row;

  f32x4_t qv[NE], ov[NE];
  const float* qp = p.q + (((long long)b * p.Hq + hq) * p.Nq + my_q) * D;
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    qv[e] = (my_q < p.Nq) ? *reinterpret_cast<const f32x4_t*>(qp + 4 * (part + 4 * e))
                          : f32x4_t{0.f, 0.f, 0.f, 0.f};
    ov[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  int kend = p.Nk;
  if (p.causal) {
    const int last = min(qblk * kRows + kRows, p.Nq) - 1;
    const long long lim = (long long)last + p.q_offset + 1;
    if (lim < kend) kend = (int)(lim < 0 ? 0 : lim);
  }
  const long long lim_row = (long long)my_q + p.q_offset;
  const float* kg = p.k + ((long long)b * p.Hkv + kvh) * (long long)p.Nk * D;
  const float* vg = p.v + ((long long)b * p.Hkv + kvh) * (long long)p.Nk * D;

  float m_run = neg_inf();
  float l_run = 0.f;
  for (int k0 = 0; k0 < kend; k0 += kKeys) {
    __syncthreads();
    for (int c = tid; c < kKeys * D / 4; c += 256) {
      const int r = c / (D / 4);
      const int col = (c % (D / 4)) * 4;
      f32x4_t kk = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (k0 + r < p.Nk) {
        kk = *reinterpret_cast<const f32x4_t*>(kg + (long long)(k0 + r) * D + col);
        vv = *reinterpret_cast<const f32x4_t*>(vg + (long long)(k0 + r) * D + col);
      }
      *reinterpret_cast<f32x4_t*>(kt + r * D + col) = kk;
      *reinterpret_cast<f32x4_t*>(vt + r * D + col) = vv;
    }
    __syncthreads();

    float s[kKeys];
    float mx = neg_inf();
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const f32x4_t kk = *reinterpret_cast<const f32x4_t*>(kt + j * D + 4 * (part + 4 * e));
        a = __builtin_fmaf(qv[e][0], kk[0], a);
        a = __builtin_fmaf(qv[e][1], kk[1], a);
        a = __builtin_fmaf(qv[e][2], kk[2], a);
        a = __builtin_fmaf(qv[e][3], kk[3], a);
      }
      a += __shfl_xor(a, 1, 64);
      a += __shfl_xor(a, 2, 64);
      const int key = k0 + j;
      const bool vis = key < p.Nk && (!p.causal || key <= lim_row);
      s[j] = vis ? a : neg_inf();
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx * p.c);
    const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e) ov[e] *= alpha;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      const float pj = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j], p.c, -m_use));
      rs += pj;
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const f32x4_t vv = *reinterpret_cast<const f32x4_t*>(vt + j * D + 4 * (part + 4 * e));
        ov[e][0] = __builtin_fmaf(pj, vv[0], ov[e][0]);
        ov[e][1] = __builtin_fmaf(pj, vv[1], ov[e][1]);
        ov[e][2] = __builtin_fmaf(pj, vv[2], ov[e][2]);
        ov[e][3] = __builtin_fmaf(pj, vv[3], ov[e][3]);
      }
    }
    l_run = l_run * alpha + rs;
  }

  if (my_q < p.Nq) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float* op = p.o + (((long long)b * p.Hq + hq) * p.Nq + my_q) * D;
#pragma unroll
    for (int e = 0; e < NE; ++e)
      *reinterpret_cast<f32x4_t*>(op + 4 * (part + 4 * e)) = ov[e] * inv;
    if (part == 0 && p.lse != nullptr)
      p.lse[((long long)b * p.Hq + hq) * p.Nq + my_q] =
          l_run > 0.f ? (m_run + __builtin_amdgcn_logf(l_run)) * kLn2 : neg_inf();
  }
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s) {
  F32Params pp;
  pp.q = static_cast<const float*>(a.q);
  pp.k = static_cast<const float*>(a.k);
  pp.v = static_cast<const float*>(a.v);
  pp.o = static_cast<float*>(a.o);
  pp.lse = a.lse;
  pp.B = a.B;
  pp.Hq = a.Hq;
  pp.Hkv = a.Hkv;
  pp.Nq = a.Nq;
  pp.Nk = a.Nk;
  pp.G = a.Hq / a.Hkv;
  pp.n_qblk = (a.Nq + kRows - 1) / kRows;
  pp.c = a.scale * kLog2e;
  pp.causal = a.causal;
  pp.q_offset = a.q_offset;
  const long long nblocks = (long long)pp.n_qblk * a.B * a.Hq;
  if (nblocks <= 0) return hipSuccess;
  if (nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.d == 128)
    hipLaunchKernelGGL(prefill_f32_kernel<128>, dim3((int)nblocks), dim3(256), 0, s, pp);
  else
    hipLaunchKernelGGL(prefill_f32_kernel<64>, dim3((int)nblocks), dim3(256), 0, s, pp);
  return hipGetLastError();
}

}  // namespace attn
