// fp32 prefill: the same tiled online-softmax method in full fp32 on the
// vector ALUs ("Phase 07 · 12: KV cache, Flash Attention and inference
// optimisation", sections "tiling trick" and "Build it, step 2").
//
// The fp32 path exists for exactness checks at fp32 tolerance and for small
// single-head problems, where the time is latency: a launch, one round of
// loads and a chain of dependent arithmetic per row. So the work is spread
// thin. A workgroup owns 16 query rows of one head (4 lanes per row, each
// holding a quarter of q and of the output in interleaved 16-byte chunks)
// and its 16 waves take every 16th tile of keys each, so a row's chain of
// keys is split 16 ways. Each wave streams its own tiles through a private
// double buffer in LDS with direct global->LDS loads (no workgroup barrier
// inside the loop), runs the running (max, sum) update over them, and at the
// end the 16 partial results of each row are merged through LDS with the
// same log-sum-exp weights as the split-KV decode.
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kRows = 16;    // query rows per workgroup
constexpr int kWaves = 16;   // key-parallel waves per workgroup
constexpr int kBufferFlags = 0x00020000;

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
__global__ __launch_bounds__(kWaves * 64) void prefill_f32_kernel(F32Params p) {
  constexpr int NE = D / 16;       // float4 chunks per lane
  constexpr int TK = 512 / D;      // keys per staged tile (2 KiB of K, 2 KiB of V)
  constexpr int TILEF = TK * D;    // floats per K (or V) tile
  constexpr int NL = TILEF / 256;  // 16-byte direct loads per lane per tile and tensor
  // per wave: [buffer 0: K, V][buffer 1: K, V]; reused for the final merge
  __shared__ __attribute__((aligned(16))) float lds[kWaves * 4 * TILEF];
  __shared__ float mrow[kWaves][kRows];
  __shared__ float lrow[kWaves][kRows];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int part = lane & 3;
  const int row = lane >> 2;
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
  const int ntiles = (kend + TK - 1) / TK;
  const long long lim_row = (long long)my_q + p.q_offset;
  const float* kg = p.k + ((long long)b * p.Hkv + kvh) * (long long)p.Nk * D;
  const float* vg = p.v + ((long long)b * p.Hkv + kvh) * (long long)p.Nk * D;
  float* wl = lds + wave * 4 * TILEF;

  // tile t of this head into buffer `buf` of this wave: lane l moves bytes
  // [16 l + 1024 i, +16) of the tile; keys past Nk read as zeros (the
  // resource ends at the head's last key)
  auto stage = [&](int t, int buf) __attribute__((always_inline)) {
    const long long off = (long long)t * TILEF;
    const long long left = ((long long)p.Nk * D - off) * 4;
    const int range = (int)(left < 0 ? 0 : (left > TILEF * 4 ? TILEF * 4 : left));
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kg + off), 0, range, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vg + off), 0, range, kBufferFlags);
    float* kd = wl + buf * 2 * TILEF;
    float* vd = kd + TILEF;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (ATTN_LDS void*)(kd + 256 * i), 16,
                                               16 * lane + 1024 * i, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (ATTN_LDS void*)(vd + 256 * i), 16,
                                               16 * lane + 1024 * i, 0, 0, 0);
    }
  };

  float m_run = neg_inf();  // base-2 running max of this row (this wave's keys)
  float l_run = 0.f;
  int buf = 0;
  if (wave < ntiles) stage(wave, 0);
  for (int t = wave; t < ntiles; t += kWaves) {
    if (t + kWaves < ntiles) {
      stage(t + kWaves, buf ^ 1);
      // vmcnt(2 NL): all but the next tile's loads have landed
      __builtin_amdgcn_s_waitcnt(0x0F70 | ((2 * NL) & 15) | (((2 * NL) >> 4) << 14));
    } else {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    }
    asm volatile("" ::: "memory");  // the tile's LDS reads stay after the wait
    const float* kt = wl + buf * 2 * TILEF;
    const float* vt = kt + TILEF;
    const int k0 = t * TK;

    float s[TK];
    float mx = neg_inf();
#pragma unroll
    for (int j = 0; j < TK; ++j) {
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
    for (int j = 0; j < TK; ++j) {
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
    buf ^= 1;
  }

  // ---- merge the waves' partial results of each row ----------------------------
  // O = Σ_w 2^(m_w − M) O_w / Σ_w 2^(m_w − M) l_w with M = max_w m_w (an
  // empty partial has m_w = −inf and weight 0)
  __syncthreads();  // every wave is done with its tiles: the buffers become the merge area
  float* mo = lds + (wave * kRows + row) * D;
#pragma unroll
  for (int e = 0; e < NE; ++e) *reinterpret_cast<f32x4_t*>(mo + 4 * (part + 4 * e)) = ov[e];
  if (part == 0) {
    mrow[wave][row] = m_run;
    lrow[wave][row] = l_run;
  }
  __syncthreads();
  if (wave == 0 && my_q < p.Nq) {
    float M = neg_inf();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mrow[w][row]);
    const float M_use = (M == neg_inf()) ? 0.f : M;
    float L = 0.f;
    f32x4_t acc[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = __builtin_amdgcn_exp2f(mrow[w][row] - M_use);  // 0 for an empty partial
      L += wt * lrow[w][row];
      const float* src = lds + (w * kRows + row) * D;
#pragma unroll
      for (int e = 0; e < NE; ++e)
        acc[e] += wt * *reinterpret_cast<const f32x4_t*>(src + 4 * (part + 4 * e));
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    float* op = p.o + (((long long)b * p.Hq + hq) * p.Nq + my_q) * D;
#pragma unroll
    for (int e = 0; e < NE; ++e)
      *reinterpret_cast<f32x4_t*>(op + 4 * (part + 4 * e)) = acc[e] * inv;
    if (part == 0 && p.lse != nullptr)
      p.lse[((long long)b * p.Hq + hq) * p.Nq + my_q] =
          L > 0.f ? (M + __builtin_amdgcn_logf(L)) * kLn2 : neg_inf();
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
    hipLaunchKernelGGL(prefill_f32_kernel<128>, dim3((int)nblocks), dim3(kWaves * 64), 0, s, pp);
  else
    hipLaunchKernelGGL(prefill_f32_kernel<64>, dim3((int)nblocks), dim3(kWaves * 64), 0, s, pp);
  return hipGetLastError();
}

}  // namespace attn
