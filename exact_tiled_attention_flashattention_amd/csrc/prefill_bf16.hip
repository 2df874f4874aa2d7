// Causal / non-causal GQA prefill, bf16 inputs, fp32 accumulation, gfx950 MFMA.
//
// Method ("Phase 07 · 12: KV cache, Flash Attention and inference
// optimisation", section "tiling trick"; "大模型面试笔记——Attention篇" §2):
// for each block of query rows, stream K/V tiles through on-chip memory,
// compute the tile's scores, fold them into a running (max, sum) per row,
// rescale the partial output when the max grows, accumulate P·V, and write
// the output once. Scores and probabilities live only in registers.
//
// Mapping onto CDNA4:
//   * A workgroup is 4 waves. The waves share one K/V head: with a group of
//     G = Hq/Hkv query heads ("Effizienz", "GQA im leicht lesbaren Code")
//     the 4 waves take 4 heads of the group at the same 32 positions (G % 4
//     == 0), else fewer heads at more positions. Every K/V tile is read from
//     HBM/L2 once per workgroup and used by all 4 waves.
//   * Each wave owns 32 query rows. Scores are computed transposed,
//     Sᵀ = K·Qᵀ, with v_mfma_f32_32x32x16_bf16 (K from LDS as the A
//     operand, Qᵀ held in registers as the B operand), so each lane holds
//     one query row (lane % 32) and 32 of the tile's 64 keys. The row max
//     and row sum need one cross-half exchange (permlane32 swap).
//   * The probabilities in the Sᵀ accumulator layout are already the B
//     operand (Pᵀ) of Oᵀ = Vᵀ·Pᵀ after a bf16 pack; Vᵀ comes straight out of
//     the row-major V tile in LDS through the transposing read
//     ds_read_tr16_b64. Oᵀ stays in 64 fp32 accumulators per lane.
//   * K/V tiles (64 keys) are double-buffered: the next tile's global loads
//     are in flight while the current one is computed.
//   * Softmax runs in base 2 with scale·log2(e) folded into one FMA.
//   * Causal workgroups are launched longest-first (highest query block
//     first) and skip every tile past their last row's diagonal; only tiles
//     that cross the diagonal or the ragged end of K are masked.
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kBN = 64;  // keys per tile

struct PrefillParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float* lse;
  int B, Hq, Hkv, Nq, Nk;
  int G;       // Hq / Hkv
  int hw;      // heads per workgroup (1, 2 or 4)
  int pw;      // 32-row slices per head in a workgroup (4 / hw)
  int n_qblk;  // query blocks of 32 * pw rows
  int n_hgrp;  // workgroups per K/V head and query block (G / hw)
  float c;     // scale * log2(e)
  int q_offset;
};

template <int D>
struct Smem {
  static constexpr int kStride = D + 8;  // bf16 per LDS row: 16-byte pad against bank conflicts
  static constexpr int kTile = kBN * kStride;
  static constexpr int kChunks = kBN * D / 8;       // 16-byte chunks per K (or V) tile
  static constexpr int kPerThread = kChunks / (kWaves * 64);
};

template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void prefill_bf16_kernel(PrefillParams p) {
  constexpr int NDC = D / 16;  // k-steps of the Q·Kᵀ contraction
  constexpr int NDB = D / 32;  // 32-row blocks of Oᵀ
  constexpr int STR = Smem<D>::kStride;
  constexpr int TILE = Smem<D>::kTile;
  constexpr int NL = Smem<D>::kPerThread;
  __shared__ __attribute__((aligned(16))) __bf16 lds[2 * 2 * TILE];  // [stage][K, V][tile]

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  // ---- which rows this workgroup and wave own --------------------------------
  const int per_q = p.B * p.Hkv * p.n_hgrp;
  const int qrank = blockIdx.x / per_q;
  int rest = blockIdx.x - qrank * per_q;
  const int qblk = CAUSAL ? (p.n_qblk - 1 - qrank) : qrank;  // longest first
  const int hg = rest % p.n_hgrp;
  rest /= p.n_hgrp;
  const int kvh = rest % p.Hkv;
  const int b = rest / p.Hkv;

  const int head_local = wave % p.hw;
  const int sub = wave / p.hw;
  const int hq = kvh * p.G + hg * p.hw + head_local;
  const int q0 = qblk * 32 * p.pw;
  const int my_q = q0 + sub * 32 + l32;

  int kend = p.Nk;
  if (CAUSAL) {
    const int last_row = min(q0 + 32 * p.pw, p.Nq) - 1;
    const long long lim = (long long)last_row + p.q_offset + 1;
    if (lim < kend) kend = (int)(lim < 0 ? 0 : lim);
  }
  const int ntiles = (kend + kBN - 1) / kBN;
  // first key index at which some row of the workgroup needs masking
  long long mask_from = p.Nk;
  if (CAUSAL) {
    const long long first = (long long)q0 + p.q_offset + 1;
    if (first < mask_from) mask_from = first;
  }

  // ---- Qᵀ as the B operand: lane holds row my_q, d = 16*dc + 8*g + j ---------
  bf16x8_t qf[NDC];
  {
    const __bf16* qp = p.q + (((long long)b * p.Hq + hq) * p.Nq + my_q) * D + 8 * g;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      if (my_q < p.Nq)
        qf[dc] = *reinterpret_cast<const bf16x8_t*>(qp + 16 * dc);
      else
        qf[dc] = bf16x8_t{};
    }
  }

  const long long kv_base = ((long long)b * p.Hkv + kvh) * (long long)p.Nk * D;
  const __bf16* kg = p.k + kv_base;
  const __bf16* vg = p.v + kv_base;

  u32x4_t kr[NL], vr[NL];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int c = tid + i * kWaves * 64;
      const int row = c / (D / 8);
      const int col = (c % (D / 8)) * 8;
      if (k0 + row < p.Nk) {
        const long long off = (long long)(k0 + row) * D + col;
        kr[i] = *reinterpret_cast<const u32x4_t*>(kg + off);
        vr[i] = *reinterpret_cast<const u32x4_t*>(vg + off);
      } else {
        kr[i] = u32x4_t{0, 0, 0, 0};
        vr[i] = u32x4_t{0, 0, 0, 0};
      }
    }
  };
  auto lstore = [&](int stage) {
    __bf16* kl = lds + stage * 2 * TILE;
    __bf16* vl = kl + TILE;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int c = tid + i * kWaves * 64;
      const int row = c / (D / 8);
      const int col = (c % (D / 8)) * 8;
      *reinterpret_cast<u32x4_t*>(kl + row * STR + col) = kr[i];
      *reinterpret_cast<u32x4_t*>(vl + row * STR + col) = vr[i];
    }
  };

  f32x16_t acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16_t{};
  float m_run = neg_inf();
  float l_run = 0.f;

  // transposing-read address pattern inside a 16-lane group
  const int grp = lane >> 4;     // 0..3
  const int src = lane & 15;     // lane index inside the group
  const int tr_row = src >> 2;   // row offset 0..3
  const int tr_col = 4 * (src & 3) + 16 * (grp & 1);

  if (ntiles > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int stage = it & 1;
    const int k0 = it * kBN;
    if (it + 1 < ntiles) gload(k0 + kBN);

    const __bf16* kl = lds + stage * 2 * TILE;
    const __bf16* vl = kl + TILE;

    // Sᵀ[key][row] for the two 32-key halves of the tile
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16_t{};
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) {
        const bf16x8_t a =
            *reinterpret_cast<const bf16x8_t*>(kl + (kb * 32 + l32) * STR + 16 * dc + 8 * g);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[dc], s[kb], 0, 0, 0);
      }
    }

    // mask: only tiles that reach past the ragged end or the first row's diagonal
    if (k0 + kBN > mask_from || k0 + kBN > p.Nk) {
      const long long lim = CAUSAL ? (long long)my_q + p.q_offset : (long long)p.Nk;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
          const bool vis = key < p.Nk && (!CAUSAL || key <= lim);
          if (!vis) s[kb][i] = neg_inf();
        }
    }

    // online softmax (base 2): running max m_run, partial row sum l_run
    float mx = s[0][0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[0][i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[1][i]);
    mx = max_across_halves(mx);
    const float m_new = fmaxf(m_run, mx * p.c);
    const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;

    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], p.c, -m_use));
        s[kb][i] = e;
        rs += e;
      }
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;

    // Oᵀ += Vᵀ Pᵀ, 16 keys per MFMA
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        bf16x8_t pb;
        {
          f32x4_t lo = {s[kb][8 * hf + 0], s[kb][8 * hf + 1], s[kb][8 * hf + 2], s[kb][8 * hf + 3]};
          f32x4_t hi = {s[kb][8 * hf + 4], s[kb][8 * hf + 5], s[kb][8 * hf + 6], s[kb][8 * hf + 7]};
          bf16x4_t l4 = __builtin_convertvector(lo, bf16x4_t);
          bf16x4_t h4 = __builtin_convertvector(hi, bf16x4_t);
          pb = bf16x8_t{l4[0], l4[1], l4[2], l4[3], h4[0], h4[1], h4[2], h4[3]};
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int col = 32 * db + tr_col;
          const int r0 = kb * 32 + 16 * hf + 4 * g + tr_row;
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (ATTN_LDS i16x4_t*)(vl + r0 * STR + col));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (ATTN_LDS i16x4_t*)(vl + (r0 + 8) * STR + col));
          const bf16x4_t lob = __builtin_bit_cast(bf16x4_t, lo);
          const bf16x4_t hib = __builtin_bit_cast(bf16x4_t, hi);
          const bf16x8_t a = {lob[0], lob[1], lob[2], lob[3], hib[0], hib[1], hib[2], hib[3]};
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, acc[db], 0, 0, 0);
        }
      }

    if (it + 1 < ntiles) lstore(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = Oᵀ/l written once, LSE = ln(sum) + max --------------------
  const float l_tot = sum_across_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (my_q < p.Nq) {
    __bf16* op = p.o + (((long long)b * p.Hq + hq) * p.Nq + my_q) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        f32x4_t v4 = {acc[db][4 * ii] * inv, acc[db][4 * ii + 1] * inv, acc[db][4 * ii + 2] * inv,
                      acc[db][4 * ii + 3] * inv};
        *reinterpret_cast<bf16x4_t*>(op + 32 * db + 8 * ii + 4 * g) =
            __builtin_convertvector(v4, bf16x4_t);
      }
    if (g == 0 && p.lse != nullptr) {
      p.lse[((long long)b * p.Hq + hq) * p.Nq + my_q] =
          l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : neg_inf();
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch_typed(const PrefillParams& pp, int nblocks, hipStream_t s) {
  hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL>), dim3(nblocks), dim3(kWaves * 64), 0, s, pp);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
  PrefillParams pp;
  pp.q = static_cast<const __bf16*>(a.q);
  pp.k = static_cast<const __bf16*>(a.k);
  pp.v = static_cast<const __bf16*>(a.v);
  pp.o = static_cast<__bf16*>(a.o);
  pp.lse = a.lse;
  pp.B = a.B;
  pp.Hq = a.Hq;
  pp.Hkv = a.Hkv;
  pp.Nq = a.Nq;
  pp.Nk = a.Nk;
  pp.G = a.Hq / a.Hkv;
  pp.hw = (pp.G % 4 == 0) ? 4 : ((pp.G % 2 == 0) ? 2 : 1);
  pp.pw = kWaves / pp.hw;
  pp.n_qblk = (a.Nq + 32 * pp.pw - 1) / (32 * pp.pw);
  pp.n_hgrp = pp.G / pp.hw;
  pp.c = a.scale * kLog2e;
  pp.q_offset = a.q_offset;
  const long long nblocks = (long long)pp.n_qblk * a.B * a.Hkv * pp.n_hgrp;
  if (nblocks <= 0) return hipSuccess;
  if (nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.d == 128)
    return a.causal ? launch_typed<128, true>(pp, (int)nblocks, s)
                    : launch_typed<128, false>(pp, (int)nblocks, s);
  return a.causal ? launch_typed<64, true>(pp, (int)nblocks, s)
                  : launch_typed<64, false>(pp, (int)nblocks, s);
}

}  // namespace attn
