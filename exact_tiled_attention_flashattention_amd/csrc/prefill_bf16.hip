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
#include <type_traits>

#include "common.h"
#include "launch.h"

#ifndef ATTN_PREFILL_SCHED
#define ATTN_PREFILL_SCHED 0
#endif

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kBN = 64;         // keys per tile
constexpr float kTau = 8.0f;    // rescale only when a row max grows by more than 2^8
constexpr int kBufferFlags = 0x00020000;  // raw buffer resource, 32-bit dword data

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

// K/V tiles live in LDS unpadded (D*2 bytes per key row) with the 16-byte
// chunks of row r permuted by chunk ^ swz(r). The permutation makes both LDS
// read patterns conflict-free: the K reads (16 consecutive rows, one chunk)
// and the transposing V reads (4 consecutive rows x 4 chunks per 32 lanes).
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128)
    return ((row & 3) << 2) | ((row >> 2) & 3);
  else
    return (row >> 1) & 7;
}

template <int D>
__device__ __forceinline__ int lds_off(int row, int elem) {  // byte offset of element (row, elem)
  return row * (D * 2) + ((((elem >> 3) ^ swz<D>(row))) << 4) + ((elem & 7) << 1);
}

template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void prefill_bf16_kernel(PrefillParams p) {
  constexpr int NDC = D / 16;              // k-steps of the Q·Kᵀ contraction
  constexpr int NDB = D / 32;              // 32-row blocks of Oᵀ
  constexpr int CPR = D / 8;               // 16-byte chunks per key row
  constexpr int TILE = kBN * D * 2;        // bytes of one K (or V) tile
  constexpr int NI = TILE / (kWaves * 1024);  // direct loads per wave per tile and tensor
  // K runs one tile ahead of V: tile t's K sits in kb[t % 2], its V in vb[t % 2].
  // Four separate LDS objects, so the compiler can tell that the in-flight
  // direct loads never alias the buffers being read.
  __shared__ __attribute__((aligned(1024))) char kb0[TILE];
  __shared__ __attribute__((aligned(1024))) char kb1[TILE];
  __shared__ __attribute__((aligned(1024))) char vb0[TILE];
  __shared__ __attribute__((aligned(1024))) char vb1[TILE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  long long mask_from = p.Nk;  // first key some row of the workgroup cannot see
  if (CAUSAL) {
    const long long first = (long long)q0 + p.q_offset + 1;
    if (first < mask_from) mask_from = first;
  }
  // this lane's last visible key (clamped into int range)
  long long lim64 = CAUSAL ? (long long)my_q + p.q_offset : (long long)p.Nk - 1;
  if (lim64 > (long long)p.Nk - 1) lim64 = (long long)p.Nk - 1;
  if (lim64 < -1) lim64 = -1;
  const int lim = (int)lim64;

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

  // Direct global->LDS loads through buffer resources (one per K/V head, range
  // Nk rows): instruction i of this wave fills LDS bytes
  // [(wave*NI + i)*1024, +1024), lane l its 16 bytes at +16*l, i.e. physical
  // chunk (lin % CPR) of row (lin / CPR); the lane fetches the logical chunk
  // that the swizzle stores there. The per-lane byte offsets do not depend on
  // the tile; rows at or past Nk fall outside the resource and arrive as zeros
  // (those keys are masked).
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)kg, 0, p.Nk * D * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)vg, 0, p.Nk * D * 2, kBufferFlags);
  // Lane part of the byte offset: instruction i of the wave adds
  // (wave*NI + i)*1024 (scalar) and flips the chunk bits that the swizzle
  // takes from the row's instruction index (one XOR). For d = 128 a
  // 1 KiB instruction covers rows 4*(wave*NI+i) + lane/16, swz = 4*(lane/16) + i;
  // for d = 64 rows 8*(wave*NI+i) + lane/8, swz = 4*i + lane/16.
  const int lane_base = (D == 128)
      ? ((lane >> 4) * 256) | (16 * ((lane & 15) ^ (4 * (lane >> 4))))
      : ((lane >> 3) * 128) | (16 * ((lane & 7) ^ (lane >> 4)));
  constexpr int kXorStep = (D == 128) ? 16 : 64;
  auto issue = [&](__amdgpu_buffer_rsrc_t rs, int k0, char* dst) {
    int lb = lane_base;
    asm volatile("" : "+v"(lb));  // recompute the offsets here instead of keeping them live
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (ATTN_LDS void*)(dst + (wave * NI + i) * 1024),
                                               16, lb ^ (kXorStep * i),
                                               k0 * D * 2 + (wave * NI + i) * 1024, 0, 0);
  };

  // Sᵀ[key][row] of one tile: two 32-key halves, K (A operand) from LDS
  auto scores = [&](const char* kl, f32x16_t (&s)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16_t{};
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
            kl + lds_off<D>(kb * 32 + l32, 16 * dc + 8 * g));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[dc], s[kb], 0, 0, 0);
      }
    }
  };
  // only tiles past the first row's diagonal or the ragged end hide keys
  auto needs_mask = [&](int k0) { return k0 + kBN > mask_from || k0 + kBN > p.Nk; };
  // hide the keys a row cannot see
  auto mask = [&](int k0, f32x16_t (&s)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
        if (key > lim) s[kb][i] = neg_inf();
      }
  };

  f32x16_t acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16_t{};
  float m_run = neg_inf();  // reference max (base 2) of this lane's row
  float l_run = 0.f;        // this lane's share of the row sum of P

  // transposing-read address pattern inside a 16-lane group
  const int grp = lane >> 4;
  const int src = lane & 15;
  const int tr_row = src >> 2;
  const int tr_col = 4 * (src & 3) + 16 * (grp & 1);

  // max over a tile's scores of this lane's row (raw scores): four chains of
  // v_maximum3, then across the halves, scaled to base 2. (NaN-propagating
  // max: no canonicalisation needed.)
  auto tile_max = [&](const f32x16_t (&s)[2]) __attribute__((always_inline)) {
    float mq[4] = {s[0][0], s[0][1], s[0][2], s[0][3]};
#pragma unroll
    for (int i = 4; i < 32; i += 4)
#pragma unroll
      for (int j = 0; j < 4; ++j) mq[j] = __builtin_elementwise_maximum(mq[j], s[i >> 4][(i & 15) + j]);
    float mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mq[0], mq[1]),
                                             __builtin_elementwise_maximum(mq[2], mq[3]));
    return max_across_halves(mx) * p.c;
  };

  // One pipeline step for tile `it`, whose unmasked scores are in `sc` and
  // their row max (base 2) in `mt`. K of tile it+1 is in `kn`, V of tile it in `vc`.
  // Loads in flight during the step: K of tile it+2 into `kfree` and V of
  // tile it+1 into `vfree`. The step has two MFMA phases, each paired with
  // VALU work that does not depend on it:
  //   1. Sᵀ of tile it+1 (into `sn`)  ||  P = exp2(s*c - m) and row sum of tile it
  //   2. Oᵀ += Vᵀ Pᵀ of tile it       ||  max of tile it+1 (unmasked)
  // A tile that hides keys is masked, and its max recomputed, at the start of
  // its own step, so no branch separates the two phases. On the last tile
  // (LAST) there is no next tile: phase 1 has no MFMAs.
  auto step = [&](auto last_tag, int it, f32x16_t (&sc)[2], f32x16_t (&sn)[2], float& mt,
                  const char* kn, const char* vc, char* kfree, char* vfree)
      __attribute__((always_inline)) {
    constexpr bool LAST = decltype(last_tag)::value;
    const int k0 = it * kBN;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): K(it+1) and V(it) have landed
    __syncthreads();                     // ... for every wave; the free buffers are free
    if (!LAST) {
      if (it + 2 < ntiles) issue(krs, k0 + 2 * kBN, kfree);
      issue(vrs, k0 + kBN, vfree);
    }
    if (needs_mask(k0)) {
      mask(k0, sc);
      mt = tile_max(sc);
    }

    // online softmax with a lazily moved reference: exp2(s*c - m) stays below
    // 2^kTau, so the reference only moves (and O, l are rescaled) when the
    // row max jumps by more than kTau. The result is the same softmax.
    const bool need = mt > m_run + kTau;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float m_new = need ? mt : m_run;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;  // 0 from -inf
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
    }
    const float m_use = (m_run == neg_inf()) ? 0.f : m_run;

    // ---- phase 1 ----
    if (!LAST) scores(kn, sn);
    // P = exp2(s*c - m) in fp32 for the row sum (the LSE needs the unrounded
    // values), P̃ = bf16(P) packed two per dword in Sᵀ register order for PV
    uint32_t pk[2][8];
    float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][2 * j], p.c, -m_use));
        const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][2 * j + 1], p.c, -m_use));
        ls[(2 * j) & 3] += e0;
        ls[(2 * j + 1) & 3] += e1;
        pk[kb][j] = pack_bf16x2(e0, e1);
      }
    l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
#if ATTN_PREFILL_SCHED
    if (!LAST) {
#pragma unroll
      for (int i = 0; i < 4; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < 12) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x400, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      }
    }
#endif

    // ---- phase 2: Oᵀ += Vᵀ Pᵀ, 16 keys per MFMA; Vᵀ via transposing LDS reads ----
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const u32x4_t pw4 = {pk[kb][4 * hf], pk[kb][4 * hf + 1], pk[kb][4 * hf + 2],
                             pk[kb][4 * hf + 3]};
        const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pw4);
        const int r0 = kb * 32 + 16 * hf + 4 * g + tr_row;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int col = 32 * db + tr_col;
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (ATTN_LDS i16x4_t*)(vc + lds_off<D>(r0, col)));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (ATTN_LDS i16x4_t*)(vc + lds_off<D>(r0 + 8, col)));
          const u32x2_t lo2 = __builtin_bit_cast(u32x2_t, lo);
          const u32x2_t hi2 = __builtin_bit_cast(u32x2_t, hi);
          const u32x4_t a4 = {lo2[0], lo2[1], hi2[0], hi2[1]};
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a4), pb,
                                                            acc[db], 0, 0, 0);
        }
      }
    if (!LAST) mt = tile_max(sn);
#if ATTN_PREFILL_SCHED
#pragma unroll
    for (int i = 0; i < 4; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      if (i < 14) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 1);
    }
#endif
  };

  if (ntiles > 0) {
    issue(krs, 0, kb0);
    issue(vrs, 0, vb0);
    if (ntiles > 1) issue(krs, kBN, kb1);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    f32x16_t sa[2], sb[2];
    scores(kb0, sa);
    float mt = tile_max(sa);
    // K(1) may still be in flight for other waves: the first step's barrier
    // orders it; its V(0) wait is already satisfied.
    using more_t = std::integral_constant<bool, false>;
    using last_t = std::integral_constant<bool, true>;
    int it = 0;
    for (; it + 2 < ntiles; it += 2) {
      step(more_t{}, it, sa, sb, mt, kb1, vb0, kb0, vb1);
      step(more_t{}, it + 1, sb, sa, mt, kb0, vb1, kb1, vb0);
    }
    if (it + 1 < ntiles) {
      step(more_t{}, it, sa, sb, mt, kb1, vb0, kb0, vb1);
      step(last_t{}, it + 1, sb, sa, mt, kb0, vb1, kb1, vb0);
    } else {
      step(last_t{}, it, sa, sb, mt, kb1, vb0, kb0, vb1);
    }
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
