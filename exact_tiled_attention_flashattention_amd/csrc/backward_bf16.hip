// Backward pass of causal / non-causal GQA prefill attention, bf16 inputs,
// fp32 accumulation, gfx950 MFMA.
//
// Method ("Phase 07 · 12: KV cache, Flash Attention and inference
// optimisation", section "tiling trick": the backward pass recomputes the
// forward's intermediate values instead of storing them). With the forward's
// per-row log-sum-exp L, a tile's probabilities are recomputed exactly as
// P = exp(scale·q·k − L) without any running max, and the chain rule through
// O = P V, the row softmax and S = scale·Q Kᵀ gives, per tile,
//     dV += Pᵀ dO,  dP = dO Vᵀ,  dS = P ∘ (dP − D),  dQ += scale·dS K,
//     dK += scale·dSᵀ Q,        with D_i = dO_i · O_i (one number per row).
// Neither S, P nor dS ever reaches device memory.
//
// Two kernels, so that no output needs atomics:
//   * bwd_dq_kernel: one workgroup per (query block, K/V head, head group),
//     the forward's decomposition. A wave owns 32 query rows and streams the
//     K/V tiles through LDS; it computes Sᵀ = K·Qᵀ and dPᵀ = V·dOᵀ with Qᵀ,
//     dOᵀ in registers (one query row per lane), so L and D are per-lane
//     constants, and dQᵀ += Kᵀ·dSᵀ with Kᵀ read through the transposing LDS
//     read. It also writes D to the workspace.
//   * bwd_dkdv_kernel: one workgroup per (128-key block, K/V head, share of
//     the group's query heads), 8 waves: each 32-key slice has a dV wave and
//     a dK wave, the dK wave one tile step behind. The dV wave holds the
//     slice's K rows, computes S = Q·Kᵀ (one key per lane), P, and
//     dVᵀ += dOᵀ·P, and leaves P in LDS; the dK wave holds the V rows,
//     computes dP = dO·Vᵀ, dS = P ∘ (dP − D) from that P, and dKᵀ += Qᵀ·dS.
//     dOᵀ and Qᵀ come from the transposing LDS read. The sum over the query
//     heads happens in the accumulators. When the group is shared by several
//     workgroups (so that, under a causal mask, no workgroup holds far more
//     than its share of the work), each writes fp32 partial sums and
//     bwd_reduce_kernel adds them in a fixed order: the result does not
//     depend on timing.
// Tiles are 64 rows of D bf16, loaded straight from global memory into an
// XOR-swizzled LDS layout in which both the row reads (MFMA A operand) and
// the transposing reads are conflict-free, double-buffered (triple-buffered
// in the dK/dV kernel) with one barrier per tile.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kTile = 64;                  // rows per streamed tile
constexpr int kBufferFlags = 0x00020000;   // raw buffer resource, 32-bit dword data
// sched_barrier mask: VALU, SALU and transcendental instructions may be
// scheduled across it; LDS reads and MFMAs may not
constexpr int kSchedAluOnly = 0x406;

struct BwdParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* o;
  const __bf16* dout;
  const float* lse;
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  float* drow;  // [B, Hq, Nq] workspace: D_i = dO_i · O_i
  float* lrow;  // [B, Hq, Nq] workspace: the row's base-2 LSE (+inf for a row that saw no key)
  int B, Hq, Hkv, Nq, Nk;
  int G;       // Hq / Hkv
  int hw;      // heads per dQ workgroup (1, 2 or 4)
  int pw;      // 32-row slices per head in a dQ workgroup (4 / hw)
  int n_qblk;  // dQ query blocks of 32 * pw rows
  int n_hgrp;  // dQ workgroups per K/V head and query block (G / hw)
  int n_kblk;  // dK/dV key blocks of 128 keys
  int nsplit;  // dK/dV workgroups per (key block, K/V head): each takes G / nsplit query heads
  float* part;  // nsplit > 1: fp32 partial dK then dV, [nsplit][B][Hkv][Nk][D] each
  float c;     // scale * log2(e)
  float scale;
  int q_offset;
  int causal;
};

// Tiles (64 rows of D bf16) live in LDS as D/32 column blocks: the 64 rows
// of elements [32c, 32c + 32) form a 4 KiB block, 64 bytes per row, and the
// four 16-byte chunks q of row r sit at slot q ^ ((r >> 2) & 3). Both read
// patterns are conflict-free: 16 consecutive rows at one chunk (the MFMA A
// operand read row-wise) cover every 16-byte slot of 256 bytes once, and the
// transposing reads (4 consecutive rows x 64 bytes per 32 lanes) 256
// contiguous bytes. Every read of a wave then differs from one of four
// per-lane offsets by a constant (see RowOff / TrOff).
constexpr int kBlk = kTile * 64;  // bytes of one column block

// direct-to-LDS loads of one tile: load j of the tile (1 KiB, LDS bytes
// [1024j, +1024)) carries rows 16*(j%4) + lane/4 of column block j/4, the
// lane's slot lane%4 holding logical chunk (lane%4) ^ (lane/16)
template <int D>
__device__ __forceinline__ int tile_lane_offset(int lane) {
  return (lane >> 2) * (D * 2) + ((((lane & 3) ^ (lane >> 4))) << 4);
}

// Loads of one 64-row tile (rows of 2*D bytes, contiguous from `tile`, of
// which `bytes` are valid) into LDS `dst`: each of the 4 waves issues NI of
// the tile's loads. The resource starts at the tile and ends after its valid
// bytes, and every offset is a per-lane (range-checked) one, so rows past the
// end arrive as zeros.
template <int D>
__device__ __forceinline__ void load_tile(const void* tile, long long bytes, char* dst, int wave,
                                          int lane) {
  constexpr int NI = kTile * D * 2 / (kWaves * 1024);
  const int range = (int)(bytes < 0 ? 0 : (bytes > kTile * D * 2 ? kTile * D * 2 : bytes));
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(tile), 0, range, kBufferFlags);
  int lb = tile_lane_offset<D>(lane);
  asm volatile("" : "+v"(lb));
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int j = wave * NI + i;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (ATTN_LDS void*)(dst + j * 1024), 16,
                                             lb + 16 * (j & 3) * (D * 2) + 64 * (j >> 2), 0, 0,
                                             0);
  }
}

// Per-lane offsets of the row-wise A-operand reads: lane l reads row
// base + l%32, elements 16*dc + 8*(l/32) .. +8, at
//   tile + off[dc % 2] + (dc / 2) * kBlk + base * 64      (base % 32 == 0)
struct RowOff {
  int off[2];
};
__device__ __forceinline__ RowOff row_offsets(int lane) {
  const int l32 = lane & 31, g = lane >> 5;
  RowOff r;
#pragma unroll
  for (int h = 0; h < 2; ++h) r.off[h] = l32 * 64 + ((((2 * h + g) ^ ((l32 >> 2) & 3))) << 4);
  return r;
}
template <int D>
__device__ __forceinline__ bf16x8_t read_row(const char* tile, const RowOff& ro, int base,
                                             int dc) {
  return *reinterpret_cast<const bf16x8_t*>(tile + ro.off[dc & 1] + (dc >> 1) * kBlk + base * 64);
}

// Per-lane offsets of the transposing reads: a 32(d) x 16(row) A operand
// from rows base + 16*hf + [4*(l/32) + (l%16)/4, +8] and columns
// 32*db + [4*(l%4) + 16*((l/16)%2)] is
//   tile + off[h] + db * kBlk + (base + 16*hf + 8*h) * 64   for the halves h = 0, 1
struct TrOff {
  int off[2];
};
__device__ __forceinline__ TrOff tr_offsets(int lane) {
  const int g = lane >> 5, grp = lane >> 4, src = lane & 15;
  const int tr_row = src >> 2;
  const int tr_col = 4 * (src & 3) + 16 * (grp & 1);
  TrOff t;
#pragma unroll
  for (int h = 0; h < 2; ++h)
    t.off[h] = (4 * g + tr_row) * 64 + (((((tr_col >> 3) & 3) ^ g ^ (2 * h))) << 4) +
               ((tr_col & 7) << 1);
  return t;
}
__device__ __forceinline__ bf16x8_t read_tr(const char* tile, const TrOff& to, int base, int hf,
                                            int db) {
  const char* p0 = tile + db * kBlk + (base + 16 * hf) * 64;
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4_t*)(p0 + to.off[0]));
  const i16x4_t hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4_t*)(p0 + 8 * 64 + to.off[1]));
  const u32x2_t lo2 = __builtin_bit_cast(u32x2_t, lo);
  const u32x2_t hi2 = __builtin_bit_cast(u32x2_t, hi);
  const u32x4_t a4 = {lo2[0], lo2[1], hi2[0], hi2[1]};
  return __builtin_bit_cast(bf16x8_t, a4);
}

// base-2 log-sum-exp of a row from the forward's natural-log LSE; a row that
// saw no key (LSE = -inf) gets +inf, so every recomputed P of it is 0
__device__ __forceinline__ float lse2_of(float lse) {
  return lse == neg_inf() ? __builtin_inff() : lse * kLog2e;
}

// ============================================================================
// dQ (and D)
// ============================================================================
template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(BwdParams p) {
  constexpr int NDC = D / 16;
  constexpr int NDB = D / 32;
  constexpr int TILE = kTile * D * 2;
  __shared__ __attribute__((aligned(1024))) char kb0[TILE];
  __shared__ __attribute__((aligned(1024))) char kb1[TILE];
  __shared__ __attribute__((aligned(1024))) char vb0[TILE];
  __shared__ __attribute__((aligned(1024))) char vb1[TILE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const int per_q = p.B * p.Hkv * p.n_hgrp;
  const int qrank = blockIdx.x / per_q;
  int rest = blockIdx.x - qrank * per_q;
  const int hg = rest % p.n_hgrp;
  rest /= p.n_hgrp;
  const int kvh = rest % p.Hkv;
  const int b = rest / p.Hkv;
  const int qblk = CAUSAL ? (p.n_qblk - 1 - qrank) : qrank;
  const int head_local = wave % p.hw;
  const int sub = wave / p.hw;
  const int hq = kvh * p.G + hg * p.hw + head_local;
  const int q0 = qblk * 32 * p.pw;
  const int my_q = q0 + sub * 32 + l32;
  const bool row_ok = my_q < p.Nq;

  int kend = p.Nk;
  if (CAUSAL) {
    const long long lim = (long long)min(q0 + 32 * p.pw, p.Nq) - 1 + p.q_offset + 1;
    if (lim < kend) kend = (int)(lim < 0 ? 0 : lim);
  }
  const int ntiles = (kend + kTile - 1) / kTile;
  long long mask_from = p.Nk;
  if (CAUSAL) {
    const long long first = (long long)q0 + p.q_offset + 1;
    if (first < mask_from) mask_from = first;
  }
  long long lim64 = CAUSAL ? (long long)my_q + p.q_offset : (long long)p.Nk - 1;
  if (lim64 > (long long)p.Nk - 1) lim64 = (long long)p.Nk - 1;
  if (lim64 < -1) lim64 = -1;
  const int lim = (int)lim64;

  // Qᵀ and dOᵀ as B operands: lane holds row my_q, d = 16*dc + 8*g + j; and
  // D = dO·O of the row (the lane's half of d, then across the halves)
  const long long row_off = (((long long)b * p.Hq + hq) * p.Nq + my_q) * D + 8 * g;
  bf16x8_t qf[NDC], df[NDC];
  float dsum = 0.f;
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc) {
    if (row_ok) {
      qf[dc] = *reinterpret_cast<const bf16x8_t*>(p.q + row_off + 16 * dc);
      df[dc] = *reinterpret_cast<const bf16x8_t*>(p.dout + row_off + 16 * dc);
      const bf16x8_t of = *reinterpret_cast<const bf16x8_t*>(p.o + row_off + 16 * dc);
#pragma unroll
      for (int j = 0; j < 8; ++j) dsum += (float)df[dc][j] * (float)of[j];
    } else {
      qf[dc] = bf16x8_t{};
      df[dc] = bf16x8_t{};
    }
  }
  const float drow = sum_across_halves(dsum);
  const long long ridx = ((long long)b * p.Hq + hq) * p.Nq + my_q;
  const float lse2 = row_ok ? lse2_of(p.lse[ridx]) : __builtin_inff();
  if (row_ok && g == 0) {
    p.drow[ridx] = drow;
    p.lrow[ridx] = lse2;
  }

  const long long kv_base = ((long long)b * p.Hkv + kvh) * (long long)p.Nk * D;
  const long long kv_bytes = (long long)p.Nk * D * 2;

  f32x16_t acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16_t{};

  const RowOff ro = row_offsets(lane);
  const TrOff to = tr_offsets(lane);

  // One 64-key tile: Sᵀ = K·Qᵀ and dPᵀ = V·dOᵀ, dSᵀ = Pᵀ ∘ (dPᵀ − D), then
  // dQᵀ += Kᵀ·dSᵀ. Only tiles that cross a row's last visible key (the causal
  // diagonal, the ragged end) are MASKED.
  auto tile_step = [&](auto masked_tag, int it, const char* kl, const char* vl)
      __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int k0 = it * kTile;
    // per 32-key half: Sᵀ, dPᵀ, then dSᵀ = Pᵀ ∘ (dPᵀ − D) packed to bf16 in
    // Sᵀ register order
    uint32_t pk[2][8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16_t s = f32x16_t{}, dp = f32x16_t{};
      bf16x8_t ka[NDC];
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) ka[dc] = read_row<D>(kl, ro, kb * 32, dc);
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[dc], qf[dc], s, 0, 0, 0);
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) ka[dc] = read_row<D>(vl, ro, kb * 32, dc);
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc)
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[dc], df[dc], dp, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float e[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int i = 2 * j + h;
          float x = s[i];
          if (MASKED) {
            const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
            if (key > lim) x = neg_inf();
          }
          const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(x, p.c, -lse2));
          e[h] = pr * (dp[i] - drow);
        }
        pk[kb][j] = pack_bf16x2(e[0], e[1]);
      }
    }
    // dQᵀ += Kᵀ dSᵀ, 16 keys per MFMA; Kᵀ through the transposing LDS read
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const u32x4_t w4 = {pk[kb][4 * hf], pk[kb][4 * hf + 1], pk[kb][4 * hf + 2],
                            pk[kb][4 * hf + 3]};
        const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, w4);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr(kl, to, kb * 32, hf, db), bop,
                                                            acc[db], 0, 0, 0);
      }
  };

  // tiles before m0 hide no key from any row of the workgroup
  const long long mlim = mask_from < (long long)p.Nk ? mask_from : (long long)p.Nk;
  const int m0 = (int)(mlim / kTile);
  // tile it (buffers it % 2, a compile-time choice): wait for it, free it-1's
  // buffers, load it+1 into them, compute it
  auto step = [&](auto buf_tag, int it) __attribute__((always_inline)) {
    constexpr int BUF = decltype(buf_tag)::value;
    char* kc = BUF ? kb1 : kb0;
    char* vc = BUF ? vb1 : vb0;
    char* kn = BUF ? kb0 : kb1;
    char* vn = BUF ? vb0 : vb1;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile it has landed
    __syncthreads();                     // ... for every wave; tile it-1's buffers are free
    if (it + 1 < ntiles) {
      const long long t0 = (long long)(it + 1) * kTile * D;
      load_tile<D>(p.k + kv_base + t0, kv_bytes - 2 * t0, kn, wave, lane);
      load_tile<D>(p.v + kv_base + t0, kv_bytes - 2 * t0, vn, wave, lane);
    }
    if (it < m0)
      tile_step(std::integral_constant<bool, false>{}, it, kc, vc);
    else
      tile_step(std::integral_constant<bool, true>{}, it, kc, vc);
  };

  if (ntiles > 0) {
    load_tile<D>(p.k + kv_base, kv_bytes, kb0, wave, lane);
    load_tile<D>(p.v + kv_base, kv_bytes, vb0, wave, lane);
    for (int it = 0; it < ntiles; it += 2) {
      step(std::integral_constant<int, 0>{}, it);
      if (it + 1 < ntiles) step(std::integral_constant<int, 1>{}, it + 1);
    }
  }

  // dQ rows pass through the wave's own 32 rows of the (then free) tile
  // buffers, so that each store writes whole rows, 16 bytes per lane, instead
  // of 8-byte pieces of 32 rows
  constexpr int RB = D * 2;    // bytes per row
  constexpr int NCH = D / 8;   // 16-byte chunks per row; chunk c of row r sits at c ^ (r % NCH)
  static_assert(2 * 32 * RB == TILE, "two waves' rows fill one tile buffer");
  char* stage = ((wave >> 1) == 0 ? kb0 : vb0) + (wave & 1) * 32 * RB;
  __syncthreads();
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      f32x4_t v4 = {acc[db][4 * ii] * p.scale, acc[db][4 * ii + 1] * p.scale,
                    acc[db][4 * ii + 2] * p.scale, acc[db][4 * ii + 3] * p.scale};
      const int c = 4 * db + ii;
      *reinterpret_cast<bf16x4_t*>(stage + l32 * RB + ((c ^ (l32 & (NCH - 1))) << 4) + 8 * g) =
          __builtin_convertvector(v4, bf16x4_t);
    }
  __syncthreads();
  const int row0 = q0 + sub * 32;
  __bf16* const dq_head = p.dq + ((long long)b * p.Hq + hq) * p.Nq * D;
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    const int r = i * (64 / NCH) + lane / NCH;
    const int c = lane % NCH;
    const u32x4_t val =
        *reinterpret_cast<const u32x4_t*>(stage + r * RB + ((c ^ (r & (NCH - 1))) << 4));
    if (row0 + r < p.Nq)
      *reinterpret_cast<u32x4_t*>(dq_head + (long long)(row0 + r) * D + 8 * c) = val;
  }
}

// ============================================================================
// dK, dV with each 32-key slice shared by two waves and the two halves of
// the work one tile step apart. The dV wave computes S = Q·Kᵀ, P (masked,
// packed to bf16) and dVᵀ += dOᵀ·P, and leaves P in LDS; one step later the
// dK wave computes dP = dO·Vᵀ, dS = P ∘ (dP − D) from that P, and
// dKᵀ += Qᵀ·dS. Each wave holds one accumulator set and one of K, V, so two
// waves fit a SIMD; no product is computed twice. Tiles are triple-buffered
// (the dK wave reads step s−1 while the dV wave reads step s and step s+1 is
// loading); the one barrier per step orders every hand-over.
// ============================================================================
template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_kernel(BwdParams p) {
  constexpr int NDC = D / 16;
  constexpr int NDB = D / 32;
  constexpr int TILE = kTile * D * 2;
  __shared__ __attribute__((aligned(1024))) char qbuf[3][TILE];
  __shared__ __attribute__((aligned(1024))) char obuf[3][TILE];  // dO tiles
  __shared__ __attribute__((aligned(16))) float lbuf[3][2 * kTile];  // base-2 LSE, then D
  // P of a step, bf16 pairs in S register order, the two 16-byte halves of a
  // lane's 32 bytes in separate planes (lane-contiguous, conflict-free):
  // [buffer][slice][query half qb][plane][lane]
  __shared__ __attribute__((aligned(16))) u32x4_t pbuf[3][kWaves][2][2][64];

  const int tid = threadIdx.x;
  const int wave8 = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int role = wave8 >> 2;  // 0: dV (and P), 1: dK
  const int wave = wave8 & 3;   // key slice
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const int per_k = p.B * p.Hkv * p.nsplit;
  const int kblk = blockIdx.x / per_k;
  int rest = blockIdx.x - kblk * per_k;
  const int split = rest % p.nsplit;
  rest /= p.nsplit;
  const int kvh = rest % p.Hkv;
  const int b = rest / p.Hkv;
  const int gs = p.G / p.nsplit;
  const int k0 = kblk * (kWaves * 32);
  const int kw0 = k0 + wave * 32;
  const int my_key = kw0 + l32;

  // K rows (dV role) or V rows (dK role) of the slice as B operands
  const long long kv_base = ((long long)b * p.Hkv + kvh) * (long long)p.Nk * D;
  const __bf16* kvsrc = role == 0 ? p.k : p.v;
  bf16x8_t kv[NDC];
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc)
    kv[dc] = my_key < p.Nk ? *reinterpret_cast<const bf16x8_t*>(
                                 kvsrc + kv_base + (long long)my_key * D + 16 * dc + 8 * g)
                           : bf16x8_t{};

  int qt_lo = 0;
  if (CAUSAL) {
    const long long first_row = (long long)k0 - p.q_offset;
    qt_lo = first_row <= 0 ? 0 : (int)min(first_row / kTile, (long long)0x3fffffff);
  }
  const int n_qt = (p.Nq + kTile - 1) / kTile;
  const int per_head = n_qt > qt_lo ? n_qt - qt_lo : 0;
  const int nsteps = per_head * gs;

  f32x16_t acc[NDB];  // dVᵀ (role 0) or dKᵀ (role 1)
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16_t{};

  const int kq = my_key - p.q_offset;
  const RowOff ro = row_offsets(lane);
  const TrOff to = tr_offsets(lane);

  // step s's tiles into buffer s % 3, issued by the dV waves
  auto issue = [&](int s, int bi) __attribute__((always_inline)) {
    const int hq = kvh * p.G + split * gs + s / per_head;
    const int qt = qt_lo + s % per_head;
    const long long hbase = ((long long)b * p.Hq + hq) * (long long)p.Nq;
    const long long r0 = (long long)qt * kTile;
    const long long left = (long long)p.Nq - r0;
    load_tile<D>(p.q + (hbase + r0) * D, left * D * 2, qbuf[bi], wave, lane);
    load_tile<D>(p.dout + (hbase + r0) * D, left * D * 2, obuf[bi], wave, lane);
    if (wave < 2) {
      const float* srcp = (wave == 0 ? p.lrow : p.drow) + hbase + r0;
      const __amdgpu_buffer_rsrc_t lrs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(srcp), 0, (int)(left >= kTile ? kTile * 4 : left * 4), kBufferFlags);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(lrs, (ATTN_LDS void*)(lbuf[bi] + wave * kTile), 4,
                                               4 * lane, 0, 0, 0);
    }
  };

  // dV role, step s (buffers BI = s % 3): S, P (left in LDS for the dK wave),
  // dVᵀ += dOᵀ P; only steps whose query rows reach below the slice's last
  // key under a causal mask are MASKED
  auto step_v = [&](bool masked, auto buf_tag, int s) __attribute__((always_inline)) {
    constexpr int BI = decltype(buf_tag)::value;
    const char* ql = qbuf[BI];
    const char* ol = obuf[BI];
    const float* ll = lbuf[BI];
    const int qrow0 = (qt_lo + s % per_head) * kTile;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16_t sc = f32x16_t{};
      // every LDS read of the S chain and the softmax is issued before the MFMAs
      bf16x8_t qa[NDC];
      f32x4_t l4[4];
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) qa[dc] = read_row<D>(ql, ro, qb * 32, dc);
#pragma unroll
      for (int m = 0; m < 4; ++m)
        l4[m] = *reinterpret_cast<const f32x4_t*>(ll + qb * 32 + 8 * m + 4 * g);
      // the chain's reads all issue before its first MFMA (VALU/SALU may cross)
      __builtin_amdgcn_sched_barrier(kSchedAluOnly);
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc)
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[dc], kv[dc], sc, 0, 0, 0);
      // a uniform branch around the masking alone keeps one copy of the step
      if (masked) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kq > qrow0 + qb * 32 + 8 * (i >> 2) + 4 * g + (i & 3)) sc[i] = neg_inf();
      }
      uint32_t pk[8];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        float pv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = sc[4 * m + r];
          pv[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(x, p.c, -l4[m][r]));
        }
        pk[2 * m] = pack_bf16x2(pv[0], pv[1]);
        pk[2 * m + 1] = pack_bf16x2(pv[2], pv[3]);
      }
      pbuf[BI][wave][qb][0][lane] = u32x4_t{pk[0], pk[1], pk[2], pk[3]};
      pbuf[BI][wave][qb][1][lane] = u32x4_t{pk[4], pk[5], pk[6], pk[7]};
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const u32x4_t w4 = {pk[4 * hf], pk[4 * hf + 1], pk[4 * hf + 2], pk[4 * hf + 3]};
        const bf16x8_t bo = __builtin_bit_cast(bf16x8_t, w4);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr(ol, to, qb * 32, hf, db), bo,
                                                            acc[db], 0, 0, 0);
      }
    }
  };

  // dK role, step s (one step behind; buffers BI = s % 3): dP, dS = P ∘ (dP − D),
  // dKᵀ += Qᵀ dS
  auto step_k = [&](auto buf_tag) __attribute__((always_inline)) {
    constexpr int BI = decltype(buf_tag)::value;
    const char* ql = qbuf[BI];
    const char* ol = obuf[BI];
    const float* ll = lbuf[BI];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16_t dp = f32x16_t{};
      // every LDS read of the dP chain and of dS's other factors first
      bf16x8_t oa[NDC];
      f32x4_t d4[4];
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) oa[dc] = read_row<D>(ol, ro, qb * 32, dc);
      const u32x4_t p0 = pbuf[BI][wave][qb][0][lane];
      const u32x4_t p1 = pbuf[BI][wave][qb][1][lane];
#pragma unroll
      for (int m = 0; m < 4; ++m)
        d4[m] = *reinterpret_cast<const f32x4_t*>(ll + kTile + qb * 32 + 8 * m + 4 * g);
      // the chain's reads all issue before its first MFMA (VALU/SALU may cross)
      __builtin_amdgcn_sched_barrier(kSchedAluOnly);
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc)
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[dc], kv[dc], dp, 0, 0, 0);
      const uint32_t pp[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
      uint32_t pd[8];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float e0 = bf16_lo(pp[2 * m]) * (dp[4 * m] - d4[m][0]);
        const float e1 = bf16_hi(pp[2 * m]) * (dp[4 * m + 1] - d4[m][1]);
        const float e2 = bf16_lo(pp[2 * m + 1]) * (dp[4 * m + 2] - d4[m][2]);
        const float e3 = bf16_hi(pp[2 * m + 1]) * (dp[4 * m + 3] - d4[m][3]);
        pd[2 * m] = pack_bf16x2(e0, e1);
        pd[2 * m + 1] = pack_bf16x2(e2, e3);
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const u32x4_t w4 = {pd[4 * hf], pd[4 * hf + 1], pd[4 * hf + 2], pd[4 * hf + 3]};
        const bf16x8_t bo = __builtin_bit_cast(bf16x8_t, w4);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr(ql, to, qb * 32, hf, db), bo,
                                                            acc[db], 0, 0, 0);
      }
    }
  };

  // Barrier n: step n's tiles have landed and every wave is past step n-1
  // (n = 0 .. nsteps). After it the dV waves load step n+1 into buffer
  // (n+1) % 3 and compute step n from buffer n % 3; the dK waves compute step
  // n-1. Each role runs its own loop, unrolled by three so that every buffer
  // index is a compile-time constant, with the same barrier count; the
  // remainder of fewer than three steps is peeled.
  auto barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads have landed
    __syncthreads();
  };
  auto v_iter = [&](auto r_tag, int it) __attribute__((always_inline)) {
    constexpr int R = decltype(r_tag)::value;
    barrier();
    if (it + 1 < nsteps) issue(it + 1, (R + 1) % 3);
    const int qrow0 = (qt_lo + it % per_head) * kTile;
    const bool masked = p.causal != 0 && (long long)qrow0 + p.q_offset < (long long)kw0 + 31;
    step_v(masked, r_tag, it);
  };
  auto k_iter = [&](auto r_tag) __attribute__((always_inline)) {
    barrier();
    step_k(r_tag);
  };
  using R0 = std::integral_constant<int, 0>;
  using R1 = std::integral_constant<int, 1>;
  using R2 = std::integral_constant<int, 2>;

  if (nsteps > 0) {
    if (role == 0) {
      issue(0, 0);
      int it = 0;
      for (; it + 3 <= nsteps; it += 3) {
        v_iter(R0{}, it);
        v_iter(R1{}, it + 1);
        v_iter(R2{}, it + 2);
      }
      if (it < nsteps) v_iter(R0{}, it);
      if (it + 1 < nsteps) v_iter(R1{}, it + 1);
      barrier();  // barrier nsteps: the dK waves' last step
    } else {
      barrier();  // barrier 0: nothing to do yet
      int j = 0;
      for (; j + 3 <= nsteps; j += 3) {
        k_iter(R0{});
        k_iter(R1{});
        k_iter(R2{});
      }
      if (j < nsteps) k_iter(R0{});
      if (j + 1 < nsteps) k_iter(R1{});
    }
  }

  // The slice's 32 rows pass through LDS (a region of the then free tile and
  // P buffers per wave) so that each store writes whole rows, 16 bytes per
  // lane, instead of pieces of 32 rows: bf16 rows when the workgroup owns the
  // whole sum, fp32 partial rows otherwise.
  static_assert(sizeof(pbuf) >= 2 * TILE && 32 * D * 4 == TILE, "eight regions of 32 fp32 rows");
  char* const stage = wave8 < 3   ? qbuf[wave8]
                      : wave8 < 6 ? obuf[wave8 - 3]
                                  : reinterpret_cast<char*>(pbuf) + (wave8 - 6) * TILE;
  const float f = role == 0 ? 1.f : p.scale;
  const bool whole = p.nsplit == 1;
  constexpr int RB = D * 2, NCH = D / 8;    // bf16 rows: bytes, 16-byte chunks
  constexpr int RF = D * 4, NCF = D / 4;    // fp32 rows
  __syncthreads();
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      f32x4_t v4 = {acc[db][4 * ii] * f, acc[db][4 * ii + 1] * f, acc[db][4 * ii + 2] * f,
                    acc[db][4 * ii + 3] * f};
      if (whole) {
        const int c = 4 * db + ii;
        *reinterpret_cast<bf16x4_t*>(stage + l32 * RB + ((c ^ (l32 & (NCH - 1))) << 4) + 8 * g) =
            __builtin_convertvector(v4, bf16x4_t);
      } else {
        const int c = 8 * db + 2 * ii + g;
        *reinterpret_cast<f32x4_t*>(stage + l32 * RF + ((c ^ (l32 & (NCF - 1))) << 4)) = v4;
      }
    }
  __syncthreads();
  const long long plane = (long long)p.B * p.Hkv * p.Nk * D;
  if (whole) {
    __bf16* const out = (role == 0 ? p.dv : p.dk) + kv_base;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      const int r = i * (64 / NCH) + lane / NCH;
      const int c = lane % NCH;
      const u32x4_t val =
          *reinterpret_cast<const u32x4_t*>(stage + r * RB + ((c ^ (r & (NCH - 1))) << 4));
      if (kw0 + r < p.Nk)
        *reinterpret_cast<u32x4_t*>(out + (long long)(kw0 + r) * D + 8 * c) = val;
    }
  } else {
    float* const part = p.part + ((role == 0 ? p.nsplit : 0) + split) * plane + kv_base;
#pragma unroll
    for (int i = 0; i < D / 8; ++i) {
      const int r = i * (64 / NCF) + lane / NCF;
      const int c = lane % NCF;
      const f32x4_t val =
          *reinterpret_cast<const f32x4_t*>(stage + r * RF + ((c ^ (r & (NCF - 1))) << 4));
      if (kw0 + r < p.Nk)
        *reinterpret_cast<f32x4_t*>(part + (long long)(kw0 + r) * D + 4 * c) = val;
    }
  }
}

// dK, dV = the sums of the nsplit partial sums, added in split order; one
// thread per 8 elements.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdParams p, long long n8) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const long long plane = n8 * 8;  // elements of dK (and of dV)
  const long long e = i * 8;
  f32x4_t k0 = {0.f, 0.f, 0.f, 0.f}, k1 = k0, v0 = k0, v1 = k0;
  for (int sp = 0; sp < p.nsplit; ++sp) {
    const float* a = p.part + sp * plane + e;
    const float* c = p.part + (p.nsplit + sp) * plane + e;
    k0 += *reinterpret_cast<const f32x4_t*>(a);
    k1 += *reinterpret_cast<const f32x4_t*>(a + 4);
    v0 += *reinterpret_cast<const f32x4_t*>(c);
    v1 += *reinterpret_cast<const f32x4_t*>(c + 4);
  }
  *reinterpret_cast<bf16x4_t*>(p.dk + e) = __builtin_convertvector(k0, bf16x4_t);
  *reinterpret_cast<bf16x4_t*>(p.dk + e + 4) = __builtin_convertvector(k1, bf16x4_t);
  *reinterpret_cast<bf16x4_t*>(p.dv + e) = __builtin_convertvector(v0, bf16x4_t);
  *reinterpret_cast<bf16x4_t*>(p.dv + e + 4) = __builtin_convertvector(v1, bf16x4_t);
}

template <int D>
hipError_t launch_d(const BwdParams& bp, bool causal, int nq_blocks, int nk_blocks,
                    hipStream_t s) {
  const long long n8 = (long long)bp.B * bp.Hkv * bp.Nk * D / 8;
  if (nq_blocks > 0) {
    if (causal)
      hipLaunchKernelGGL((bwd_dq_kernel<D, true>), dim3(nq_blocks), dim3(kWaves * 64), 0, s, bp);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<D, false>), dim3(nq_blocks), dim3(kWaves * 64), 0, s, bp);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (nk_blocks > 0) {
    if (causal)
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, true>), dim3(nk_blocks), dim3(2 * kWaves * 64), 0, s,
                         bp);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, false>), dim3(nk_blocks), dim3(2 * kWaves * 64), 0, s,
                         bp);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || bp.nsplit == 1) return e;
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, bp,
                       n8);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

BackwardPlan plan_backward(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                           int q_offset, int compute_units) {
  BackwardPlan pl;
  const int G = Hq / Hkv;
  const long long n_kblk = (Nk + kWaves * 32 - 1) / (kWaves * 32);
  const long long n_qt = (Nq + kTile - 1) / kTile;
  // query tiles each key block streams per query head, as the kernel counts them
  long long total = 0, longest = 0;
  for (long long kb = 0; kb < n_kblk; ++kb) {
    long long lo = 0;
    if (causal) {
      const long long first_row = kb * kWaves * 32 - q_offset;
      lo = first_row <= 0 ? 0 : first_row / kTile;
    }
    const long long st = n_qt > lo ? n_qt - lo : 0;
    total += st;
    longest = st > longest ? st : longest;
  }
  total *= (long long)G * B * Hkv;
  // one dK/dV workgroup per compute unit at a time: split the group's query
  // heads over the fewest workgroups that keep the longest one within the
  // average load of a compute unit
  const long long slots = compute_units > 0 ? compute_units : 1;
  pl.nsplit = G;
  for (int sp = 1; sp <= G; ++sp) {
    if (G % sp) continue;
    if (longest * (G / sp) * slots <= total) {
      pl.nsplit = sp;
      break;
    }
  }
  // D at 0, the base-2 LSE at lrow_offset, then the partial sums; each part
  // 256-byte aligned and at least 256 bytes
  size_t rows = ((size_t)B * Hq * Nq * sizeof(float) + 255) / 256 * 256;
  if (rows == 0) rows = 256;
  pl.lrow_offset = rows;
  pl.part_offset = 2 * rows;
  const size_t part = pl.nsplit > 1 ? 2ull * pl.nsplit * B * Hkv * (size_t)Nk * d * sizeof(float)
                                    : 0;
  pl.bytes = pl.part_offset + part;
  return pl;
}

hipError_t launch_backward_bf16(const BackwardArgs& a, hipStream_t s) {
  BwdParams bp;
  bp.q = static_cast<const __bf16*>(a.q);
  bp.k = static_cast<const __bf16*>(a.k);
  bp.v = static_cast<const __bf16*>(a.v);
  bp.o = static_cast<const __bf16*>(a.o);
  bp.dout = static_cast<const __bf16*>(a.dout);
  bp.lse = a.lse;
  bp.dq = static_cast<__bf16*>(a.dq);
  bp.dk = static_cast<__bf16*>(a.dk);
  bp.dv = static_cast<__bf16*>(a.dv);
  bp.drow = a.drow;
  bp.lrow = a.lrow;
  bp.B = a.B;
  bp.Hq = a.Hq;
  bp.Hkv = a.Hkv;
  bp.Nq = a.Nq;
  bp.Nk = a.Nk;
  bp.G = a.Hq / a.Hkv;
  bp.hw = (bp.G % 4 == 0) ? 4 : ((bp.G % 2 == 0) ? 2 : 1);
  bp.pw = kWaves / bp.hw;
  bp.n_qblk = (a.Nq + 32 * bp.pw - 1) / (32 * bp.pw);
  bp.n_hgrp = bp.G / bp.hw;
  bp.n_kblk = (a.Nk + kWaves * 32 - 1) / (kWaves * 32);
  bp.nsplit = a.nsplit;
  bp.part = a.part;
  bp.c = a.scale * kLog2e;
  bp.scale = a.scale;
  bp.q_offset = a.q_offset;
  bp.causal = a.causal != 0;
  const long long nq = (long long)bp.n_qblk * a.B * a.Hkv * bp.n_hgrp;
  const long long nk = (long long)bp.n_kblk * a.B * a.Hkv * bp.nsplit;
  if (nq > 0x7fffffffLL || nk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.d == 128) return launch_d<128>(bp, a.causal != 0, (int)nq, (int)nk, s);
  return launch_d<64>(bp, a.causal != 0, (int)nq, (int)nk, s);
}

}  // namespace attn
