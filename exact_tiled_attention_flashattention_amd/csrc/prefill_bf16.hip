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
//   * A workgroup is 8 waves (4 for launches with fewer than two 8-wave
//     workgroups per CU). The waves share one K/V head: with a group of
//     G = Hq/Hkv query heads ("Effizienz", "GQA im leicht lesbaren Code")
//     they take 4 heads of the group at 64 (32) positions (G % 4 == 0), else
//     fewer heads at more positions. Every K/V tile is read from HBM/L2 once
//     per workgroup and used by all its waves. An 8-wave workgroup fills a CU
//     (two waves per SIMD), and the two waves sharing a SIMD step through the
//     same tiles between the same barriers, so they progress at the same rate.
//   * Each wave owns 32 query rows. Scores are computed transposed,
//     Sᵀ = K·Qᵀ, with v_mfma_f32_32x32x16_bf16 (K from LDS as the A
//     operand, Qᵀ held in registers as the B operand), so each lane holds
//     one query row (lane % 32) and 32 of the tile's 64 keys. The row max
//     and row sum need one cross-half exchange (permlane32 swap).
//   * The probabilities in the Sᵀ accumulator layout are already the B
//     operand (Pᵀ) of Oᵀ = Vᵀ·Pᵀ after a bf16 pack; Vᵀ comes straight out of
//     the V tile in LDS (stored as 64-byte column blocks) through the
//     transposing read ds_read_tr16_b64. Oᵀ stays in 64 fp32 accumulators
//     per lane.
//   * K/V tiles (64 keys) arrive by direct global-to-LDS loads into two
//     buffers each: K runs two tiles ahead of the PV product, V one, so the
//     loads are in flight while the current tile is computed. A cached K/V
//     tile is four 16-token blocks found through the block table.
//   * Softmax runs in base 2 with scale·log2(e) folded into one FMA.
//   * Causal workgroups are launched longest-first (highest query block
//     first) and skip every tile past their last row's diagonal; only tiles
//     that cross the diagonal or the ragged end of K are masked.
#include <type_traits>

#include "common.h"
#include "launch.h"


namespace attn {
namespace {

constexpr int kBN = 64;         // keys per tile
constexpr float kTau = 8.0f;    // rescale only when a row max grows by more than 2^8
constexpr int kBufferFlags = 0x00020000;  // raw buffer resource, 32-bit dword data
// sched_barrier mask: VALU, SALU and transcendental instructions may be
// scheduled across it; LDS reads and MFMAs may not
constexpr int kSchedAluOnly = 0x406;

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
  long long sqb, sqh, sqr;  // element strides of q and o: batch, head, row
  // token-major K/V cache (CACHE kernels): k, v are [num_blocks, 16, Hkv, D]
  // pools behind `table`, or [B, max_len, Hkv, D] when `table` is null;
  // sequence b has clamp(seq_lens[b]) keys and its query row i sits at
  // position seq_lens[b] - Nq + i
  const int32_t* table;
  int max_blocks, num_blocks, max_len;
  const int32_t* seq_lens;
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

// V tiles live in LDS in column blocks: the 64 rows of elements [32c, 32c + 32)
// form a 4 KiB block, 64 bytes per row. The transposing reads of PV (4
// consecutive rows x 64 bytes per 32 lanes) then touch 256 contiguous bytes,
// conflict-free without a swizzle, and every read of a wave differs from the
// others by a constant: one address register serves them all.
constexpr int kVBlockBytes = kBN * 64;
__device__ __forceinline__ int v_lds_off(int row, int elem) {
  return (elem >> 5) * kVBlockBytes + row * 64 + ((elem & 31) << 1);
}

// kWaves waves per workgroup: 8 (one workgroup fills a CU) or 4 (two share
// one) -- see launch_prefill_bf16
template <int D, bool CAUSAL, bool CACHE, int kWaves>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kWaves, 64 * kWaves),
                          amdgpu_waves_per_eu(2, 2)))
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
  // Workgroups are launched longest first. Slabs: by query block (causal
  // blocks near the end see the most keys). Cache: by sequence, the longest
  // first (a sequence's cached length dominates its work), then by query
  // block.
  int qrank, hg, kvh, b;
  if constexpr (!CACHE) {
    const int per_q = p.B * p.Hkv * p.n_hgrp;
    qrank = blockIdx.x / per_q;
    int rest = blockIdx.x - qrank * per_q;
    hg = rest % p.n_hgrp;
    rest /= p.n_hgrp;
    kvh = rest % p.Hkv;
    b = rest / p.Hkv;
  } else {
    const int per_s = p.Hkv * p.n_hgrp;
    const int per_b = p.n_qblk * per_s;
    const int slot = blockIdx.x / per_b;
    int rest = blockIdx.x - slot * per_b;
    qrank = rest / per_s;
    rest -= qrank * per_s;
    hg = rest % p.n_hgrp;
    kvh = rest / p.n_hgrp;
    b = slot;
    if (p.B <= 64) {
      // the sequence of rank `slot` when ordered by length (longest first,
      // ties by index): lane l ranks sequence l against all others
      const int n_l = lane < p.B ? p.seq_lens[lane] : 0;
      int rank = 0;
      for (int j = 0; j < p.B; ++j) {
        const int n_j = __builtin_amdgcn_readlane(n_l, j);
        rank += (n_j > n_l || (n_j == n_l && j < lane)) ? 1 : 0;
      }
      const unsigned long long hit = __builtin_amdgcn_ballot_w64(lane < p.B && rank == slot);
      b = hit != 0 ? __builtin_ctzll(hit) : slot;
    }
    b = __builtin_amdgcn_readfirstlane(b);
  }
  const int qblk = CAUSAL ? (p.n_qblk - 1 - qrank) : qrank;

  const int head_local = wave % p.hw;
  const int sub = wave / p.hw;
  const int hq = kvh * p.G + hg * p.hw + head_local;
  const int q0 = qblk * 32 * p.pw;
  const int my_q = q0 + sub * 32 + l32;

  // keys of this sequence and the position of query row 0
  int nk = p.Nk;
  int qoff = p.q_offset;
  if constexpr (CACHE) {
    long long cap = p.max_len;
    if (p.table != nullptr && (long long)p.max_blocks * kBlockTokens < cap)
      cap = (long long)p.max_blocks * kBlockTokens;
    const int n = p.seq_lens[b];
    nk = n < 0 ? 0 : (n > cap ? (int)cap : n);
    qoff = nk - p.Nq;
  }

  int kend = nk;
  if (CAUSAL) {
    const int last_row = min(q0 + 32 * p.pw, p.Nq) - 1;
    const long long lim = (long long)last_row + qoff + 1;
    if (lim < kend) kend = (int)(lim < 0 ? 0 : lim);
  }
  const int ntiles = (kend + kBN - 1) / kBN;
  long long mask_from = nk;  // first key some row of the workgroup cannot see
  if (CAUSAL) {
    const long long first = (long long)q0 + qoff + 1;
    if (first < mask_from) mask_from = first;
  }
  // this lane's last visible key (clamped into int range)
  long long lim64 = CAUSAL ? (long long)my_q + qoff : (long long)nk - 1;
  if (lim64 > (long long)nk - 1) lim64 = (long long)nk - 1;
  if (lim64 < -1) lim64 = -1;
  const int lim = (int)lim64;

  // ---- Qᵀ as the B operand: lane holds row my_q, d = 16*dc + 8*g + j ---------
  bf16x8_t qf[NDC];
  {
    const __bf16* qp = p.q + b * p.sqb + hq * p.sqh + my_q * p.sqr + 8 * g;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      if (my_q < p.Nq)
        qf[dc] = *reinterpret_cast<const bf16x8_t*>(qp + 16 * dc);
      else
        qf[dc] = bf16x8_t{};
    }
  }

  // Direct global->LDS loads through buffer resources: instruction i of this
  // wave fills LDS bytes [(wave*NI + i)*1024, +1024), lane l its 16 bytes at
  // +16*l, i.e. physical chunk (lin % CPR) of tile row (lin / CPR); the lane
  // fetches the logical chunk that the swizzle stores there. Rows outside a
  // resource's range arrive as zeros (those keys are masked). With j =
  // wave*NI + i, a 1 KiB instruction covers rows 4j + lane/16 for d = 128
  // (swz = 4*(lane/16) + j%4) and rows 8j + lane/8 for d = 64 (swz = 4*(j%2)
  // + lane/16): the instruction index only flips chunk bits (one XOR).
  constexpr int kXorStep = (D == 128) ? 16 : 64;
  constexpr int RPI = 1024 / (D * 2);  // tile rows per load instruction
  auto lane_offset = [&](int row_bytes) {
    return (D == 128) ? ((lane >> 4) * row_bytes) | (16 * ((lane & 15) ^ (4 * (lane >> 4))))
                      : ((lane >> 3) * row_bytes) | (16 * ((lane & 7) ^ (lane >> 4)));
  };
  auto load_rows = [&](__amdgpu_buffer_rsrc_t rs, int soff, int row_bytes, char* dst)
      __attribute__((always_inline)) {
    int lb = lane_offset(row_bytes);
    asm volatile("" : "+v"(lb));  // recompute the offsets here instead of keeping them live
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (ATTN_LDS void*)(dst + (wave * NI + i) * 1024),
                                               16, lb ^ (kXorStep * ((wave * NI + i) & (D == 128 ? 3 : 1))),
                                               soff + i * RPI * row_bytes, 0, 0);
  };

  // V into the column-block layout: instruction j of a tile (1 KiB) holds
  // rows 16*(j%4) + lane/4 of column block j/4, 16 bytes (lane%4) each.
  auto load_v_rows = [&](__amdgpu_buffer_rsrc_t rs, int soff, int row_bytes, char* dst)
      __attribute__((always_inline)) {
    int lb = (lane >> 2) * row_bytes + 16 * (lane & 3);
    asm volatile("" : "+v"(lb));
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int j = wave * NI + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (ATTN_LDS void*)(dst + j * 1024), 16, lb,
                                               soff + 16 * (j & 3) * row_bytes + 64 * (j >> 2),
                                               0, 0);
    }
  };

  // [B, Hkv, Nk, D] slabs: one resource per K/V head (range Nk rows); the
  // tile's rows are contiguous, wave w's share starts at row (64/kWaves)*w.
  const long long kv_base = CACHE ? 0 : ((long long)b * p.Hkv + kvh) * (long long)p.Nk * D;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + kv_base), 0, CACHE ? 0 : p.Nk * D * 2,
                                        kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + kv_base), 0, CACHE ? 0 : p.Nk * D * 2,
                                        kBufferFlags);

  // Token-major cache: a 64-key tile is four 16-token blocks; each block is
  // loaded by two waves (8 rows each) through a resource that ends after the
  // block's last valid row. A tile's four block-table entries arrive by one
  // vector load (lane l holds the entry of block 4t + l%4) a step before the
  // tile's K is loaded, so they have landed at the step's load wait; the
  // wave's own entry is then a readlane and the tile's storage bits a ballot.
  // Entries past the table row clamp to its last one: those blocks lie past
  // the sequence (nk <= 16 * max_blocks), and position hides their keys.
  const int rowb = p.Hkv * D * 2;  // bytes between consecutive tokens of one head
  // A contiguous cache has no table: its block jb of sequence b starts at
  // element b * max_len * Hkv * D + jb * 16 * Hkv * D, a pool block e at
  // e * 16 * Hkv * D, so both are `seq_base + e * blk_elems` with e the
  // table entry or jb. Without a table the entry loads read seq_lens[0]
  // instead (any valid address; the value is unused), so they need no branch.
  const bool paged = p.table != nullptr;
  const long long blk_elems = (long long)kBlockTokens * p.Hkv * D;
  const long long seq_base =
      (paged ? 0 : (long long)b * p.max_len * p.Hkv * D) + (long long)kvh * D;
  const int* const trow = paged ? p.table + (long long)b * p.max_blocks : p.seq_lens;
  const int tlast = paged ? max(p.max_blocks - 1, 0) : 0;
  // entries of blocks 4t + l%4 (lane l), or of blocks 4t0 + l for the first tiles
  auto load_ents = [&](int first_block, int span) __attribute__((always_inline)) {
    return trow[min(first_block + lane % span, tlast)];
  };
  // block jb's storage: the pool entry `ent` (paged) or its place in the
  // contiguous cache; no storage (or no valid row) gives an empty range
  auto block_stored = [&](int ent) __attribute__((always_inline)) {
    return !paged || (unsigned)ent < (unsigned)p.num_blocks;
  };
  auto block_rsrc = [&](const __bf16* pool, int jb, int ent) __attribute__((always_inline)) {
    const int valid = min(kBlockTokens, nk - kBlockTokens * jb);
    const bool ok = block_stored(ent) && valid > 0;
    const long long off = seq_base + (long long)(paged ? ent : jb) * blk_elems;
    return __builtin_amdgcn_make_buffer_rsrc(
        (void*)(pool + (ok ? off : 0)), 0, ok ? (valid - 1) * rowb + D * 2 : 0, kBufferFlags);
  };
  // the waves split the tile's four 16-token blocks evenly, WB = waves per block
  constexpr int WB = kWaves / 4;
  const int wq = wave / WB;  // this wave's block of a tile
  auto load_block = [&](const __bf16* pool, int t, int ent, char* dst)
      __attribute__((always_inline)) {
    // K: wave w loads rows [16/WB*(w%WB), +16/WB) of block 4t + w/WB
    load_rows(block_rsrc(pool, 4 * t + wq, ent), (wave % WB) * (kBlockTokens / WB) * rowb, rowb,
              dst);
  };
  auto load_v_block = [&](const __bf16* pool, int t, int ent, char* dst)
      __attribute__((always_inline)) {
    // V: wave w loads column blocks [NI*(w%WB), +NI) of block q = w/WB, the
    // block's 16 rows of each (LDS bytes 1024*q of the column block)
    const __amdgpu_buffer_rsrc_t rs = block_rsrc(pool, 4 * t + wq, ent);
    int lb = (lane >> 2) * rowb + 16 * (lane & 3);
    asm volatile("" : "+v"(lb));
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int db = (wave % WB) * NI + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (ATTN_LDS void*)(dst + db * kVBlockBytes + wq * 1024), 16, lb, 64 * db, 0, 0);
    }
  };
  // lanes [l0, l0 + 4) of `ents` hold tile t's entries: bit q = block 4t + q
  // has storage (blocks past the sequence count as present; their keys are
  // masked by position)
  auto tile_ok_bits = [&](int t, int ents, int l0) -> unsigned {
    const int jb = 4 * t + lane - l0;
    const bool ok = block_stored(ents) || nk - kBlockTokens * jb <= 0;
    return (unsigned)(__builtin_amdgcn_ballot_w64(ok) >> l0) & 0xFu;
  };
  int vk = 0;         // lanes 0..3: entries of the tile whose K is loaded next
  int ent_v = 0;      // this wave's entry of the tile whose V is loaded next
  // tile t's K, V into LDS; issue_k returns the tile's block bits (cache)
  auto issue_k = [&](int t, char* dst) __attribute__((always_inline)) -> unsigned {
    if constexpr (CACHE) {
      // vk holds tile t's entries in lanes 0..3
      const int ent = __builtin_amdgcn_readlane(vk, wq);
      load_block(p.k, t, ent, dst);
      return tile_ok_bits(t, vk, 0);
    } else {
      load_rows(krs, t * kBN * D * 2 + wave * NI * 1024, D * 2, dst);
      return 0xFu;
    }
  };
  auto issue_v = [&](int t, char* dst) __attribute__((always_inline)) {
    if constexpr (CACHE)
      load_v_block(p.v, t, ent_v, dst);
    else
      load_v_rows(vrs, t * kBN * D * 2, D * 2, dst);
  };
  // block bits of tiles it, it+1, it+2 in bits [3:0], [7:4], [11:8]
  unsigned okq = 0xFFFu;

  // Sᵀ[key][row] of one tile: two 32-key halves, K (A operand) from LDS
  auto scores = [&](const char* kl, f32x16_t (&s)[2]) {
    // Each K operand read is issued four MFMAs before the MFMA that takes it;
    // the scheduling barriers keep that order (VALU and SALU work may still
    // move across them). The two 32-key halves' accumulation chains
    // alternate (MFMA i adds k-step i/2 to half i%2), so no MFMA waits on the
    // one just issued; each half still sums its k-steps in order.
    constexpr int NM = 2 * NDC;
    constexpr int LA = 4;
    bf16x8_t a[NM];
    auto rd = [&](int i) __attribute__((always_inline)) {
      return *reinterpret_cast<const bf16x8_t*>(
          kl + lds_off<D>((i & 1) * 32 + l32, 16 * (i >> 1) + 8 * g));
    };
#pragma unroll
    for (int i = 0; i < LA; ++i) a[i] = rd(i);
    s[0] = f32x16_t{};
    s[1] = f32x16_t{};
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      if (i + LA < NM) a[i + LA] = rd(i + LA);
      __builtin_amdgcn_sched_barrier(kSchedAluOnly);
      s[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], qf[i >> 1], s[i & 1], 0, 0, 0);
    }
  };
  // only tiles past the first row's diagonal, the ragged end or a missing
  // cache block hide keys
  auto needs_mask = [&](int k0) {
    return k0 + kBN > mask_from || k0 + kBN > nk || (CACHE && (okq & 0xFu) != 0xFu);
  };
  // hide the keys a row cannot see (key slot i of half kb lies in block
  // 2*kb + (i >= 8) of the tile)
  auto mask = [&](int k0, f32x16_t (&s)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
        const bool stored = !CACHE || ((okq >> (2 * kb + (i >= 8 ? 1 : 0))) & 1u);
        if (key > lim || !stored) s[kb][i] = neg_inf();
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
    // (cache) the table entries loaded last step are read only after the wait
    if constexpr (CACHE) asm volatile("" : "+v"(vk));
    if (!LAST) {
      int ent_k = 0;
      if constexpr (CACHE) ent_k = __builtin_amdgcn_readlane(vk, wq);  // tile it+2
      if (it + 2 < ntiles) okq |= issue_k(it + 2, kfree) << 8;
      issue_v(it + 1, vfree);
      if constexpr (CACHE) {
        ent_v = ent_k;
        if (it + 3 < ntiles) vk = load_ents(4 * (it + 3), 4);
      }
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
              (ATTN_LDS i16x4_t*)(vc + v_lds_off(r0, col)));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (ATTN_LDS i16x4_t*)(vc + v_lds_off(r0 + 8, col)));
          const u32x2_t lo2 = __builtin_bit_cast(u32x2_t, lo);
          const u32x2_t hi2 = __builtin_bit_cast(u32x2_t, hi);
          const u32x4_t a4 = {lo2[0], lo2[1], hi2[0], hi2[1]};
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a4), pb,
                                                            acc[db], 0, 0, 0);
        }
      }
    if (!LAST) mt = tile_max(sn);
    okq >>= 4;
  };

  if (ntiles > 0) {
    if constexpr (CACHE) {
      // the entries of tiles 0..2 (lanes 0..11), before any tile load
      const int e3 = load_ents(0, 12);
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      vk = e3;
      ent_v = __builtin_amdgcn_readlane(e3, wq);
      load_block(p.k, 0, ent_v, kb0);
      okq = tile_ok_bits(0, e3, 0);
      issue_v(0, vb0);
      if (ntiles > 1) {
        ent_v = __builtin_amdgcn_readlane(e3, 4 + wq);
        load_block(p.k, 1, ent_v, kb1);
        okq |= tile_ok_bits(1, e3, 4) << 4;
      }
      vk = __shfl(e3, 8 + (lane & 3), 64);  // tile 2's entries to lanes 0..3
    } else {
      okq = issue_k(0, kb0);
      issue_v(0, vb0);
      if (ntiles > 1) okq |= issue_k(1, kb1) << 4;
    }
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
  // A lane holds 8-byte pieces of its row; written straight out, every store
  // would touch 32 rows. The wave's 32 rows therefore pass through LDS (its
  // own 32 rows of the tile buffers, free once every wave is past its last
  // tile: the barrier below) and leave as whole rows, 16 bytes per lane.
  const float l_tot = sum_across_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  constexpr int RB = D * 2;    // bytes per row
  constexpr int NCH = D / 8;   // 16-byte chunks per row; chunk c of row r sits at c ^ (r % NCH)
  char* stage = ((wave >> 1) == 0 ? kb0 : (wave >> 1) == 1 ? kb1 : (wave >> 1) == 2 ? vb0 : vb1) +
                (wave & 1) * 32 * RB;
  static_assert(2 * 32 * RB == TILE, "two waves' rows fill one tile buffer");
  __syncthreads();
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      f32x4_t v4 = {acc[db][4 * ii] * inv, acc[db][4 * ii + 1] * inv, acc[db][4 * ii + 2] * inv,
                    acc[db][4 * ii + 3] * inv};
      const int c = 4 * db + ii;
      *reinterpret_cast<bf16x4_t*>(stage + l32 * RB + ((c ^ (l32 & (NCH - 1))) << 4) + 8 * g) =
          __builtin_convertvector(v4, bf16x4_t);
    }
  __syncthreads();
  {
    const int row0 = q0 + sub * 32;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      const int r = i * (64 / NCH) + lane / NCH;
      const int c = lane % NCH;
      const u32x4_t val =
          *reinterpret_cast<const u32x4_t*>(stage + r * RB + ((c ^ (r & (NCH - 1))) << 4));
      if (row0 + r < p.Nq)
        *reinterpret_cast<u32x4_t*>(p.o + b * p.sqb + hq * p.sqh + (row0 + r) * p.sqr + 8 * c) =
            val;
    }
  }
  if (my_q < p.Nq) {
    if (g == 0 && p.lse != nullptr) {
      p.lse[((long long)b * p.Hq + hq) * p.Nq + my_q] =
          l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : neg_inf();
    }
  }
}

template <int D, bool CAUSAL, bool CACHE, int W>
hipError_t launch_typed(const PrefillParams& pp, int nblocks, hipStream_t s) {
  hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL, CACHE, W>), dim3(nblocks), dim3(W * 64), 0,
                     s, pp);
  return hipGetLastError();
}

template <int D, int W>
hipError_t launch_d(const PrefillParams& pp, bool causal, bool cache, int nblocks, hipStream_t s) {
  if (cache)
    return causal ? launch_typed<D, true, true, W>(pp, nblocks, s)
                  : launch_typed<D, false, true, W>(pp, nblocks, s);
  return causal ? launch_typed<D, true, false, W>(pp, nblocks, s)
                : launch_typed<D, false, false, W>(pp, nblocks, s);
}

}  // namespace

// 8-wave workgroups (the two waves on a SIMD step through the same tiles)
// when they fill the chip: one per CU at least, and under a causal mask
// (workgroups of unequal length) two per CU, so that long and short ones can
// follow each other. Otherwise two 4-wave workgroups share each CU (a causal
// prefill of 2048 rows: 49 against 58 us; a non-causal one of 1024 rows:
// 27-30 against 36 us).
int prefill_bf16_waves(int B, int Hq, int Hkv, int Nq, int causal, int compute_units) {
  const int G = Hq / Hkv;
  const int hw = (G % 4 == 0) ? 4 : ((G % 2 == 0) ? 2 : 1);
  const long long per_row_block = (long long)B * Hkv * (G / hw);
  const long long nq8 = (Nq + 32 * (8 / hw) - 1) / (32 * (8 / hw));
  const long long need8 = (long long)compute_units * (causal ? 2 : 1);
  return nq8 * per_row_block >= need8 ? 8 : 4;
}

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
  pp.n_hgrp = pp.G / pp.hw;
  const int W = a.waves != 0 ? a.waves
                             : prefill_bf16_waves(a.B, a.Hq, a.Hkv, a.Nq, a.causal,
                                                  device_compute_units());
  if (W != 4 && W != 8) return hipErrorInvalidValue;
  pp.pw = W / pp.hw;
  pp.n_qblk = (a.Nq + 32 * pp.pw - 1) / (32 * pp.pw);
  pp.c = a.scale * kLog2e;
  pp.q_offset = a.q_offset;
  const long long d = a.d;
  if (a.q_token_major) {  // [B, Nq, Hq, d]
    pp.sqr = (long long)a.Hq * d;
    pp.sqh = d;
    pp.sqb = (long long)a.Nq * a.Hq * d;
  } else {  // [B, Hq, Nq, d]
    pp.sqr = d;
    pp.sqh = (long long)a.Nq * d;
    pp.sqb = (long long)a.Hq * a.Nq * d;
  }
  pp.table = a.block_table;
  pp.max_blocks = a.max_blocks;
  pp.num_blocks = a.num_blocks;
  pp.max_len = a.max_len;
  pp.seq_lens = a.seq_lens;
  const long long nblocks = (long long)pp.n_qblk * a.B * a.Hkv * pp.n_hgrp;
  if (nblocks <= 0) return hipSuccess;
  if (nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const bool cache = a.cache != 0;
  if (W == 8)
    return a.d == 128 ? launch_d<128, 8>(pp, a.causal, cache, (int)nblocks, s)
                      : launch_d<64, 8>(pp, a.causal, cache, (int)nblocks, s);
  return a.d == 128 ? launch_d<128, 4>(pp, a.causal, cache, (int)nblocks, s)
                    : launch_d<64, 4>(pp, a.causal, cache, (int)nblocks, s);
}

}  // namespace attn
