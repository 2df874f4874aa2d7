// Split-KV decode against a paged or contiguous cache of bf16 or E4M3 codes,
// gfx950.
//
// Method: Flash-Decoding ("[BEE-30062] FlashAttention 與高效注意力核心",
// Background): during decode the batch and the query length are small, so
// the keys of each sequence are cut into chunks processed in parallel; each
// chunk yields a partial softmax result that a second pass merges in a
// numerically stable way. The cache is either the (batch, seqlen, n_kv_heads,
// head_dim) layout of "為長上下文推論啟用 FlashDecoding" or the same rows cut
// into 16-token blocks behind a page table ("Phase 07 · 12", section "Paged
// attention"). Query row i of sequence b sits at position seq_len - Nq + i
// ("Effizienz", "Der wichtige Maskenfehler beim Cache").
//
// Mapping onto CDNA4. Decode reads every K/V byte once and does ~4 flops per
// byte, so it is bound by HBM bandwidth; the kernel's job is to keep enough
// bytes in flight and to spend little issue bandwidth per byte.
//   * Work split ("stream-K"): per K/V head, the 32-key steps of all
//     sequences are laid end to end and the head's Wh waves each take an
//     equal contiguous range of them, so the load stays balanced whatever the
//     sequence lengths. Wave w serves head w % Hkv, so the waves resident
//     side by side read the same token rows of every head. A wave writes one
//     partial result per sequence piece it covers; the piece of wave j of
//     (K/V head, row group) vh in sequence b lives at index vh*(Wh + B) + j + b,
//     which is unique. With fewer steps than waves only the first (number of
//     steps) waves of a head run.
//   * The G·Nq query rows that share a K/V head (G = Hq/Hkv query heads ×
//     Nq new tokens, up to 64) are cut into groups of 16, each group the 16
//     columns of v_mfma_f32_16x16x32_bf16: a K/V byte is loaded once per
//     group and used by all of its rows. With G·Nq <= 16 (the usual decode
//     shapes) there is one group, so every K/V byte is loaded once; the
//     groups of one head run on neighbouring waves, so further groups
//     mostly hit in L2.
//   * Sᵀ = K·Qᵀ: K rows come straight from global memory into the A operand
//     (lane = key, 8 consecutive d per lane), Qᵀ sits in registers.
//   * Oᵀ = Vᵀ·Pᵀ: V rows are loaded 16 bytes per lane (8 consecutive d of one
//     key, a whole 256-byte row per 16 lanes) and transposed in registers with
//     byte permutes into the A operand, one MFMA per d residue mod 8. Pᵀ is
//     the Sᵀ accumulator packed to bf16.
//   * Each 16-token stretch of a head is one buffer resource whose range ends
//     after its last valid row: tokens past seq_len and blocks outside the
//     pool read as zeros (and are masked), so stale or NaN cache contents
//     cannot leak into the result and no load needs a branch.
//   * Partial results (normalised O and base-2 LSE per piece and row) go to
//     the caller's workspace; the combine kernel (one wave per output row)
//     merges the pieces of each row in wave order with weights
//     exp2(LSE_s - max LSE_s) and writes O (bf16) and the natural-log LSE.
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

struct DecodeParams {
  const __bf16* q;
  const char* k;          // cache bytes: bf16, or E4M3 codes (KV8)
  const char* v;
  const float* ksc;       // KV8: per-K/V-head scales of the codes
  const float* vsc;
  CacheView cv;
  const int32_t* seq_lens;
  __bf16* o;
  float* lse;
  float* part_o;          // [HV * (Wh + B) pieces][MP][D]
  float* part_lse;        // [HV * (Wh + B) pieces][MP]
  long long* prefix;      // [B + 1]: 32-key steps of sequences 0..b-1
  int B, Hq, Hkv, Nq, G, M;
  int RG;                 // groups of up to 16 query rows per K/V head
  int MP;                 // rows per group (min(M, 16))
  int HV;                 // (K/V head, row group) pairs: Hkv * RG
  int W;                  // waves launched: Wh per (K/V head, row group)
  int Wh;
  float c;  // scale * log2(e)
  int causal;
};

// 32-key steps of sequence b (its clamped length rounded up)
__device__ __forceinline__ int seq_steps(const DecodeParams& p, int b) {
  return (cache_len_clamped(p.cv, p.seq_lens[b]) + 31) >> 5;
}

// A value every lane of the wave holds alike, moved to scalar registers. The
// compiler cannot prove that values read from memory with a uniform address,
// or taken out of a shuffle, are uniform; without this, the buffer resources
// built from them live in vector registers and every load gets a loop over
// lanes around it.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ long long uniform(long long x) {
  const int lo = __builtin_amdgcn_readfirstlane((int)(x & 0xffffffffLL));
  const int hi = __builtin_amdgcn_readfirstlane((int)(x >> 32));
  return ((long long)hi << 32) | (unsigned)lo;
}

__device__ __forceinline__ long long wave_sum64(long long x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// inclusive prefix sum over the 64 lanes
__device__ __forceinline__ int wave_scan(int x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

// the wave whose range of steps contains step x: largest w with w*U/W <= x
__device__ __forceinline__ int wave_of(long long x, long long U, int W) {
  return (int)(((x + 1) * W - 1) / U);
}

__device__ __forceinline__ uint32_t perm_lo(uint32_t x, uint32_t y) {
  // (low 16 bits of x) | (low 16 bits of y) << 16
  return __builtin_amdgcn_perm(y, x, 0x05040100u);
}
__device__ __forceinline__ uint32_t perm_hi(uint32_t x, uint32_t y) {
  // (high 16 bits of x) | (high 16 bits of y) << 16
  return __builtin_amdgcn_perm(y, x, 0x07060302u);
}

constexpr float kTau = 8.0f;               // rescale only when a row max grows by more than 2^8
constexpr int kBufferFlags = 0x00020000;  // raw buffer resource, 32-bit dword data

// K/V of one 32-key step as loaded.
template <int D, bool KV8>
struct StepRegs;
template <int D>
struct StepRegs<D, false> {  // bf16: already the MFMA operands
  bf16x8_t kf[2][D / 32];    // A operand of Sᵀ: lane = key (r16) of half h2, 8 d at 32c + 8g
  u32x4_t vv[2][4];          // 8 d (chunk r16) of keys 16*h2 + 4*g + jj
};
template <int D>
struct StepRegs<D, true> {  // E4M3 codes, widened to bf16 where they are used
  u32x4_t kq[2][D / 64];    // key r16 of half h2, 16 d at 64*c2 + 16*g
  u32x2_t vq[2][4];         // 8 d (d = 8*r16 ...) of keys 16*h2 + 4*g + jj
};

// two E4M3 codes (bytes 2*hi, 2*hi+1 of w) as a bf16 pair packed in a dword;
// E4M3 values are exact in bf16
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t,
                            __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI));
}

// One 16-token stretch of one K/V head as a buffer resource whose range ends
// after its last valid row: loads past it (tokens beyond the sequence, a
// block outside the pool) return zeros, with no branch per load.
struct Span {
  __amdgpu_buffer_rsrc_t k, v;
  bool ok;  // the stretch has storage (its keys may be visible)
};

// 32-key steps per pipeline: the loads of DEPTH - 1 steps are in flight while
// one is computed (an E4M3 step is half the bytes, so it keeps more in flight)
constexpr int kDepthBf16 = 2;
constexpr int kDepthFp8 = 3;

template <int D, bool KV8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_partial_kernel(DecodeParams p) {
  constexpr int EB = KV8 ? 1 : 2;  // bytes per cached element
  constexpr int DEPTH = KV8 ? kDepthFp8 : kDepthBf16;
  constexpr int NC = D / 32;  // MFMAs per 16 keys for Sᵀ (32 d each)
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;  // query row (Sᵀ/Oᵀ column) of this lane
  const int g = lane >> 4;    // lane group 0..3
  // wave-uniform indices live in scalar registers
  const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (w >= p.W) return;

  // ---- this wave's range of 32-key steps --------------------------------------
  // Wave w serves row group rg of K/V head kvh, vh = w % HV = kvh*RG + rg;
  // the Wh waves of a (head, row group) split its steps of all sequences
  // laid end to end. Neighbouring waves thus read the same token rows of
  // the same or neighbouring heads.
  const int vh = w % p.HV;
  const int kvh = vh / p.RG;
  const int rg = vh - kvh * p.RG;
  const int j = w / p.HV;
  // Total steps per head; wave 0 also records the per-sequence prefix for the combine.
  long long tot = 0;
  for (int b0 = 0; b0 < p.B; b0 += 64) {
    const int b = b0 + lane;
    const int st = b < p.B ? seq_steps(p, b) : 0;
    const int incl = wave_scan(st, lane);
    if (w == 0) {
      if (b < p.B) p.prefix[b] = tot + incl - st;
      if (b == p.B - 1) p.prefix[p.B] = tot + incl;
    }
    tot += __shfl(incl, 63, 64);
  }
  tot = uniform(tot);
  // at most one wave per step, so every wave's range is non-empty and the
  // pieces of a sequence come from consecutive waves with no gap
  const int We = (int)min((long long)p.Wh, tot);
  if (j >= We) return;
  const long long x0 = (long long)j * tot / We;
  const long long x1 = (long long)(j + 1) * tot / We;
  // the sequence holding step x0: first b with prefix[b + 1] > x0
  int b = 0;
  long long pb = 0;  // prefix[b]
  {
    long long run = 0;
    for (int b0 = 0; b0 < p.B; b0 += 64) {
      const int bb = b0 + lane;
      const int st = bb < p.B ? seq_steps(p, bb) : 0;
      const int incl = wave_scan(st, lane);
      const unsigned long long hit = __builtin_amdgcn_ballot_w64(bb < p.B && run + incl > x0);
      if (hit != 0) {
        const int l = __builtin_ctzll(hit);
        b = b0 + l;
        pb = run + __shfl(incl - st, l, 64);
        break;
      }
      run += __shfl(incl, 63, 64);
    }
  }
  b = uniform(b);
  pb = uniform(pb);

  const int rowb = p.cv.hkv * D * EB;  // bytes between consecutive tokens of one head
  // loop-invariant lane byte offsets inside a 16-token stretch
  // K: token r16, 16 bytes at 16*g (+64 per further load); V: token 4*g (+jj
  // via soffset), the 8 d from 8*r16
  const int koff = r16 * rowb + 16 * g;
  // A V chunk holds 8 d; with D = 64 only lanes r16 < 8 have one inside the
  // head, and the others take an offset past every range (zeros, no memory
  // traffic) instead of the neighbouring head's bytes. Their PV outputs (d
  // rows 64..127) are never stored.
  const int voff = 8 * r16 < D ? (4 * g) * rowb + 8 * EB * r16 : 0x40000000;
  const int row = 16 * rg + r16;                // rows r = qi * G + h, r < M
  const bool row_ok = r16 < p.MP && row < p.M;
  const int qi = row_ok ? row / p.G : 0;
  const int hrow = row_ok ? row % p.G : 0;

  // ---- one piece: keys [kb0, ke) of head kvh of sequence b ---------------------
  auto piece = [&](int b, int kvh, int n, int kb0, int ke, long long id)
      __attribute__((always_inline)) {
    float* po = p.part_o + id * p.MP * D;
    float* pl = p.part_lse + id * p.MP;
    int limit = ke;  // keys of this piece visible to the row: [kb0, limit)
    if (p.causal) limit = min(limit, n - p.Nq + qi + 1);

    // Qᵀ as the B operand: lane holds row r16 and, for MFMA c, the 8 d that
    // the K operand of lane group g holds: d = 32*c + 8*g + j (bf16 cache) or
    // d = 64*(c/2) + 16*g + 8*(c%2) + j (E4M3 cache: one 16-byte load per
    // lane holds two MFMAs' worth of K)
    bf16x8_t qf[NC];
    {
      const __bf16* qp =
          p.q + (((long long)b * p.Nq + qi) * p.Hq + (long long)kvh * p.G + hrow) * D;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int d0 = KV8 ? 64 * (c >> 1) + 16 * g + 8 * (c & 1) : 32 * c + 8 * g;
        qf[c] = row_ok ? *reinterpret_cast<const bf16x8_t*>(qp + d0) : bf16x8_t{};
      }
    }
    // score scale in base 2, and the factor of O; E4M3 codes carry per-head scales
    const float cs = KV8 ? p.c * p.ksc[kvh] : p.c;
    const float os = KV8 ? p.vsc[kvh] : 1.f;

    f32x4_t acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = f32x4_t{};
    float m_run = neg_inf();
    float l_run = 0.f;

    // Paged: the table entries of 64 consecutive blocks starting at tab_base,
    // one per lane, fetched with one load and picked with readlane, so a
    // stretch's K/V loads do not wait on a table load of their own.
    int tab = -1;
    int tab_base = -64;
    // The stretch of tokens [t0, t0 + 16) of this head (t0 a multiple of 16);
    // rows at or past n read as zeros.
    auto span = [&](int t0) __attribute__((always_inline)) {
      Span sp;
      const int valid = min(16, n - t0);
      long long row = -1;
      if (valid > 0) {  // t0 < n, which is within max_len and the table's capacity
        if (p.cv.table == nullptr) {
          row = ((long long)b * p.cv.max_len + t0) * p.cv.hkv * D;
        } else {
          const int blk = t0 / kBlockTokens;
          if (blk - tab_base >= 64) {
            tab_base = blk;
            const int i = blk + lane;
            tab = i < p.cv.max_blocks ? p.cv.table[(long long)b * p.cv.max_blocks + i] : -1;
          }
          const int e = __builtin_amdgcn_readlane(tab, blk - tab_base);
          if (e >= 0 && e < p.cv.num_blocks) row = (long long)e * kBlockTokens * p.cv.hkv * D;
        }
      }
      sp.ok = row >= 0;
      const long long base = sp.ok ? (row + (long long)kvh * D) * EB : 0;
      const int bytes = sp.ok ? (valid - 1) * rowb + D * EB : 0;
      sp.k = __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + base), 0, bytes, kBufferFlags);
      sp.v = __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + base), 0, bytes, kBufferFlags);
      return sp;
    };

    auto load = [&](const Span (&sp)[2], StepRegs<D, KV8>& r) __attribute__((always_inline)) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        if constexpr (KV8) {
#pragma unroll
          for (int c2 = 0; c2 < D / 64; ++c2)
            r.kq[h2][c2] = __builtin_bit_cast(
                u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(sp[h2].k, koff + 64 * c2, 0, 0));
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            r.vq[h2][jj] = __builtin_bit_cast(
                u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(sp[h2].v, voff, jj * rowb, 0));
        } else {
#pragma unroll
          for (int c = 0; c < NC; ++c)
            r.kf[h2][c] = __builtin_bit_cast(
                bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(sp[h2].k, koff + 64 * c, 0, 0));
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            r.vv[h2][jj] = __builtin_bit_cast(
                u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(sp[h2].v, voff, jj * rowb, 0));
        }
      }
    };
    // the MFMA operands of a step: K fragment (h2, c) and V chunk (h2, jj)
    auto kfrag = [&](const StepRegs<D, KV8>& r, int h2, int c) __attribute__((always_inline)) {
      if constexpr (KV8) {
        const u32x4_t w = r.kq[h2][c >> 1];
        const uint32_t w0 = (c & 1) ? w[2] : w[0];
        const uint32_t w1 = (c & 1) ? w[3] : w[1];
        const u32x4_t f = {fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0),
                           fp8x2_to_bf16x2<false>(w1), fp8x2_to_bf16x2<true>(w1)};
        return __builtin_bit_cast(bf16x8_t, f);
      } else {
        return r.kf[h2][c];
      }
    };
    auto vchunk = [&](const StepRegs<D, KV8>& r, int h2, int jj) __attribute__((always_inline)) {
      if constexpr (KV8) {
        const u32x2_t w = r.vq[h2][jj];
        const u32x4_t f = {fp8x2_to_bf16x2<false>(w[0]), fp8x2_to_bf16x2<true>(w[0]),
                           fp8x2_to_bf16x2<false>(w[1]), fp8x2_to_bf16x2<true>(w[1])};
        return f;
      } else {
        return r.vv[h2][jj];
      }
    };

    auto compute = [&](int k0, const Span (&sp)[2], const StepRegs<D, KV8>& r)
        __attribute__((always_inline)) {
      f32x4_t s[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        s[h2] = f32x4_t{};
#pragma unroll
        for (int c = 0; c < NC; ++c)
          s[h2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfrag(r, h2, c), qf[c], s[h2], 0, 0, 0);
      }
      float mx = neg_inf();
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = k0 + 16 * h2 + 4 * g + i;
          if (!sp[h2].ok || key >= limit) s[h2][i] = neg_inf();
          mx = __builtin_elementwise_maximum(mx, s[h2][i]);
        }
      mx = max_across_rows16(mx);
      mx = max_across_halves(mx);
      const float mt = mx * cs;
      // the reference max only moves (and O, l are rescaled) when the row max
      // jumps by more than kTau
      const bool need = mt > m_run + kTau;
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
        const float m_new = need ? mt : m_run;
        const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;  // 0 from -inf
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] *= alpha;
      }
      const float m_use = (m_run == neg_inf()) ? 0.f : m_run;
      float rs = 0.f;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[h2][i], cs, -m_use));
          s[h2][i] = e;
          rs += e;
        }
      l_run += rs;

      // Oᵀ += Vᵀ Pᵀ: key slot j of lane group g is key 16*(j/4) + 4*g + j%4
      const bf16x4_t p0 = __builtin_convertvector(s[0], bf16x4_t);
      const bf16x4_t p1 = __builtin_convertvector(s[1], bf16x4_t);
      const bf16x8_t pb8 = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
      u32x4_t vv[2][4];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) vv[h2][jj] = vchunk(r, h2, jj);
#pragma unroll
      for (int e = 0; e < 4; ++e) {  // dword e of each V chunk holds d = 8*r16 + 2e, 2e+1
        u32x4_t lo, hi;
        lo[0] = perm_lo(vv[0][0][e], vv[0][1][e]);
        lo[1] = perm_lo(vv[0][2][e], vv[0][3][e]);
        lo[2] = perm_lo(vv[1][0][e], vv[1][1][e]);
        lo[3] = perm_lo(vv[1][2][e], vv[1][3][e]);
        hi[0] = perm_hi(vv[0][0][e], vv[0][1][e]);
        hi[1] = perm_hi(vv[0][2][e], vv[0][3][e]);
        hi[2] = perm_hi(vv[1][0][e], vv[1][1][e]);
        hi[3] = perm_hi(vv[1][2][e], vv[1][3][e]);
        acc[2 * e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, lo),
                                                             pb8, acc[2 * e], 0, 0, 0);
        acc[2 * e + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, hi),
                                                                 pb8, acc[2 * e + 1], 0, 0, 0);
      }
    };

    // software pipeline: the block lookups and loads of step k+DEPTH-1 are
    // issued (into the registers step k-1 has just released) before step k
    // is computed, so DEPTH-1 steps of K/V are in flight per wave
    StepRegs<D, KV8> r[DEPTH];
    Span sp[DEPTH][2];
#pragma unroll
    for (int j = 0; j + 1 < DEPTH; ++j) {
      if (kb0 + 32 * j < ke) {
        sp[j][0] = span(kb0 + 32 * j);
        sp[j][1] = span(kb0 + 32 * j + 16);
        load(sp[j], r[j]);
      }
    }
    for (int k0 = kb0; k0 < ke; k0 += 32 * DEPTH) {
#pragma unroll
      for (int j = 0; j < DEPTH; ++j) {
        const int kc = k0 + 32 * j;
        if (kc >= ke) break;
        const int jn = (j + DEPTH - 1) % DEPTH;
        const int kn = kc + 32 * (DEPTH - 1);
        if (kn < ke) {
          sp[jn][0] = span(kn);
          sp[jn][1] = span(kn + 16);
          load(sp[jn], r[jn]);
        }
        compute(kc, sp[j], r[j]);
      }
    }

    // partial result of this piece
    float l_tot = sum_across_rows16(l_run);
    l_tot = sum_across_halves(l_tot);
    const float inv = l_tot > 0.f ? os / l_tot : 0.f;
    if (row_ok) {
      // Oᵀ element (m = 4*g + i, c) is d = 8*m + c = 32*g + 8*i + c
      if (32 * g < D) {
        float* dst = po + (long long)r16 * D + 32 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f32x4_t a = {acc[0][i] * inv, acc[1][i] * inv, acc[2][i] * inv, acc[3][i] * inv};
          f32x4_t bq = {acc[4][i] * inv, acc[5][i] * inv, acc[6][i] * inv, acc[7][i] * inv};
          *reinterpret_cast<f32x4_t*>(dst + 8 * i) = a;
          *reinterpret_cast<f32x4_t*>(dst + 8 * i + 4) = bq;
        }
      }
      if (g == 0) pl[r16] = l_tot > 0.f ? m_run + __builtin_amdgcn_logf(l_tot) : neg_inf();
    }
  };

  // ---- walk the sequences that [x0, x1) covers ---------------------------------
  int st_b = uniform(seq_steps(p, b));
  long long seg = pb;  // first step of sequence b
  long long x = x0;
  while (x < x1) {
    const int lo = (int)(x - seg);
    const int hi = (int)min((long long)st_b, x1 - seg);
    const int n = uniform(cache_len_clamped(p.cv, p.seq_lens[b]));
    piece(b, kvh, n, 32 * lo, min(n, 32 * hi), (long long)vh * (p.Wh + p.B) + j + b);
    x = seg + hi;
    seg += st_b;
    do {
      ++b;
      st_b = b < p.B ? uniform(seq_steps(p, b)) : 1;
    } while (b < p.B && st_b == 0);
  }
}

// One wave per (sequence, K/V head, query row), four rows per workgroup.
// The pieces of sequence b for row r were written by waves w_first..w_last
// of the row's (K/V head, row group) vh at index vh*(Wh + B) + b + j. The
// wave's four 16-lane groups take every fourth piece (group q: pieces q,
// q+4, ...), weight them by exp2(LSE - max LSE), and the group sums are then
// added in a fixed order with lane exchanges, so the result is
// deterministic. A lane owns D/16 consecutive output elements.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeParams p) {
  constexpr int E = D / 16;  // elements per lane
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4;
  const int l16 = lane & 15;
  const long long rid = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rid >= (long long)p.B * p.Hkv * p.M) return;
  const int r = (int)(rid % p.M);
  const long long bk = rid / p.M;
  const int b = (int)(bk / p.Hkv);
  const int kvh = (int)(bk % p.Hkv);
  const int qi = r / p.G;
  const int hq = kvh * p.G + r % p.G;
  const long long T = p.prefix[p.B];  // steps per (head, row group)
  const int We = (int)min((long long)p.Wh, T);  // waves per (head, row group) that took a range
  const int st_b = seq_steps(p, b);
  int w_first = 0, w_last = -1;
  if (st_b > 0) {
    w_first = wave_of(p.prefix[b], T, We);
    w_last = wave_of(p.prefix[b] + st_b - 1, T, We);
  }
  const int vh = kvh * p.RG + r / 16;  // row r lives in row group r / 16, slot r % 16
  const long long first = (long long)vh * (p.Wh + p.B) + b + w_first;
  const float* pl = p.part_lse + first * p.MP + (r % 16);
  const float* po = p.part_o + (first * p.MP + (r % 16)) * D + E * l16;
  const long long so = (long long)p.MP * D;  // stride between pieces in part_o
  const int used = w_last - w_first + 1;

  float mx = neg_inf();
  for (int i = grp; i < used; i += 4)
    mx = __builtin_elementwise_maximum(mx, pl[(long long)i * p.MP]);
  mx = __builtin_elementwise_maximum(mx, __shfl_xor(mx, 16, 64));
  mx = __builtin_elementwise_maximum(mx, __shfl_xor(mx, 32, 64));
  f32x4_t acc[E / 4];
#pragma unroll
  for (int e = 0; e < E / 4; ++e) acc[e] = f32x4_t{};
  float tot = 0.f;
  if (mx != neg_inf()) {
    for (int i = grp; i < used; i += 4) {
      const float ls = pl[(long long)i * p.MP];
      const float wt = (ls == neg_inf()) ? 0.f : __builtin_amdgcn_exp2f(ls - mx);
      tot += wt;
      const f32x4_t* src = reinterpret_cast<const f32x4_t*>(po + (long long)i * so);
#pragma unroll
      for (int e = 0; e < E / 4; ++e) acc[e] += wt * src[e];
    }
  }
  // add the four groups' sums: (g0 + g1) + (g2 + g3) in every lane
#pragma unroll
  for (int sh = 16; sh <= 32; sh <<= 1) {
    tot += __shfl_xor(tot, sh, 64);
#pragma unroll
    for (int e = 0; e < E / 4; ++e)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[e][c] += __shfl_xor(acc[e][c], sh, 64);
  }
  if (grp == 0) {
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
    __bf16* op = p.o + (((long long)b * p.Nq + qi) * p.Hq + hq) * D + E * l16;
#pragma unroll
    for (int e = 0; e < E / 4; ++e)
      *reinterpret_cast<bf16x4_t*>(op + 4 * e) = __builtin_convertvector(acc[e] * inv, bf16x4_t);
    if (l16 == 0 && p.lse != nullptr)
      p.lse[((long long)b * p.Hq + hq) * p.Nq + qi] =
          tot > 0.f ? (mx + __builtin_amdgcn_logf(tot)) * kLn2 : neg_inf();
  }
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s) {
  DecodeParams pp;
  pp.q = static_cast<const __bf16*>(a.q);
  pp.k = static_cast<const char*>(a.k_cache);
  pp.v = static_cast<const char*>(a.v_cache);
  pp.ksc = a.k_scale;
  pp.vsc = a.v_scale;
  pp.cv.table = a.block_table;
  pp.cv.max_blocks = a.max_blocks;
  pp.cv.num_blocks = a.num_blocks;
  pp.cv.max_len = a.max_seq_len;
  pp.cv.hkv = a.Hkv;
  pp.cv.d = a.d;
  pp.seq_lens = a.seq_lens;
  pp.o = static_cast<__bf16*>(a.o);
  pp.lse = a.lse;
  pp.part_o = a.part_o;
  pp.part_lse = a.part_lse;
  pp.prefix = a.prefix;
  pp.B = a.B;
  pp.Hq = a.Hq;
  pp.Hkv = a.Hkv;
  pp.Nq = a.Nq;
  pp.G = a.Hq / a.Hkv;
  pp.M = pp.G * a.Nq;
  if (pp.M <= 0) return hipSuccess;  // no query rows
  pp.RG = (pp.M + 15) / 16;
  pp.MP = pp.M < 16 ? pp.M : 16;
  pp.HV = a.Hkv * pp.RG;
  pp.Wh = a.workers / pp.HV;
  pp.W = pp.Wh * pp.HV;
  pp.c = a.scale * kLog2e;
  pp.causal = a.causal;
  if (a.B <= 0 || pp.Wh <= 0) return hipSuccess;
  const long long blocks = (pp.W + 3) / 4;
  const long long cblocks = ((long long)a.B * a.Hkv * pp.M + 3) / 4;
  if (blocks > 0x7fffffffLL || cblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  auto partial = a.d == 128 ? (a.kv8 ? decode_partial_kernel<128, true>
                                      : decode_partial_kernel<128, false>)
                           : (a.kv8 ? decode_partial_kernel<64, true>
                                    : decode_partial_kernel<64, false>);
  hipLaunchKernelGGL(partial, dim3((int)blocks), dim3(256), 0, s, pp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.d == 128)
    hipLaunchKernelGGL(decode_combine_kernel<128>, dim3((int)cblocks), dim3(256), 0, s, pp);
  else
    hipLaunchKernelGGL(decode_combine_kernel<64>, dim3((int)cblocks), dim3(256), 0, s, pp);
  return hipGetLastError();
}

}  // namespace attn
