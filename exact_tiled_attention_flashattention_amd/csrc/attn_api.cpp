// Host side of the C ABI declared in include/attn.h: argument validation,
// dispatch on dtype / head dim / causal, split sizing, launch on the caller's
// stream. Nothing here allocates, frees or synchronises; every error is
// detected before the first launch.
#include "attn.h"

#include <atomic>
#include <cmath>
#include <cstdint>

#include "launch.h"

namespace attn {

int device_compute_units() {
  constexpr int kFallbackCus = 256;  // MI355X, when no device can be queried
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return kFallbackCus;
  }
  int cus = cache[dev].load(std::memory_order_relaxed);
  if (cus > 0) return cus;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0) {
    (void)hipGetLastError();
    return kFallbackCus;
  }
  cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

}  // namespace attn

namespace {

constexpr int kWavesPerCu = 4;          // default bf16-cache decode workers per CU (one per SIMD)
constexpr int kWavesPerCuFp8 = 4;       // default fp8-cache decode workers per CU (one per SIMD)
constexpr int kMaxWorkers = 1 << 20;
constexpr int kMaxRows = 64;            // G*Nq rows per K/V head (four groups of 16)

bool misaligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

bool head_dim_ok(int d) { return d == 64 || d == 128; }

int status_of(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_EHIP; }

// Default number of decode workers: one per SIMD of the current device, for
// either cache format (the paged 4-token workload over an fp8 cache, on one
// MI355X: 122.5-124.5 us with one wave per SIMD, 126.7-126.9 us with two, and
// 137-144 us for counts that are not a multiple of the SIMD count).
int default_workers(bool kv8) {
  return attn::device_compute_units() * (kv8 ? kWavesPerCuFp8 : kWavesPerCu);
}

// Query rows that share a K/V head, and the (K/V head, group of up to 16
// rows) pairs the decode kernel spreads its workers over (at least Hkv).
long long decode_rows(int Hq, int Hkv, int Nq) { return (long long)(Hq / Hkv) * Nq; }
int virtual_heads(int Hq, int Hkv, int Nq) {
  const long long M = decode_rows(Hq, Hkv, Nq);
  return Hkv * (M > 16 ? (int)((M + 15) / 16) : 1);
}

// Workers actually launched: a whole number (at least one) per (K/V head,
// row group).
int plan_workers(int num_splits, int Hq, int Hkv, int Nq, bool kv8) {
  const int hv = virtual_heads(Hq, Hkv, Nq);
  int w = num_splits > 0 ? num_splits : default_workers(kv8);
  if (w > kMaxWorkers) w = kMaxWorkers;
  const int per_head = w / hv > 0 ? w / hv : 1;
  return per_head * hv;
}

int check_decode_shape(int dtype, int B, int Hq, int Hkv, int Nq, int d, int max_seq_len,
                       int num_splits) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Nq < 0 || max_seq_len < 0 || num_splits < 0)
    return ATTN_EINVAL;
  if (Hq % Hkv != 0) return ATTN_EINVAL;
  if (dtype != ATTN_BF16) return ATTN_EUNSUPPORTED;
  if (!head_dim_ok(d)) return ATTN_EUNSUPPORTED;
  if ((long long)(Hq / Hkv) * Nq > kMaxRows) return ATTN_EUNSUPPORTED;
  // one 16-token stretch of a head is addressed with 32-bit byte offsets
  if ((long long)16 * Hkv * d * 2 > 0x7fffffffLL) return ATTN_EUNSUPPORTED;
  return ATTN_OK;
}

struct WorkspaceLayout {
  size_t part_lse_off, prefix_off, total;
};

// [pieces * MP * d f32 partial O][pieces * MP f32 partial LSE][(B+1) int64 prefix],
// MP = min(G*Nq, 16) rows per piece, pieces = workers + B*HV with HV the
// (K/V head, row group) pairs and workers a multiple of HV; each part
// 256-byte aligned
WorkspaceLayout workspace_layout(int B, int Hq, int Hkv, int Nq, int d, int workers) {
  const long long rows = decode_rows(Hq, Hkv, Nq);
  const long long M = rows < 16 ? rows : 16;
  const long long pieces = (long long)workers + (long long)B * virtual_heads(Hq, Hkv, Nq);
  auto up = [](long long x) { return (x + 255) / 256 * 256; };
  WorkspaceLayout l;
  const long long o_bytes = up(pieces * M * d * 4);
  const long long lse_bytes = up(pieces * M * 4);
  l.part_lse_off = (size_t)o_bytes;
  l.prefix_off = (size_t)(o_bytes + lse_bytes);
  l.total = (size_t)(o_bytes + lse_bytes + ((long long)B + 1) * 8);
  return l;
}

}  // namespace

extern "C" {

const char* attn_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_EINVAL: return "invalid argument";
    case ATTN_EUNSUPPORTED: return "unsupported dtype, head dim or group size";
    case ATTN_EWORKSPACE: return "workspace missing or too small";
    case ATTN_EHIP: return "HIP runtime error at launch";
    case ATTN_ENOSPACE: return "not enough free blocks in the pool";
    default: return "unknown status";
  }
}

int attn_prefill(const void* q, const void* k, const void* v, void* o, float* lse, int dtype,
                 int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                 int q_offset, void* stream) {
  return attn_prefill_waves(q, k, v, o, lse, dtype, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                            q_offset, 0, stream);
}

int attn_prefill_workgroup_waves(int dtype, int B, int Hq, int Hkv, int Nq, int causal) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Nq < 0 || Hq % Hkv != 0) return ATTN_EINVAL;
  if (dtype != ATTN_BF16) return ATTN_EUNSUPPORTED;
  return attn::prefill_bf16_waves(B, Hq, Hkv, Nq, causal != 0, attn::device_compute_units());
}

int attn_prefill_waves(const void* q, const void* k, const void* v, void* o, float* lse,
                       int dtype, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                       int causal, int q_offset, int waves, void* stream) {
  if (waves != 0 && (dtype != ATTN_BF16 || (waves != 4 && waves != 8))) return ATTN_EINVAL;
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Nq < 0 || Nk < 0) return ATTN_EINVAL;
  if (Hq % Hkv != 0) return ATTN_EINVAL;
  if (!std::isfinite(scale) || !(scale > 0.f)) return ATTN_EINVAL;
  if (q_offset > (1 << 30) || q_offset < -(1 << 30)) return ATTN_EINVAL;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_EUNSUPPORTED;
  if (!head_dim_ok(d)) return ATTN_EUNSUPPORTED;
  // one K/V head's rows are addressed with 32-bit byte offsets
  if ((long long)Nk * d * 4 > 0x7fffffffLL) return ATTN_EUNSUPPORTED;
  if (B == 0 || Nq == 0) return ATTN_OK;
  if (q == nullptr || o == nullptr) return ATTN_EINVAL;
  if (Nk > 0 && (k == nullptr || v == nullptr)) return ATTN_EINVAL;
  if (misaligned16(q) || misaligned16(o) || misaligned16(k) || misaligned16(v) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u))
    return ATTN_EINVAL;
  attn::PrefillArgs a{q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal != 0, q_offset};
  a.waves = waves;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return status_of(dtype == ATTN_BF16 ? attn::launch_prefill_bf16(a, s)
                                      : attn::launch_prefill_f32(a, s));
}

static bool backward_sizes_ok(int B, int Hq, int Hkv, int Nq, int Nk, int d, int q_offset) {
  return B >= 0 && Hq > 0 && Hkv > 0 && Nq >= 0 && Nk >= 0 && Hq % Hkv == 0 && head_dim_ok(d) &&
         q_offset <= (1 << 30) && q_offset >= -(1 << 30);
}

size_t attn_prefill_backward_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d,
                                             int causal, int q_offset) {
  if (!backward_sizes_ok(B, Hq, Hkv, Nq, Nk, d, q_offset)) return 0;
  return attn::plan_backward(B, Hq, Hkv, Nq, Nk, d, causal != 0, q_offset,
                             attn::device_compute_units())
      .bytes;
}

int attn_prefill_backward(const void* q, const void* k, const void* v, const void* o,
                          const float* lse, const void* dout, void* dq, void* dk, void* dv,
                          int dtype, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                          int causal, int q_offset, void* workspace, size_t workspace_bytes_given,
                          void* stream) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Nq < 0 || Nk < 0) return ATTN_EINVAL;
  if (Hq % Hkv != 0) return ATTN_EINVAL;
  if (!std::isfinite(scale) || !(scale > 0.f)) return ATTN_EINVAL;
  if (q_offset > (1 << 30) || q_offset < -(1 << 30)) return ATTN_EINVAL;
  if (dtype != ATTN_BF16) return ATTN_EUNSUPPORTED;
  if (!head_dim_ok(d)) return ATTN_EUNSUPPORTED;
  if ((long long)Nk * d * 2 > 0x7fffffffLL || (long long)Nq * d * 2 > 0x7fffffffLL)
    return ATTN_EUNSUPPORTED;
  if (B == 0 || (Nq == 0 && Nk == 0)) return ATTN_OK;
  if (Nq > 0 && (q == nullptr || o == nullptr || lse == nullptr || dout == nullptr ||
                 dq == nullptr))
    return ATTN_EINVAL;
  if (Nk > 0 && (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr))
    return ATTN_EINVAL;
  if (misaligned16(q) || misaligned16(k) || misaligned16(v) || misaligned16(o) ||
      misaligned16(dout) || misaligned16(dq) || misaligned16(dk) || misaligned16(dv) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u))
    return ATTN_EINVAL;
  const attn::BackwardPlan pl = attn::plan_backward(B, Hq, Hkv, Nq, Nk, d, causal != 0, q_offset,
                                                    attn::device_compute_units());
  if (workspace == nullptr || misaligned16(workspace) || workspace_bytes_given < pl.bytes)
    return ATTN_EWORKSPACE;
  attn::BackwardArgs a{q, k, v, o, dout, lse, dq, dk, dv, static_cast<float*>(workspace),
                       reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.lrow_offset),
                       B, Hq, Hkv, Nq, Nk, d, scale, causal != 0, q_offset};
  a.nsplit = pl.nsplit;
  a.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.part_offset);
  return status_of(attn::launch_backward_bf16(a, static_cast<hipStream_t>(stream)));
}

int attn_prefill_paged(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_table, int max_blocks_per_seq, int num_blocks,
                       const int32_t* seq_lens, void* o, float* lse, int dtype, int B, int Hq,
                       int Hkv, int Nq, int d, float scale, int causal, int max_seq_len,
                       void* stream) {
  return attn_prefill_paged_waves(q, k_cache, v_cache, block_table, max_blocks_per_seq,
                                  num_blocks, seq_lens, o, lse, dtype, B, Hq, Hkv, Nq, d, scale,
                                  causal, max_seq_len, 0, stream);
}

int attn_prefill_paged_waves(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_table, int max_blocks_per_seq, int num_blocks,
                             const int32_t* seq_lens, void* o, float* lse, int dtype, int B,
                             int Hq, int Hkv, int Nq, int d, float scale, int causal,
                             int max_seq_len, int waves, void* stream) {
  if (waves != 0 && waves != 4 && waves != 8) return ATTN_EINVAL;
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Nq < 0 || max_seq_len < 0) return ATTN_EINVAL;
  if (Hq % Hkv != 0) return ATTN_EINVAL;
  if (!std::isfinite(scale) || !(scale > 0.f)) return ATTN_EINVAL;
  if (block_table != nullptr && (max_blocks_per_seq <= 0 || num_blocks < 0)) return ATTN_EINVAL;
  if (dtype != ATTN_BF16) return ATTN_EUNSUPPORTED;
  if (!head_dim_ok(d)) return ATTN_EUNSUPPORTED;
  // one 16-token block of a head is addressed with 32-bit byte offsets
  if ((long long)16 * Hkv * d * 2 > 0x7fffffffLL) return ATTN_EUNSUPPORTED;
  if (B == 0 || Nq == 0) return ATTN_OK;
  if (q == nullptr || o == nullptr || seq_lens == nullptr) return ATTN_EINVAL;
  if (max_seq_len > 0 && (k_cache == nullptr || v_cache == nullptr)) return ATTN_EINVAL;
  if (misaligned16(q) || misaligned16(o) || misaligned16(k_cache) || misaligned16(v_cache) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u) ||
      (reinterpret_cast<uintptr_t>(block_table) & 3u))
    return ATTN_EINVAL;
  attn::PrefillArgs a{q, k_cache, v_cache, o, lse, B, Hq, Hkv, Nq, 0, d, scale, causal != 0, 0};
  a.q_token_major = 1;
  a.cache = 1;
  a.block_table = block_table;
  a.max_blocks = block_table ? max_blocks_per_seq : 0;
  a.num_blocks = block_table ? num_blocks : 0;
  a.max_len = max_seq_len;
  a.seq_lens = seq_lens;
  a.waves = waves;
  return status_of(attn::launch_prefill_bf16(a, static_cast<hipStream_t>(stream)));
}

int attn_decode_num_splits(int B, int Hq, int Hkv, int Nq, int d, int max_seq_len,
                           int num_splits) {
  const int st = check_decode_shape(ATTN_BF16, B, Hq, Hkv, Nq, d, max_seq_len, num_splits);
  if (st != ATTN_OK) return st;
  return plan_workers(num_splits, Hq, Hkv, Nq, false);
}

size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int Nq, int d, int max_seq_len,
                                   int num_splits) {
  if (check_decode_shape(ATTN_BF16, B, Hq, Hkv, Nq, d, max_seq_len, num_splits) != ATTN_OK)
    return 0;
  // Sized for the larger of the two cache formats' worker counts, so one
  // workspace serves attn_decode_paged and attn_decode_paged_fp8 alike.
  const size_t a = workspace_layout(B, Hq, Hkv, Nq, d,
                                    plan_workers(num_splits, Hq, Hkv, Nq, false)).total;
  const size_t b = workspace_layout(B, Hq, Hkv, Nq, d,
                                    plan_workers(num_splits, Hq, Hkv, Nq, true)).total;
  return a > b ? a : b;
}

}  // extern "C"

int attn::decode_call(const void* q, const void* k_cache, const void* v_cache, int kv8,
                      const float* k_scale, const float* v_scale, const int32_t* block_table,
                      int max_blocks_per_seq, int num_blocks, const int32_t* seq_lens, void* o,
                      float* lse, int dtype, int B, int Hq, int Hkv, int Nq, int d, float scale,
                      int causal, int max_seq_len, int num_splits, void* workspace,
                      size_t workspace_bytes_given, void* stream, size_t* plan_bytes) {
  const int st = check_decode_shape(dtype, B, Hq, Hkv, Nq, d, max_seq_len, num_splits);
  if (st != ATTN_OK) return st;
  if (!std::isfinite(scale) || !(scale > 0.f)) return ATTN_EINVAL;
  if (block_table != nullptr && (max_blocks_per_seq <= 0 || num_blocks < 0)) return ATTN_EINVAL;
  if (B == 0 || Nq == 0) return ATTN_OK;
  if (q == nullptr || o == nullptr || seq_lens == nullptr) return ATTN_EINVAL;
  if (kv8 && (k_scale == nullptr || v_scale == nullptr ||
              (reinterpret_cast<uintptr_t>(k_scale) & 3u) ||
              (reinterpret_cast<uintptr_t>(v_scale) & 3u)))
    return ATTN_EINVAL;
  if (max_seq_len > 0 && (k_cache == nullptr || v_cache == nullptr)) return ATTN_EINVAL;
  if (misaligned16(q) || misaligned16(o) || misaligned16(k_cache) || misaligned16(v_cache) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u) ||
      (reinterpret_cast<uintptr_t>(block_table) & 3u))
    return ATTN_EINVAL;
  const int workers = plan_workers(num_splits, Hq, Hkv, Nq, kv8 != 0);
  const WorkspaceLayout lay = workspace_layout(B, Hq, Hkv, Nq, d, workers);
  if (plan_bytes != nullptr) {  // validation and sizing only
    *plan_bytes = lay.total;
    return ATTN_OK;
  }
  if (workspace == nullptr || misaligned16(workspace) || workspace_bytes_given < lay.total)
    return ATTN_EWORKSPACE;
  attn::DecodeArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.max_blocks = block_table ? max_blocks_per_seq : 0;
  a.num_blocks = block_table ? num_blocks : 0;
  a.seq_lens = seq_lens;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Nq = Nq;
  a.d = d;
  a.scale = scale;
  a.causal = causal != 0;
  a.max_seq_len = max_seq_len;
  a.workers = workers;
  a.kv8 = kv8;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  char* ws = static_cast<char*>(workspace);
  a.part_o = reinterpret_cast<float*>(ws);
  a.part_lse = reinterpret_cast<float*>(ws + lay.part_lse_off);
  a.prefix = reinterpret_cast<long long*>(ws + lay.prefix_off);
  return status_of(attn::launch_decode_bf16(a, static_cast<hipStream_t>(stream)));
}

extern "C" {

int attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_table, int max_blocks_per_seq, int num_blocks,
                      const int32_t* seq_lens, void* o, float* lse, int dtype, int B, int Hq,
                      int Hkv, int Nq, int d, float scale, int causal, int max_seq_len,
                      int num_splits, void* workspace, size_t workspace_bytes_given,
                      void* stream) {
  return attn::decode_call(q, k_cache, v_cache, 0, nullptr, nullptr, block_table,
                           max_blocks_per_seq, num_blocks, seq_lens, o, lse, dtype, B, Hq, Hkv,
                           Nq, d, scale, causal, max_seq_len, num_splits, workspace,
                           workspace_bytes_given, stream, nullptr);
}

int attn_decode_paged_fp8(const void* q, const void* k_cache, const void* v_cache,
                          const float* k_scale, const float* v_scale,
                          const int32_t* block_table, int max_blocks_per_seq, int num_blocks,
                          const int32_t* seq_lens, void* o, float* lse, int B, int Hq, int Hkv,
                          int Nq, int d, float scale, int causal, int max_seq_len,
                          int num_splits, void* workspace, size_t workspace_bytes_given,
                          void* stream) {
  return attn::decode_call(q, k_cache, v_cache, 1, k_scale, v_scale, block_table,
                           max_blocks_per_seq, num_blocks, seq_lens, o, lse, ATTN_BF16, B, Hq,
                           Hkv, Nq, d, scale, causal, max_seq_len, num_splits, workspace,
                           workspace_bytes_given, stream, nullptr);
}

static int check_copy(const void* a, const void* b, const int32_t* block_table,
                      int max_blocks_per_seq, int num_blocks, const int32_t* lens, int dtype,
                      int B, int Hkv, int n, int d, int max_seq_len) {
  if (B < 0 || Hkv <= 0 || n < 0 || max_seq_len < 0) return ATTN_EINVAL;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_EUNSUPPORTED;
  if (!head_dim_ok(d)) return ATTN_EUNSUPPORTED;
  if (block_table != nullptr && (max_blocks_per_seq <= 0 || num_blocks < 0)) return ATTN_EINVAL;
  if (B == 0 || n == 0) return ATTN_OK;
  if (a == nullptr || b == nullptr || lens == nullptr) return ATTN_EINVAL;
  if (misaligned16(a) || misaligned16(b) || (reinterpret_cast<uintptr_t>(lens) & 3u) ||
      (reinterpret_cast<uintptr_t>(block_table) & 3u))
    return ATTN_EINVAL;
  return 1;  // proceed
}

int kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
              const int32_t* block_table, int max_blocks_per_seq, int num_blocks,
              const int32_t* cache_lens, int dtype, int B, int Hkv, int Nnew, int d,
              int max_seq_len, void* stream) {
  int st = check_copy(k_new, v_new, block_table, max_blocks_per_seq, num_blocks, cache_lens,
                      dtype, B, Hkv, Nnew, d, max_seq_len);
  if (st <= 0) return st;
  if (max_seq_len == 0) return ATTN_OK;  // no position can be written
  if (k_cache == nullptr || v_cache == nullptr || misaligned16(k_cache) || misaligned16(v_cache))
    return ATTN_EINVAL;
  attn::CacheCopyArgs a;
  a.src_k = k_new;
  a.src_v = v_new;
  a.dst_k = k_cache;
  a.dst_v = v_cache;
  a.block_table = block_table;
  a.max_blocks = block_table ? max_blocks_per_seq : 0;
  a.num_blocks = block_table ? num_blocks : 0;
  a.lens = cache_lens;
  a.elem_bytes = dtype == ATTN_BF16 ? 2 : 4;
  a.B = B;
  a.Hkv = Hkv;
  a.Nnew = Nnew;
  a.d = d;
  a.max_seq_len = max_seq_len;
  return status_of(attn::launch_kv_append(a, static_cast<hipStream_t>(stream)));
}

int kv_append_fp8(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                  const float* k_scale, const float* v_scale, const int32_t* block_table,
                  int max_blocks_per_seq, int num_blocks, const int32_t* cache_lens, int B,
                  int Hkv, int Nnew, int d, int max_seq_len, void* stream) {
  int st = check_copy(k_new, v_new, block_table, max_blocks_per_seq, num_blocks, cache_lens,
                      ATTN_BF16, B, Hkv, Nnew, d, max_seq_len);
  if (st <= 0) return st;
  if (k_scale == nullptr || v_scale == nullptr || (reinterpret_cast<uintptr_t>(k_scale) & 3u) ||
      (reinterpret_cast<uintptr_t>(v_scale) & 3u))
    return ATTN_EINVAL;
  if (max_seq_len == 0) return ATTN_OK;  // no position can be written
  if (k_cache == nullptr || v_cache == nullptr || misaligned16(k_cache) || misaligned16(v_cache))
    return ATTN_EINVAL;
  attn::CacheCopyArgs a;
  a.src_k = k_new;
  a.src_v = v_new;
  a.dst_k = k_cache;
  a.dst_v = v_cache;
  a.block_table = block_table;
  a.max_blocks = block_table ? max_blocks_per_seq : 0;
  a.num_blocks = block_table ? num_blocks : 0;
  a.lens = cache_lens;
  a.elem_bytes = 2;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.B = B;
  a.Hkv = Hkv;
  a.Nnew = Nnew;
  a.d = d;
  a.max_seq_len = max_seq_len;
  return status_of(attn::launch_kv_append_fp8(a, static_cast<hipStream_t>(stream)));
}

int attn_gather_paged(const void* cache, const int32_t* block_table, int max_blocks_per_seq,
                      int num_blocks, const int32_t* seq_lens, void* out, int dtype, int B,
                      int Hkv, int d, int max_seq_len, void* stream) {
  int st = check_copy(cache, out, block_table, max_blocks_per_seq, num_blocks, seq_lens, dtype,
                      B, Hkv, max_seq_len, d, max_seq_len);
  if (st <= 0) return st;
  attn::CacheCopyArgs a;
  a.src_k = cache;
  a.src_v = nullptr;
  a.dst_k = out;
  a.dst_v = nullptr;
  a.block_table = block_table;
  a.max_blocks = block_table ? max_blocks_per_seq : 0;
  a.num_blocks = block_table ? num_blocks : 0;
  a.lens = seq_lens;
  a.elem_bytes = dtype == ATTN_BF16 ? 2 : 4;
  a.B = B;
  a.Hkv = Hkv;
  a.Nnew = 0;
  a.d = d;
  a.max_seq_len = max_seq_len;
  return status_of(attn::launch_gather(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
