// Internal host-side launchers (one per kernel family). The C ABI in attn.h
// validates every argument before calling these; they only size grids and
// enqueue on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, Nq, Nk, d;
  float scale;
  int causal;
  int q_offset;
  int q_token_major = 0;  // q, o are [B, Nq, Hq, d] (else [B, Hq, Nq, d])
  // cache != 0: k, v are a token-major cache, [num_blocks, 16, Hkv, d] pools
  // behind block_table or [B, max_len, Hkv, d] when block_table is null;
  // Nk and q_offset then come from seq_lens per sequence
  int cache = 0;
  const int32_t* block_table = nullptr;
  int max_blocks = 0, num_blocks = 0, max_len = 0;
  const int32_t* seq_lens = nullptr;
  int waves = 0;  // bf16 workgroup width: 4 or 8, 0 = prefill_bf16_waves()
};

// Waves per workgroup the bf16 prefill kernel uses for a launch of this
// shape when the caller does not force one (4 or 8).
int prefill_bf16_waves(int B, int Hq, int Hkv, int Nq, int causal, int compute_units);

struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  int max_blocks;
  int num_blocks;
  const int32_t* seq_lens;
  void* o;
  float* lse;
  int B, Hq, Hkv, Nq, d;
  float scale;
  int causal;
  int max_seq_len;
  int kv8 = 0;        // caches hold E4M3 codes with per-K/V-head scales
  const float* k_scale = nullptr;
  const float* v_scale = nullptr;
  int workers;        // waves sharing the key space
  float* part_o;      // [(workers + B*Hkv) * M, d]
  float* part_lse;    // [(workers + B*Hkv) * M]
  long long* prefix;  // [B + 1]
};

struct CacheCopyArgs {
  const void* src_k;  // append: new rows; gather: the cache
  const void* src_v;  // append only
  void* dst_k;        // append: the cache; gather: out
  void* dst_v;        // append only
  const int32_t* block_table;
  int max_blocks;
  int num_blocks;
  const int32_t* lens;  // append: cache_lens; gather: seq_lens
  int elem_bytes;
  // append only: the cache holds E4M3 codes of x / scale[kv head]
  const float* k_scale = nullptr;
  const float* v_scale = nullptr;
  int B, Hkv, Nnew, d;
  int max_seq_len;
};

struct BackwardArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* drow;  // workspace: [B, Hq, Nq] f32, D of every row
  float* lrow;  // workspace: [B, Hq, Nq] f32, base-2 LSE of every row
  int B, Hq, Hkv, Nq, Nk, d;
  float scale;
  int causal;
  int q_offset;
  int nsplit = 1;        // dK/dV workgroups per (key block, K/V head)
  float* part = nullptr;  // nsplit > 1: workspace for the fp32 partial sums
};

// How the backward splits its dK/dV work and lays out its workspace (D, then
// the partial sums when nsplit > 1).
struct BackwardPlan {
  int nsplit = 1;
  size_t lrow_offset = 256;
  size_t part_offset = 512;
  size_t bytes = 512;
};
BackwardPlan plan_backward(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                           int q_offset, int compute_units);

// Compute units of the current device (cached per device; 256 when none can
// be queried).
int device_compute_units();

// attn_decode_paged / attn_decode_paged_fp8 (kv8 != 0) after argument
// validation. With plan_bytes != nullptr the call only validates its
// arguments (the workspace aside) and stores the workspace bytes it needs,
// launching nothing; a call with nothing to do (B or Nq zero) returns ATTN_OK
// and leaves *plan_bytes untouched.
int decode_call(const void* q, const void* k_cache, const void* v_cache, int kv8,
                const float* k_scale, const float* v_scale, const int32_t* block_table,
                int max_blocks_per_seq, int num_blocks, const int32_t* seq_lens, void* o,
                float* lse, int dtype, int B, int Hq, int Hkv, int Nq, int d, float scale,
                int causal, int max_seq_len, int num_splits, void* workspace,
                size_t workspace_bytes, void* stream, size_t* plan_bytes);

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s);
hipError_t launch_backward_bf16(const BackwardArgs& a, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s);
hipError_t launch_kv_append(const CacheCopyArgs& a, hipStream_t s);
hipError_t launch_kv_append_fp8(const CacheCopyArgs& a, hipStream_t s);
hipError_t launch_gather(const CacheCopyArgs& a, hipStream_t s);

}  // namespace attn
