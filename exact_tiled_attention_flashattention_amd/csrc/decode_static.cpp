// attn_decode_paged_noalloc: split-KV decode whose partial results live in a
// library-owned device array instead of a caller-provided workspace, for
// callers that cannot allocate device memory (code under HIP graph capture,
// serving loops that forbid hipMalloc). The kernels are the ones
// attn_decode_paged launches; only where their scratch comes from differs.
//
// The array is a file-scope __device__ object: every GPU the library runs on
// holds its own copy, from module load until the process ends. Host code
// must not use the array's name as a device address (it names a host-side
// stand-in); the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "attn.h"
#include "launch.h"

namespace {

constexpr size_t kScratchBytes = ATTN_DECODE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices];  // scratch's device address on each device, once looked up

// The address of `scratch` on the current device.
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return ATTN_EHIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return ATTN_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return ATTN_EHIP;
    }
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" int attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                         const int32_t* block_table, int max_blocks_per_seq,
                                         int num_blocks, const int32_t* seq_lens, void* o,
                                         float* lse, int dtype, int B, int Hq, int Hkv, int Nq,
                                         int d, float scale, int causal, int max_seq_len,
                                         int num_splits, void* stream) {
  size_t need = 0;
  int st = attn::decode_call(q, k_cache, v_cache, 0, nullptr, nullptr, block_table,
                             max_blocks_per_seq, num_blocks, seq_lens, o, lse, dtype, B, Hq, Hkv,
                             Nq, d, scale, causal, max_seq_len, num_splits, nullptr, 0, stream,
                             &need);
  if (st != ATTN_OK) return st;
  if (need == 0) return ATTN_OK;  // nothing to launch
  if (need > kScratchBytes) return ATTN_EWORKSPACE;
  void* ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st != ATTN_OK) return st;
  return attn::decode_call(q, k_cache, v_cache, 0, nullptr, nullptr, block_table,
                           max_blocks_per_seq, num_blocks, seq_lens, o, lse, dtype, B, Hq, Hkv,
                           Nq, d, scale, causal, max_seq_len, num_splits, ws, kScratchBytes,
                           stream, nullptr);
}
