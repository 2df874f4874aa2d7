// Host-side pool of the paged cache's physical 16-token blocks.
//
// "Phase 07 · 12: KV cache, Flash Attention and inference optimisation",
// sections "Paged attention" (the cache is cut into 16-token blocks and a page
// table maps a sequence's logical positions to physical blocks) and
// "Exercises" (a toy paged cache whose blocks go back to the pool as soon as a
// sequence finishes). The pool decides which physical block backs each
// logical block of a sequence; the kernels only ever read the resulting
// table.
//
// State, all in one caller-owned host buffer (attn_block_pool_bytes):
//   Header | int32 free[num_blocks] | uint8 owned[num_blocks]
// `free` is a stack of free block ids (top at free[free_count - 1]); a fresh
// pool pops 0, 1, 2, ... in order. `owned[e]` is 1 while block e belongs to
// some sequence, which lets release() refuse a double free or a foreign id
// before it changes anything.
#include <stdint.h>
#include <string.h>

#include "attn.h"

namespace {

constexpr uint32_t kMagic = 0x4b56504cu;  // "KVPL"

struct Header {
  uint32_t magic;
  int32_t num_blocks;
  int32_t free_count;
  int32_t reserved;
};

size_t pool_bytes(int num_blocks) {
  return sizeof(Header) + (size_t)num_blocks * sizeof(int32_t) + (size_t)num_blocks;
}

Header* header(void* pool) { return static_cast<Header*>(pool); }
int32_t* free_stack(void* pool) {
  return reinterpret_cast<int32_t*>(static_cast<char*>(pool) + sizeof(Header));
}
uint8_t* owned(void* pool) {
  Header* h = header(pool);
  return reinterpret_cast<uint8_t*>(static_cast<char*>(pool) + sizeof(Header) +
                                    (size_t)h->num_blocks * sizeof(int32_t));
}

bool valid_pool(const void* pool) {
  if (pool == nullptr || (reinterpret_cast<uintptr_t>(pool) & 3u)) return false;
  const Header* h = static_cast<const Header*>(pool);
  return h->magic == kMagic && h->num_blocks >= 0 && h->free_count >= 0 &&
         h->free_count <= h->num_blocks;
}

// logical blocks that hold positions [0, len)
long long blocks_for(long long len) { return (len + ATTN_BLOCK_TOKENS - 1) / ATTN_BLOCK_TOKENS; }

}  // namespace

extern "C" {

size_t attn_block_pool_bytes(int num_blocks) {
  return num_blocks < 0 ? 0 : pool_bytes(num_blocks);
}

int attn_block_pool_init(void* pool, size_t pool_bytes_given, int num_blocks) {
  if (pool == nullptr || num_blocks < 0 || (reinterpret_cast<uintptr_t>(pool) & 3u))
    return ATTN_EINVAL;
  if (pool_bytes_given < pool_bytes(num_blocks)) return ATTN_EWORKSPACE;
  Header* h = header(pool);
  h->magic = kMagic;
  h->num_blocks = num_blocks;
  h->free_count = num_blocks;
  h->reserved = 0;
  int32_t* st = free_stack(pool);
  for (int i = 0; i < num_blocks; ++i) st[i] = num_blocks - 1 - i;  // pops 0, 1, 2, ...
  memset(owned(pool), 0, (size_t)num_blocks);
  return ATTN_OK;
}

int attn_block_pool_free_count(const void* pool) {
  if (!valid_pool(pool)) return ATTN_EINVAL;
  return static_cast<const Header*>(pool)->free_count;
}

int attn_block_pool_grow(void* pool, int32_t* table_row, int max_blocks_per_seq, int cur_len,
                         int new_len) {
  if (!valid_pool(pool) || table_row == nullptr || max_blocks_per_seq < 0 || cur_len < 0 ||
      new_len < cur_len)
    return ATTN_EINVAL;
  const long long first = blocks_for(cur_len);
  const long long last = blocks_for(new_len);  // logical blocks [first, last) need storage
  if (last > max_blocks_per_seq) return ATTN_EINVAL;
  for (long long j = first; j < last; ++j)
    if (table_row[j] != -1) return ATTN_EINVAL;  // would overwrite (and leak) a block
  Header* h = header(pool);
  if (last - first > h->free_count) return ATTN_ENOSPACE;
  int32_t* st = free_stack(pool);
  uint8_t* own = owned(pool);
  for (long long j = first; j < last; ++j) {
    const int32_t e = st[--h->free_count];
    own[e] = 1;
    table_row[j] = e;
  }
  return ATTN_OK;
}

int attn_block_pool_release(void* pool, int32_t* table_row, int max_blocks_per_seq, int len) {
  if (!valid_pool(pool) || table_row == nullptr || max_blocks_per_seq < 0 || len < 0)
    return ATTN_EINVAL;
  const long long n = blocks_for(len);
  if (n > max_blocks_per_seq) return ATTN_EINVAL;
  Header* h = header(pool);
  uint8_t* own = owned(pool);
  // validate first (ids in range, owned, no id twice in the row), then apply
  long long j = 0;
  for (; j < n; ++j) {
    const int32_t e = table_row[j];
    if (e < 0 || e >= h->num_blocks || own[e] != 1) break;
    own[e] = 2;
  }
  for (long long i = 0; i < j; ++i) own[table_row[i]] = 1;
  if (j < n) return ATTN_EINVAL;
  // push the last logical block first, so the sequence's first block ends on
  // top: an equal-length grow right after gets the same blocks in order
  int32_t* st = free_stack(pool);
  for (long long i = n - 1; i >= 0; --i) {
    const int32_t e = table_row[i];
    own[e] = 0;
    st[h->free_count++] = e;
    table_row[i] = -1;
  }
  return ATTN_OK;
}

}  // extern "C"
