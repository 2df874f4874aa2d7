/*
 * attn.h — C ABI of libattn.so: exact tiled attention for AMD MI355X (gfx950).
 *
 * What it computes. O = softmax(scale · Q Kᵀ + mask) V for every query row,
 * exactly (no approximation), tile by tile with a running maximum and running
 * sum per row, so the score matrix never exists in device memory:
 *   - "Phase 07 · 12: KV cache, Flash Attention and inference optimisation"
 *     (AI Engineering from Scratch), section "tiling trick" (standard
 *     attention S = Q Kᵀ, P = softmax(S), O = P V, and the tiled loop that
 *     writes each output tile once) and "Build it, step 2" (running max/sum);
 *   - "大模型面试笔记——Attention篇" (juejin), §2 (online safe softmax, one fused
 *     kernel) and §4 (the 1/√h scaling, here the explicit `scale`);
 *   - "[BEE-30062] FlashAttention 與高效注意力核心", Background (Flash-Decoding:
 *     split K/V along the sequence, reduce the partial softmax results
 *     stably) and section "為長上下文推論啟用 FlashDecoding" (the decode cache
 *     layout and per-sequence lengths);
 *   - "Effizienz" (tokenwerk), sections "GQA im leicht lesbaren Code" (query
 *     head hq reads K/V head hq / (Hq/Hkv)) and "Der wichtige Maskenfehler
 *     beim Cache" (causal masks carry a position offset when the query is
 *     shorter than the keys).
 *
 * Conventions shared by every entry point.
 *   - Every tensor pointer is a DEVICE pointer, owned by the caller; all
 *     tensors are dense and row-major in the layouts stated below. The
 *     library never allocates, frees or synchronises device memory.
 *   - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *     on it and the call returns without waiting.
 *   - Scalars and pointers are validated on the host before anything is
 *     enqueued; on error the call returns a negative attn_status and enqueues
 *     nothing. Device-resident integers (seq_lens, cache_lens, block tables)
 *     are not read on the host; the kernels clamp them (stated per call) so
 *     that no access leaves the buffers the sizes describe.
 *   - Outputs O have the dtype of Q; LSE is always f32, natural log, in
 *     scaled-score units: LSE_i = ln Σ_{visible j} exp(scale · q_i·k_j).
 *     A row that sees no key gets O = 0 and LSE = -inf.
 *   - Kernels use no atomics: results are bitwise reproducible run to run.
 *   - The library is stateless and re-entrant, with one exception:
 *     attn_decode_paged_noalloc keeps its scratch in a device array of its
 *     own (one per GPU) and the array's address per device.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_status {
  ATTN_OK = 0,
  ATTN_EINVAL = -1,       /* bad argument: null pointer, negative size, Hq % Hkv != 0 */
  ATTN_EUNSUPPORTED = -2, /* valid but not built: dtype, head dim, group size */
  ATTN_EWORKSPACE = -3,   /* workspace NULL or smaller than attn_decode_workspace_bytes() */
  ATTN_EHIP = -4,         /* the HIP runtime reported an error at launch */
  ATTN_ENOSPACE = -5      /* block pool: not enough free blocks (nothing changed) */
} attn_status;

typedef enum attn_dtype { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype;

/* Tokens per physical block of a paged cache ("Phase 07 · 12", section
 * "Paged attention": the cache is cut into 16-token blocks). */
#define ATTN_BLOCK_TOKENS 16

/*
 * Prefill over whole prompts.
 *   q, o : [B, Hq, Nq, d]   (batch, heads, seq, head_dim — the layout of the
 *                            SDPA call on "[BEE-30062]")
 *   k, v : [B, Hkv, Nk, d]
 *   lse  : [B, Hq, Nq] f32, or NULL to skip it
 * Query head hq uses K/V head hq / (Hq/Hkv). Row i of every head sits at
 * position i + q_offset; with causal != 0 it sees key j iff j <= i + q_offset
 * (q_offset = Nk - Nq aligns the last query with the last key; 0 is the usual
 * square prefill). Without causal every row sees all Nk keys.
 * Supported: dtype ATTN_BF16 (bf16 inputs, fp32 accumulation, MFMA) and
 * ATTN_F32 (fp32 throughout), d in {64, 128}. Nq, Nk, B may be 0.
 * |q_offset| <= 2^30.
 */
int attn_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
                 int dtype, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                 float scale, int causal, int q_offset, void* stream);

/*
 * Chunked prefill against a K/V cache: the Nq new tokens of each sequence
 * attend to every cached key, including their own rows, which kv_append has
 * already written ("Phase 07 · 12", section "Paged attention": reusing the
 * cached K/V of a shared prefix; the new chunk's rows follow the cached ones,
 * so its causal mask is offset by the cached length, "Effizienz", "Der
 * wichtige Maskenfehler beim Cache"). Same arguments and cache layouts as
 * attn_decode_paged, for any Nq (the tiled MFMA path of attn_prefill; no
 * workspace):
 *   q, o        : [B, Nq, Hq, d] bf16
 *   lse         : [B, Hq, Nq] f32, or NULL to skip it
 *   paged cache : block_table != NULL; k_cache, v_cache are pools
 *                 [num_blocks, 16, Hkv, d], block_table [B, max_blocks_per_seq]
 *                 int32, token t of sequence b in block block_table[b][t / 16],
 *                 slot t % 16
 *   contiguous  : block_table == NULL; k_cache, v_cache are
 *                 [B, max_seq_len, Hkv, d]
 *   seq_lens    : [B] int32, keys of sequence b including its Nq new ones;
 *                 clamped to [0, max_seq_len] (and max_blocks_per_seq·16 when
 *                 paged). Query row i of sequence b sits at position
 *                 seq_lens[b] - Nq + i; with causal it sees keys j <= that
 *                 position, without causal all seq_lens[b] keys. Rows before
 *                 position 0 see no key (O = 0, LSE = -inf). Table entries
 *                 outside [0, num_blocks) make their 16 keys invisible.
 * Supported: dtype ATTN_BF16, d in {64, 128}, 16·Hkv·d·2 < 2^31.
 */
int attn_prefill_paged(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_table, int max_blocks_per_seq, int num_blocks,
                       const int32_t* seq_lens, void* o, float* lse,
                       int dtype, int B, int Hq, int Hkv, int Nq, int d,
                       float scale, int causal, int max_seq_len, void* stream);

/*
 * Decode of Nq new tokens per sequence against a K/V cache, split along the
 * key sequence (Flash-Decoding, "[BEE-30062]" Background) and merged with a
 * log-sum-exp combine.
 *   q, o        : [B, Nq, Hq, d]  ("[BEE-30062]", "為長上下文推論啟用
 *                                   FlashDecoding": (batch, 1, n_heads, head_dim))
 *   lse         : [B, Hq, Nq] f32, or NULL to skip it
 *   paged cache : block_table != NULL. k_cache, v_cache are pools
 *                 [num_blocks, 16, Hkv, d]; block_table is
 *                 [B, max_blocks_per_seq] int32; logical token t of sequence b
 *                 lives in block block_table[b][t / 16], slot t % 16.
 *   contiguous  : block_table == NULL. k_cache, v_cache are
 *                 [B, max_seq_len, Hkv, d] (max_blocks_per_seq, num_blocks
 *                 are ignored).
 *   seq_lens    : [B] int32, visible keys of sequence b INCLUDING the Nq new
 *                 tokens (already appended with kv_append). Query row i of
 *                 sequence b sits at position seq_lens[b] - Nq + i; with
 *                 causal it sees keys j <= that position ("Effizienz",
 *                 "Der wichtige Maskenfehler beim Cache"), without causal all
 *                 seq_lens[b] keys.
 *   max_seq_len : an upper bound of seq_lens. Device-side, seq_lens[b] is
 *                 clamped to [0, max_seq_len] (and to max_blocks_per_seq·16
 *                 when paged). Table entries outside [0, num_blocks) make
 *                 their 16 keys invisible.
 *   num_splits  : number of workers (GPU waves) that share the keys, rounded
 *                 down to a multiple of Hkv (at least Hkv). Each K/V head gets
 *                 num_splits/Hkv workers; the head's 32-key steps of all
 *                 sequences are laid end to end and cut into that many equal
 *                 ranges, so the split adapts to ragged lengths. 0 picks a
 *                 default for the current device: one worker per SIMD (four
 *                 per compute unit), for either cache format.
 *   workspace   : device scratch of at least attn_decode_workspace_bytes()
 *                 bytes for the same arguments, owned by the caller and
 *                 free again once the call's work on `stream` is done. It
 *                 holds the partial output and LSE of every piece (one per
 *                 worker and sequence it touches, at most
 *                 workers + B·Hkv of them) and a [B + 1] int64 prefix sum
 *                 of per-sequence step counts, all written before they are
 *                 read, so it needs no clearing. Calls that share one
 *                 workspace must be ordered on one stream.
 * Supported: dtype ATTN_BF16, d in {64, 128}, (Hq/Hkv)·Nq <= 64.
 */
int attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_table, int max_blocks_per_seq, int num_blocks,
                      const int32_t* seq_lens, void* o, float* lse,
                      int dtype, int B, int Hq, int Hkv, int Nq, int d,
                      float scale, int causal, int max_seq_len, int num_splits,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_paged over an fp8 K/V cache: the cache holds E4M3 codes (OCP
 * 8-bit floating point, "fn" variant: bias 7, no infinities, largest 448),
 * one byte per element, in the same paged or contiguous layouts; element x of
 * K/V head h stands for decode(code) · scale[h] ("Phase 07 · 12", section
 * "Paged attention": the fp8 cache option, which halves the bytes decode
 * reads). The scores are scale · q·k with those values; O and LSE as for
 * attn_decode_paged.
 *   k_scale, v_scale : [Hkv] f32 device arrays, finite and > 0
 *   q, o             : [B, Nq, Hq, d] bf16; everything else as attn_decode_paged
 *                      (its workspace size applies unchanged)
 */
int attn_decode_paged_fp8(const void* q, const void* k_cache, const void* v_cache,
                          const float* k_scale, const float* v_scale,
                          const int32_t* block_table, int max_blocks_per_seq, int num_blocks,
                          const int32_t* seq_lens, void* o, float* lse,
                          int B, int Hq, int Hkv, int Nq, int d,
                          float scale, int causal, int max_seq_len, int num_splits,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_paged without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The partial results live in a
 * library-owned device array of ATTN_DECODE_NOALLOC_SCRATCH_BYTES bytes, one
 * per GPU, held from the first call on that GPU until the process ends; the
 * call allocates and frees nothing. Arguments, layouts, results and errors as
 * attn_decode_paged (same kernels, same bits), except: a call whose
 * attn_decode_workspace_bytes() exceeds the array returns ATTN_EWORKSPACE
 * and enqueues nothing. At d = 128, Hkv = 8 and the default 1024 workers of
 * a 256-CU device the 32 MiB hold up to 1903 sequences with 4 query rows per
 * K/V head, 379 with 16, 190 with 32 and 95 with 64.
 * Every call on one GPU shares that GPU's array, and everything in it is
 * written before it is read within a call: calls that may overlap on one GPU
 * (other streams, other host threads) race and must be ordered by the
 * caller.
 */
#define ATTN_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, int max_blocks_per_seq, int num_blocks,
                              const int32_t* seq_lens, void* o, float* lse,
                              int dtype, int B, int Hq, int Hkv, int Nq, int d,
                              float scale, int causal, int max_seq_len, int num_splits,
                              void* stream);

/* Worker count attn_decode_paged uses for these arguments (num_splits = 0:
 * the default for the current device), or a negative attn_status. */
int attn_decode_num_splits(int B, int Hq, int Hkv, int Nq, int d, int max_seq_len,
                           int num_splits);

/* Workspace bytes attn_decode_paged and attn_decode_paged_fp8 need for these
 * arguments (the larger of the two when their default worker counts differ);
 * 0 if they are invalid. */
size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int Nq, int d, int max_seq_len,
                                   int num_splits);

/*
 * Backward pass of attn_prefill ("Phase 07 · 12", section "tiling trick": the
 * backward pass recomputes the forward's intermediate values from the inputs
 * instead of storing them). Given dout = dLoss/dO it returns
 *     dq = scale · dS K,  dk = scale · dSᵀ Q,  dv = Pᵀ dout,
 * with P the forward's probabilities, dS = P ∘ (dout Vᵀ − D) and
 * D_i = dout_i · o_i; under GQA, dk and dv of a K/V head are summed over the
 * Hq/Hkv query heads that read it. P is recomputed tile by tile from q, k and
 * the forward's lse (exp(scale·q·k − lse)); no score matrix is stored.
 *   q, o, dout, dq : [B, Hq, Nq, d] bf16   (o and lse exactly as attn_prefill
 *   k, v, dk, dv   : [B, Hkv, Nk, d] bf16   returned them for these inputs)
 *   lse            : [B, Hq, Nq] f32
 *   causal, q_offset, scale : as for attn_prefill
 *   workspace      : device scratch of at least
 *                    attn_prefill_backward_workspace_bytes() bytes for the
 *                    same sizes (it receives D and, when the dK/dV work of a
 *                    group is shared by several workgroups, their fp32
 *                    partial sums); calls that share one must be ordered on
 *                    one stream. It needs no clearing.
 * Every element of dq, dk and dv is written (keys no row sees get 0).
 * Supported: dtype ATTN_BF16 (fp32 accumulation), d in {64, 128}.
 */
int attn_prefill_backward(const void* q, const void* k, const void* v, const void* o,
                          const float* lse, const void* dout, void* dq, void* dk, void* dv,
                          int dtype, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                          int causal, int q_offset, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Workspace bytes attn_prefill_backward needs for these arguments on the
 * current device; 0 if they are invalid. */
size_t attn_prefill_backward_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d,
                                             int causal, int q_offset);

/*
 * Append Nnew new K/V rows per sequence to the cache (the decode step grows
 * the cache by concatenation: "大模型面试笔记——Attention篇" §4; "Phase 07 ·
 * 12", "Build it, step 1").
 *   k_new, v_new : [B, Nnew, Hkv, d]
 *   k_cache, v_cache, block_table, max_blocks_per_seq, num_blocks,
 *   max_seq_len  : as for attn_decode_paged (block_table NULL = contiguous).
 *   cache_lens   : [B] int32, lengths BEFORE the append. Row r of sequence b
 *                  goes to logical position cache_lens[b] + r.
 * The caller owns block allocation: the table must already cover positions
 * < cache_lens[b] + Nnew; lengths are not updated here (after the call the
 * caller uses seq_lens = cache_lens + Nnew). A row whose position is negative,
 * at or beyond max_seq_len, beyond the table, or in a block outside
 * [0, num_blocks) is not written. The copy is bit-exact.
 * Supported: dtype ATTN_BF16 or ATTN_F32, d in {64, 128}.
 */
int kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
              const int32_t* block_table, int max_blocks_per_seq, int num_blocks,
              const int32_t* cache_lens, int dtype, int B, int Hkv, int Nnew, int d,
              int max_seq_len, void* stream);

/*
 * kv_append into an fp8 (E4M3) cache: k_new, v_new are bf16 [B, Nnew, Hkv, d];
 * element x of head h is stored as the code nearest to x / scale[h] (one fp32
 * division; ties to even), with magnitudes past 448 saturating to ±448.
 * Layouts, positions and the caller's duties as for kv_append; k_scale,
 * v_scale are [Hkv] f32 device arrays (the ones attn_decode_paged_fp8 reads).
 */
int kv_append_fp8(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                  const float* k_scale, const float* v_scale,
                  const int32_t* block_table, int max_blocks_per_seq, int num_blocks,
                  const int32_t* cache_lens, int B, int Hkv, int Nnew, int d,
                  int max_seq_len, void* stream);

/*
 * Workgroup width of the bf16 prefill kernel (attn_prefill and
 * attn_prefill_paged) for a launch of this shape on the current device: 8
 * waves when the launch gives at least one such workgroup per compute unit
 * (two under a causal mask), else 4. Returns 4 or 8, or a negative
 * attn_status (dtype other than ATTN_BF16: ATTN_EUNSUPPORTED). Host only.
 */
int attn_prefill_workgroup_waves(int dtype, int B, int Hq, int Hkv, int Nq, int causal);

/*
 * Test helpers: attn_prefill and attn_prefill_paged with the bf16 kernel's
 * workgroup width forced (`waves` 4 or 8; 0 = the choice above), so that
 * both kernel widths can be checked on any shape. Same arguments, results
 * and errors as the calls they extend; a non-zero `waves` with dtype other
 * than ATTN_BF16, or other than 4 or 8, is ATTN_EINVAL. The width changes
 * only how rows are grouped into workgroups, never the result's definition.
 */
int attn_prefill_waves(const void* q, const void* k, const void* v, void* o, float* lse,
                       int dtype, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                       float scale, int causal, int q_offset, int waves, void* stream);
int attn_prefill_paged_waves(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_table, int max_blocks_per_seq,
                             int num_blocks, const int32_t* seq_lens, void* o, float* lse,
                             int dtype, int B, int Hq, int Hkv, int Nq, int d, float scale,
                             int causal, int max_seq_len, int waves, void* stream);

/*
 * Gather the first seq_lens[b] logical rows of every sequence out of a paged
 * (or, with block_table NULL, contiguous) cache into out [B, max_seq_len,
 * Hkv, d], using the same address computation as attn_decode_paged. Rows at
 * or beyond the clamped length are left untouched; keys in invalid blocks are
 * not copied. Exists so tests can check the page-table walk bit for bit.
 */
int attn_gather_paged(const void* cache, const int32_t* block_table, int max_blocks_per_seq,
                      int num_blocks, const int32_t* seq_lens, void* out, int dtype, int B,
                      int Hkv, int d, int max_seq_len, void* stream);

/*
 * Block pool of a paged cache ("Phase 07 · 12", sections "Paged attention"
 * and "Exercises": fixed 16-token blocks behind a page table, returned to the
 * pool as soon as a sequence finishes). HOST-side bookkeeping only: it decides
 * which physical block of a [num_blocks, 16, Hkv, d] pool backs each logical
 * block of a sequence, writing block ids into a HOST copy of that sequence's
 * block-table row (int32, -1 = no block); the caller copies the table to the
 * device before the kernels read it. The pool's state lives in `pool`, a
 * caller-owned host buffer of attn_block_pool_bytes(num_blocks) bytes, 4-byte
 * aligned; the library allocates nothing. A fresh pool hands out blocks
 * 0, 1, 2, ... in order; released blocks are reused last-freed first. Not
 * thread-safe: calls on one pool must be serialised by the caller.
 */
size_t attn_block_pool_bytes(int num_blocks);

/* Set up a pool of num_blocks free blocks in `pool` (pool_bytes at least
 * attn_block_pool_bytes(num_blocks), else ATTN_EWORKSPACE). */
int attn_block_pool_init(void* pool, size_t pool_bytes, int num_blocks);

/* Free blocks left, or ATTN_EINVAL for a buffer that holds no pool. */
int attn_block_pool_free_count(const void* pool);

/* Give a sequence growing from cur_len to new_len tokens storage: the logical
 * blocks [ceil(cur_len/16), ceil(new_len/16)) of table_row (which must be -1
 * there, else ATTN_EINVAL) receive fresh blocks. All or nothing: with too few
 * free blocks it returns ATTN_ENOSPACE and changes nothing.
 * ceil(new_len/16) must not exceed max_blocks_per_seq. */
int attn_block_pool_grow(void* pool, int32_t* table_row, int max_blocks_per_seq, int cur_len,
                         int new_len);

/* Free-on-finish: return the ceil(len/16) blocks of a finished sequence to
 * the pool and set those entries of table_row to -1. Every entry must name a
 * block this pool handed out and that is not yet released (each at most once),
 * else ATTN_EINVAL and nothing changes. */
int attn_block_pool_release(void* pool, int32_t* table_row, int max_blocks_per_seq, int len);

/* A static string naming a status code. */
const char* attn_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
