/*
 * pagedkv.h -- C ABI of libpagedkv.so: PagedAttention decode on AMD Instinct MI355X (gfx950).
 *
 * The operation (the pages' statement of the problem):
 *   - The KV cache is a pool of fixed-size blocks, allocated per sequence as it grows and
 *     not contiguous in memory ("vllm-project-vllm -- L2", section 3 Q2; section 9 "Memory
 *     Management").  Here a pool is [num_blocks, block_size, num_kv_heads, head_dim],
 *     row-major, one pool for K and one for V.
 *   - A block table maps (sequence, logical block) to a physical block id; the GPU only reads
 *     it (same page, section 6 "KV Cache Block Tables").  Here it is int32
 *     [num_seqs, max_blocks]; logical token t of sequence b lives in physical block
 *     block_tables[b][t / block_size] at offset t % block_size.
 *   - Decode attends one new query token per sequence over that sequence's whole cache
 *     (same page, section 7: decode reads the full KV cache per layer and is bound by memory
 *     bandwidth).  Query head h reads KV head h / (num_heads / num_kv_heads).
 *   - Blocks are extended every decode step (same page, section 6): paged_kv_write stores the
 *     step's new K/V rows at the slots the allocator handed out (slot = block*block_size +
 *     offset).
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The library allocates
 *     nothing, keeps no pointer after returning and never synchronises the device (the one
 *     exception, the measurement hook pkv_time_next_call, holds two event handles until the
 *     next attention call returns).
 *   - All launches go to `stream` (a hipStream_t; NULL = the null stream) and are
 *     asynchronous.  A decode step is paged_kv_write -> paged_attn_decode ->
 *     (paged_attn_reduce), ordered by the stream.
 *   - Tensors are dense row-major.  Pointers to K/V pools, query, key/value rows, out and
 *     tmp_out must be 16-byte aligned; everything else 4-byte (slot_mapping 8-byte).
 *   - Return value: PKV_OK (0) or a negative pkv_status.  Argument checks happen on the host
 *     before any launch, so an error return means nothing was enqueued.  PKV_ERR_LAUNCH
 *     reports a HIP launch failure.  A fault inside a kernel surfaces at the caller's next
 *     synchronisation.
 *   - Device-resident values (block ids, context lengths, slots) are not read on the host.
 *     Kernels clamp them so that every access stays inside the buffers the sizes describe:
 *     a block id outside [0, num_blocks) or a length beyond the table gives an unspecified
 *     result for that sequence, never an out-of-bounds access (lengths are clamped to
 *     max_context_len by every kernel of a call alike, and table indices to the row, so the
 *     other sequences' results are unaffected).  With the environment variable PKV_CHECK=1 the
 *     library instead copies them to the host (synchronising `stream`), validates them and
 *     returns PKV_ERR_CHECK on a violation.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  FP8_E4M3 is OCP E4M3FN: bias 7, max +-448, NaN = S.1111.111, no inf. */
typedef enum { PKV_F16 = 0, PKV_BF16 = 1, PKV_FP8_E4M3 = 2 } pkv_dtype;

typedef enum {
  PKV_OK = 0,
  PKV_ERR_NULL = -1,       /* a required pointer is NULL */
  PKV_ERR_SHAPE = -2,      /* a size is negative, inconsistent or outside the supported set */
  PKV_ERR_DTYPE = -3,      /* unsupported dtype or dtype combination */
  PKV_ERR_ALIGN = -4,      /* a pointer is not aligned as required */
  PKV_ERR_WORKSPACE = -5,  /* split-K buffers missing */
  PKV_ERR_LAUNCH = -6,     /* the HIP runtime rejected a launch */
  PKV_ERR_CHECK = -7,      /* PKV_CHECK=1 found an invalid device-resident value */
  PKV_ERR_STATE = -8,      /* block manager: sequence id in use, or sequence in the wrong state */
  PKV_ERR_NOT_FOUND = -9,  /* block manager: unknown sequence id */
  PKV_ERR_NO_SPACE = -10,  /* block manager: not enough free blocks */
  PKV_ERR_HOST = -11,      /* a host buffer is not pinned, device-mapped memory of the needed size */
  PKV_ERR_SCRATCH = -12    /* paged_attn_decode_noalloc: the call needs more than the fixed scratch */
} pkv_status;

/* Flags of the attention calls. */
enum {
  /* Some physical blocks are named by several rows of the block table (copy-on-write sharing,
     e.g. a common prefix).  K/V loads then use the default cache policy so that the other
     readers find the shared blocks in the Infinity Cache.  Without it every K/V byte is
     assumed to be read once per call and is loaded non-temporally (faster for private
     blocks; correct either way). */
  PKV_FLAG_SHARED_BLOCKS = 1
};

/*
 * paged_kv_write -- scatter this step's new K and V rows into the block pools.
 *
 * For every i < num_tokens with s = slot_mapping[i] in [0, num_blocks*block_size):
 *   key_cache  [s / block_size][s % block_size][:][:] = conv(key  [i][:][:], k_scale)
 *   value_cache[s / block_size][s % block_size][:][:] = conv(value[i][:][:], v_scale)
 * Negative slots (padding tokens) and slots past the pool are skipped.  No other byte of
 * either pool changes.  Two tokens with the same slot: the result is unspecified.
 *
 *   key, value        [num_tokens, num_kv_heads, head_dim], src_dtype (PKV_F16 | PKV_BF16)
 *   key_cache,
 *   value_cache       [num_blocks, block_size, num_kv_heads, head_dim], cache_dtype
 *   slot_mapping      [num_tokens] int64
 *   cache_dtype       == src_dtype: bit copy.  PKV_FP8_E4M3: each element x becomes the
 *                     E4M3FN code of y = x / scale computed as an IEEE fp32 division, rounded
 *                     to nearest with ties to the even code; |y| >= 448 (and +-inf) saturate
 *                     to +-448; NaN gives the NaN code with the sign of y.
 *   k_scale, v_scale  per-tensor fp32 scales (fp8 cache only; must be finite and > 0)
 *   head_dim          multiple of 8 (16 for an fp8 cache); num_kv_heads >= 1
 *
 * Bit-exact by construction: the same inputs always produce the same pool bytes.
 */
int paged_kv_write(const void* key, const void* value, void* key_cache, void* value_cache,
                   const int64_t* slot_mapping, int num_tokens, int num_blocks, int block_size,
                   int num_kv_heads, int head_dim, int src_dtype, int cache_dtype, float k_scale,
                   float v_scale, void* stream);

/*
 * paged_attn_decode -- one query token per sequence against its paged KV cache.
 *
 * For sequence b < num_seqs, query head h < num_heads, with G = num_heads / num_kv_heads,
 * n = context_lens[b] and K_t, V_t the rows of KV head h / G at logical token t < n:
 *   s_t = scale * k_scale * (q[b][h] . K_t)                 (K_t as stored)
 *   out[b][h] = v_scale * sum_t exp(s_t - max s) V_t / sum_t exp(s_t - max s)
 * n = 0 gives a zero row.  k_scale and v_scale apply to an fp8 cache and must be 1 otherwise.
 * Tokens at positions >= n (stale tail slots, unused table entries) never influence the
 * output, whatever bytes they hold.
 *
 *   out              [num_seqs, num_heads, head_dim], q_dtype.  Written when partition_size == 0.
 *   query            [num_seqs, num_heads, head_dim], q_dtype (PKV_F16 | PKV_BF16)
 *   key_cache,
 *   value_cache      [num_blocks, block_size, num_kv_heads, head_dim], kv_dtype
 *   block_tables     [num_seqs, max_blocks] int32; only entries < ceil(n / block_size) are read
 *   context_lens     [num_seqs] int32
 *   max_context_len  host-side upper bound of every context_lens[b]; sizes the split-K grid
 *   partition_size   0: single pass, the output is written directly.
 *                    > 0: split-K over fixed partitions.  Partition p of sequence b covers
 *                    tokens [p*partition_size, min((p+1)*partition_size, n)).  For every
 *                    p < ceil(n / partition_size) the kernel writes the partial
 *                      max_logits[b][h][p] = m_p = max_t s_t
 *                      exp_sums  [b][h][p] = l_p = sum_t exp(s_t - m_p)
 *                      tmp_out   [b][h][p] = v_scale * sum_t exp(s_t - m_p) V_t / l_p
 *                    Must be a multiple of 16 and of block_size.
 *                    < 0: split-K over a balanced schedule: the batch's 16-token tiles, in
 *                    (sequence, position) order, each sequence's tiles preceded by one extra
 *                    unit for the cost of starting it, are cut into W = -partition_size equal
 *                    contiguous ranges of units (fewer if a range would drop below 8 units),
 *                    one per workgroup, so every workgroup does about the same work whatever
 *                    the length mix.  Each (sequence, range) overlap writes one partial
 *                    (m, l, o as above, over the tokens of that overlap) at slot
 *                    p = range - (range of the sequence's first tile).
 *                    paged_attn_balanced_split() gives the W that fills the device once.
 *                    In both split-K modes the p extent is Pslots =
 *                    paged_attn_partial_slots(max_context_len, partition_size): tmp_out is fp32
 *                    [num_seqs, num_heads, Pslots, head_dim], max_logits and exp_sums fp32
 *                    [num_seqs, num_heads, Pslots].  paged_attn_reduce, called with the same
 *                    partition_size, then forms `out`.
 *   flags            0 or PKV_FLAG_SHARED_BLOCKS (see the flag); any other bit is PKV_ERR_SHAPE.
 *   Supported: head_dim 64 or 128; block_size 16, 32, 64, 128 or 256; num_kv_heads <= 16;
 *   G <= 16; (q, kv) dtypes (F16, F16), (BF16, BF16), (BF16, FP8_E4M3), (F16, FP8_E4M3).
 *   Every context_lens[b] must be <= max_context_len and <= max_blocks * block_size.
 *
 * The result is deterministic: identical inputs give bit-identical outputs, and so does any
 * relabelling of physical blocks that leaves each sequence's logical content unchanged.
 */
int paged_attn_decode(void* out, const void* query, const void* key_cache, const void* value_cache,
                      const int32_t* block_tables, int max_blocks, const int32_t* context_lens,
                      int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
                      int num_blocks, float scale, int q_dtype, int kv_dtype, float k_scale,
                      float v_scale, int max_context_len, int partition_size, float* tmp_out,
                      float* max_logits, float* exp_sums, int flags, void* stream);

/*
 * paged_attn_multi_query -- q_len new query tokens per sequence against its paged KV cache,
 * causal among themselves (scoring k speculative draft tokens in one pass: "vLLM vs vllm",
 * speculative decoding; several new tokens of a sequence at once: "vllm-project-vllm -- L2",
 * chunked prefill in the mechanisms table).
 *
 * The L = q_len new tokens are the last L of the n = context_lens[b] cached tokens (their K/V
 * rows are already in the pools).  New token i < L sits at position n - L + i and attends to
 * the tokens t < n - L + 1 + i, i.e. to itself and everything before it; with no visible
 * token the row is 0.  With L = 1 this is paged_attn_decode.
 *   query  [num_seqs, q_len, num_heads, head_dim]
 *   out    [num_seqs, q_len, num_heads, head_dim] (written when partition_size == 0)
 *   split-K partials as for paged_attn_decode with num_heads' = q_len * num_heads rows per
 *   sequence ([num_seqs, q_len, num_heads, Pslots, ...]); paged_attn_reduce called with
 *   num_heads = q_len * num_heads forms `out`.
 * Every other argument, the supported set and the error behaviour are those of
 * paged_attn_decode, plus 1 <= q_len <= 4096.  Kernels: with G * q_len <= 32 (G = num_heads /
 * num_kv_heads) the (head, new token) pairs of a KV group fill one or two MFMA tiles of a decode
 * wave, which streams the cache once for them; with more pairs a tiled kernel stages 64-token
 * K/V blocks in LDS and scores them against up to 128 pairs per workgroup on the matrix cores
 * (paged_attn_multi_query_split() gives the balanced W that fills the device for it).
 */
int paged_attn_multi_query(void* out, const void* query, const void* key_cache, const void* value_cache,
                           const int32_t* block_tables, int max_blocks, const int32_t* context_lens,
                           int num_seqs, int q_len, int num_heads, int num_kv_heads, int head_dim,
                           int block_size, int num_blocks, float scale, int q_dtype, int kv_dtype,
                           float k_scale, float v_scale, int max_context_len, int partition_size,
                           float* tmp_out, float* max_logits, float* exp_sums, int flags, void* stream);

/*
 * paged_attn_decode_noalloc -- paged_attn_decode followed by paged_attn_reduce in one call that
 * allocates nothing and takes no workspace: for callers that cannot call hipMalloc or own a
 * workspace (code under HIP graph capture, tight serving loops, harnesses that forbid device
 * allocation).  It writes the same `out` as that pair of calls, bit for bit.
 *
 *   partition_size  0: single pass (no partials).  < 0: the balanced split over W =
 *                   -partition_size workgroups (paged_attn_balanced_split()), with the split-K
 *                   partials kept in the library's own fixed device buffer (`scratch`, 32 MiB,
 *                   one per GPU the library runs on, held until the process ends).  > 0 is
 *                   PKV_ERR_SHAPE.
 *   out             [num_seqs, num_heads, head_dim], q_dtype; always written.
 * Scratch need of a balanced call: (num_seqs + Weff - 1) * num_heads * (head_dim + 2) * 4 bytes,
 * Weff = max(1, min(W, num_seqs * (ceil(max_context_len / 16) + 1) / 8)); a call that needs more
 * than 32 MiB returns PKV_ERR_SCRATCH before any launch (e.g. 12.7 MB for 128 sequences x 64
 * heads x head_dim 128 at W = 256).
 * Every call on one GPU shares that GPU's buffer and leaves its partials there: calls that
 * overlap on one GPU (different streams, or other threads) race and give unspecified results;
 * calls ordered on one stream are safe.  The first call on a device looks up the buffer's
 * address (hipGetSymbolAddress) and keeps it; no call allocates, frees or synchronises.
 * PKV_CHECK=1 is not honoured here (checking would copy to host memory).  Every other argument,
 * the supported set and the error behaviour are those of paged_attn_decode.
 */
int paged_attn_decode_noalloc(void* out, const void* query, const void* key_cache, const void* value_cache,
                              const int32_t* block_tables, int max_blocks, const int32_t* context_lens,
                              int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
                              int num_blocks, float scale, int q_dtype, int kv_dtype, float k_scale,
                              float v_scale, int max_context_len, int partition_size, int flags, void* stream);

/*
 * paged_attn_decode_append -- one decode step in one call for 16-bit caches: the step's new
 * token of every sequence is stored in the pool and attended to, as paged_kv_write followed by
 * paged_attn_decode would do (blocks are extended every decode step: "vllm-project-vllm -- L2",
 * section 6 "KV Cache Block Tables"; section 7 on decode).
 *
 * For every b with n = context_lens[b] >= 1 the new token sits at position n - 1: key[b] and
 * value[b] ([num_seqs, num_kv_heads, head_dim], dtype) are stored at slot
 * block_tables[b][(n-1) / block_size] * block_size + (n-1) % block_size of the pools -- the
 * bytes paged_kv_write would store with that slot_mapping -- and the attention over the n
 * tokens (the new one included) is computed exactly as paged_attn_decode computes it, with the
 * same partials and the same bits.  Sequences with n = 0 store nothing and give a zero row.
 * The caller must have made that block private to sequence b (copy-on-write), as for
 * paged_kv_write.
 *   dtype           PKV_F16 or PKV_BF16: the query, the new rows and both pools.
 *   partition_size  < 0 (balanced split): the rows are stored by the decode launch itself (the
 *                   wave that streams the tile of position n - 1 uses the new row in place of
 *                   the pool's and stores it).  >= 0: a scatter launch, then the decode.
 * Every other argument, the supported set and the error behaviour are those of
 * paged_attn_decode (k_scale = v_scale = 1).  An fp8 cache is PKV_ERR_DTYPE (use
 * paged_kv_write and paged_attn_decode).
 */
int paged_attn_decode_append(void* out, const void* query, const void* key, const void* value,
                             void* key_cache, void* value_cache, const int32_t* block_tables, int max_blocks,
                             const int32_t* context_lens, int num_seqs, int num_heads, int num_kv_heads,
                             int head_dim, int block_size, int num_blocks, float scale, int dtype,
                             int max_context_len, int partition_size, float* tmp_out, float* max_logits,
                             float* exp_sums, int flags, void* stream);

/*
 * paged_attn_decode_shared_prefix -- paged_attn_decode for a batch whose rows begin with a
 * common prefix held in shared blocks (copy-on-write sharing for prefix caching:
 * "vllm-project-vllm -- L2", section 9 "Memory Management" and the prefix-caching row of the
 * section 10 "Key Performance Mechanisms" table; "vLLM", its summary of prefix caching across
 * requests with a common prompt prefix).  It computes the same `out` as paged_attn_decode
 * (up to rounding order) but reads the prefix once per group of rows instead of once per row:
 *   1. a prefix pass scores the prefix against every row's queries at once (a dense product on
 *      the matrix cores) and writes one partial per (row, head, prefix partition);
 *   2. the balanced split-K decode streams each row's tokens past the prefix;
 *   3. the log-sum-exp merge of all partials writes `out`.
 *
 *   prefix_len             tokens of the shared prefix: >= 0, a multiple of block_size, and
 *                          prefix_len / block_size <= max_blocks.  The prefix is read through
 *                          row 0's first prefix_len / block_size table entries; every row b
 *                          must name the same blocks in its entries j < ceil(min(n, prefix_len)
 *                          / block_size).  Rows shorter than the prefix see their own n tokens.
 *   prefix_partition_size  prefix tokens per partition of the prefix pass: a positive multiple
 *                          of 16 (ignored when prefix_len == 0).
 *                          paged_attn_prefix_split() gives one that fills the device.
 *   partition_size         < 0: the balanced split of the suffix pass, as in paged_attn_decode
 *                          (paged_attn_balanced_split()).  Other values are PKV_ERR_SHAPE.
 *   tmp_out, max_logits,
 *   exp_sums               workspace with Pslots = paged_attn_shared_prefix_slots(
 *                          max_context_len, prefix_len, prefix_partition_size, partition_size)
 *                          slots per (row, head): shapes as in paged_attn_decode.  Its contents
 *                          on return are unspecified.
 *   out                    [num_seqs, num_heads, head_dim], q_dtype; always written.
 *   flags                  0 or PKV_FLAG_SHARED_BLOCKS, for the suffix pass (its blocks are
 *                          normally private to their rows).
 * Every other argument, the supported set and the error behaviour are those of
 * paged_attn_decode.  Entries that break the sharing contract give an unspecified result (no
 * out-of-bounds access); PKV_CHECK=1 validates it and returns PKV_ERR_CHECK.  Deterministic.
 */
int paged_attn_decode_shared_prefix(void* out, const void* query, const void* key_cache,
                                    const void* value_cache, const int32_t* block_tables, int max_blocks,
                                    const int32_t* context_lens, int num_seqs, int num_heads,
                                    int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                    float scale, int q_dtype, int kv_dtype, float k_scale, float v_scale,
                                    int max_context_len, int prefix_len, int prefix_partition_size,
                                    int partition_size, float* tmp_out, float* max_logits, float* exp_sums,
                                    int flags, void* stream);

/*
 * paged_attn_reduce -- merge split-K partials by log-sum-exp weighting.
 *
 * For every (b, h), with P the number of partials paged_attn_decode wrote for sequence b
 * under the same partition_size (ceil(n / partition_size) for fixed partitions; the number of
 * ranges the sequence's tiles fall in for a balanced split, recomputed from context_lens):
 *   M = max_{p<P} m_p,  w_p = l_p * exp(m_p - M),  out[b][h] = sum_p w_p o_p / sum_p w_p
 * rounded to out_dtype (nearest even).  P = 0, or partials that all saw no token (m = -inf,
 * l = 0, from the causal rows of paged_attn_multi_query), give a zero row.  Partials with
 * p >= P are never read.  Buffers and Pslots as in paged_attn_decode; num_heads counts the
 * output rows per sequence (q_len * heads after paged_attn_multi_query).
 */
int paged_attn_reduce(void* out, const float* tmp_out, const float* max_logits, const float* exp_sums,
                      const int32_t* context_lens, int num_seqs, int num_heads, int head_dim,
                      int max_context_len, int partition_size, int out_dtype, void* stream);

/*
 * paged_kv_copy_blocks -- copy whole blocks inside the K and V pools (the data side of
 * copy-on-write: "vllm-project-vllm -- L2", section 9 "Memory Management", COW sharing and
 * the COW fork for parallel sampling; the block manager below reports which copies a step
 * needs).
 *
 * For i < num_pairs: K[dst_blocks[i]] = K[src_blocks[i]] and V[dst_blocks[i]] =
 * V[src_blocks[i]], each block being block_size * num_kv_heads * head_dim elements of
 * cache_dtype (copied as bytes).  Every copy reads the pools as they were before the call:
 * destinations must be distinct and must not appear among the sources (otherwise the result
 * is unspecified).  A pair with an id outside [0, num_blocks) is skipped.
 *   key_cache, value_cache  [num_blocks, block_size, num_kv_heads, head_dim], device
 *   src_blocks, dst_blocks  [num_pairs] int32, device
 * block_size * num_kv_heads * head_dim * element bytes must be a multiple of 16.  PKV_CHECK=1
 * validates ranges and distinctness on the host (PKV_ERR_CHECK).
 */
int paged_kv_copy_blocks(void* key_cache, void* value_cache, const int32_t* src_blocks,
                         const int32_t* dst_blocks, int num_pairs, int num_blocks, int block_size,
                         int num_kv_heads, int head_dim, int cache_dtype, void* stream);

/*
 * paged_kv_swap_blocks -- move whole blocks between the device pools and pinned host pools
 * (swapping a preempted sequence's blocks to CPU memory and back: "vllm-project-vllm -- L2",
 * section 9 "Memory Management", preemptive scheduling and KV offload).
 *
 * to_host = 1: HK[host_blocks[i]] = K[dev_blocks[i]] (and V likewise); to_host = 0: the
 * reverse.  Targets must be distinct.  A pair with an id outside its pool is skipped.
 *   host_key, host_value  [num_host_blocks, block_size, num_kv_heads, head_dim] in pinned
 *                         host memory (hipHostMalloc, or a pinned torch tensor); the library
 *                         reads/writes it through its device mapping, so the transfer crosses
 *                         the host link.  PKV_ERR_HOST if the memory is not pinned and mapped
 *                         or the allocation is smaller than the pool.
 *   dev_blocks, host_blocks  [num_pairs] int32, device
 * Ordering: asynchronous on `stream` like every call; the host pool is complete after the
 * stream is synchronised.
 */
int paged_kv_swap_blocks(void* key_cache, void* value_cache, void* host_key, void* host_value,
                         const int32_t* dev_blocks, const int32_t* host_blocks, int num_pairs,
                         int num_blocks, int num_host_blocks, int block_size, int num_kv_heads,
                         int head_dim, int cache_dtype, int to_host, void* stream);

/*
 * Block manager -- host-side bookkeeping of the pool ("vllm-project-vllm -- L2", section 9
 * "Memory Management"; section 8 on the block-table invariant; section 11 steps 2 and 5).
 *
 * A sequence owns ceil(num_tokens / block_size) blocks, so at most block_size - 1 of its
 * slots are unused; appending a token allocates a block only when the last one is full.
 * A fork shares the parent's blocks (reference counts, no data copied); appending into a
 * shared last block first moves the appender to a fresh copy (copy-on-write), reported as a
 * (src, dst) pair for paged_kv_copy_blocks.  Invariant, checked by pkv_bm_check: every
 * device block is free (count 0, in the free set) or referenced exactly count times by
 * sequence tables.  Swap-out moves every block of a sequence to the host pool (shared blocks
 * are copied, the device copies stay with their other owners); swap-in brings them back into
 * fresh device blocks.
 * Policy (not fixed by the pages): the lowest-numbered free block is always taken first.
 * The handle is not thread-safe; every call is host-only and synchronous.
 */
typedef struct pkv_block_manager pkv_block_manager;

/* num_blocks device blocks and num_host_blocks host blocks of block_size tokens; NULL on
   a bad size or out of memory. */
pkv_block_manager* pkv_bm_create(int num_blocks, int block_size, int num_host_blocks);
void pkv_bm_destroy(pkv_block_manager* bm);
int pkv_bm_num_free(const pkv_block_manager* bm);
int pkv_bm_num_free_host(const pkv_block_manager* bm);
/* New sequence holding num_tokens tokens (a prompt): ceil(num_tokens / block_size) blocks. */
int pkv_bm_add(pkv_block_manager* bm, int64_t seq_id, int64_t num_tokens);
/* Append one token: *slot = block * block_size + offset of its cache row.  If the last block
   was shared, *copy_src / *copy_dst name the copy to make before writing (else both -1). */
int pkv_bm_append(pkv_block_manager* bm, int64_t seq_id, int64_t* slot, int32_t* copy_src,
                  int32_t* copy_dst);
/* child shares the parent's first num_tokens tokens (num_tokens < 0: all of them). */
int pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child, int64_t num_tokens);
int pkv_bm_free(pkv_block_manager* bm, int64_t seq_id);
/* Move a sequence's blocks out to / back from the host pool.  Fills (dev_blocks[i],
   host_blocks[i]) pairs for paged_kv_swap_blocks and returns their number (or an error). */
int pkv_bm_swap_out(pkv_block_manager* bm, int64_t seq_id, int32_t* dev_blocks, int32_t* host_blocks,
                    int capacity);
int pkv_bm_swap_in(pkv_block_manager* bm, int64_t seq_id, int32_t* host_blocks, int32_t* dev_blocks,
                   int capacity);
int pkv_bm_num_tokens(const pkv_block_manager* bm, int64_t seq_id, int64_t* num_tokens);
/* Host arrays: block_tables [num_seqs, max_blocks] (entries past a sequence's blocks are 0)
   and context_lens [num_seqs] of the listed (resident) sequences. */
int pkv_bm_table(const pkv_block_manager* bm, const int64_t* seq_ids, int num_seqs,
                 int32_t* block_tables, int max_blocks, int32_t* context_lens);
/* PKV_OK if the invariant above and the block-count bound hold, else PKV_ERR_CHECK. */
int pkv_bm_check(const pkv_block_manager* bm);

/* Partial slots per (sequence, head) a split-K schedule needs (0 for partition_size == 0). */
int paged_attn_partial_slots(int max_context_len, int partition_size);

/* Bytes of tmp_out + max_logits + exp_sums that split-K needs (0 if partition_size == 0). */
size_t paged_attn_workspace_bytes(int num_seqs, int num_heads, int head_dim, int max_context_len,
                                  int partition_size);

/* partition_size (negative) of the balanced split that fills the current HIP device once:
   -(compute units x decode workgroups resident per unit) for this shape and dtype pair.
   Returns 0 if no device is available or the shape is unsupported.  Queries the device. */
int paged_attn_balanced_split(int num_kv_heads, int head_dim, int q_dtype, int kv_dtype);

/* partition_size (negative) of the balanced split that fills the current HIP device for
   paged_attn_multi_query with q_len new tokens: paged_attn_balanced_split() when
   (num_heads / num_kv_heads) * q_len <= 32, else about one tiled workgroup per compute unit.
   Returns 0 if no device is available or the shape is unsupported.  Queries the device. */
int paged_attn_multi_query_split(int num_heads, int num_kv_heads, int head_dim, int q_len, int q_dtype,
                                 int kv_dtype);

/* Partial slots per (row, head) paged_attn_decode_shared_prefix needs: ceil(prefix_len /
   prefix_partition_size) for the prefix plus the balanced split's slots for the
   max(max_context_len - prefix_len, 0) tokens past it.  PKV_ERR_SHAPE for invalid arguments. */
int paged_attn_shared_prefix_slots(int max_context_len, int prefix_len, int prefix_partition_size,
                                   int partition_size);

/* prefix_partition_size for paged_attn_decode_shared_prefix that gives the prefix pass about one
   workgroup per compute unit of the current HIP device (a multiple of 64).
   Returns 0 if no device is available or an argument is invalid.  Queries the device. */
int paged_attn_prefix_split(int num_seqs, int num_heads, int num_kv_heads, int prefix_len);

/*
 * pkv_time_next_call -- measurement hook.  Binds two caller-owned HIP events (hipEvent_t,
 * created with timing enabled) to the kernels of the NEXT attention call made on the calling
 * thread (paged_attn_decode, paged_attn_multi_query, paged_attn_decode_append,
 * paged_attn_decode_shared_prefix, paged_attn_decode_noalloc or paged_attn_reduce):
 * `start_event` is recorded when that
 * call's first kernel starts and `stop_event` when its last kernel ends (hipExtLaunchKernel),
 * so hipEventElapsedTime(start, stop) is the call's GPU execution time with no marker packet
 * between kernels.  One-shot: the next attention call consumes the events whether or not it
 * launches anything (a call that fails its checks records nothing).  Either event may be NULL.
 * Thread-local state; the library keeps the handles only until that call returns.  Returns
 * PKV_OK.
 */
int pkv_time_next_call(void* start_event, void* stop_event);

/* Static English text for a pkv_status value. */
const char* pkv_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
