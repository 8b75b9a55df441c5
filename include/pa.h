/*
 * pa.h -- C ABI of libpa.so: paged-KV-cache decode attention on MI355X (gfx950).
 *
 * Two operations, after the pages this library follows:
 *
 *   pa_reshape_and_cache  writes the K and V of new tokens into their cache
 *                         slots ("vLLM" note, section "PagedAttention": the page
 *                         holding a token is its position divided by the block
 *                         size; the cache engine writes pages), optionally
 *                         quantising to FP8 ("vLLM 前世今生", §5.2 and §7.3).
 *   pa_decode             one decode step of attention: every sequence's query
 *                         heads attend over that sequence's cached tokens,
 *                         reached through its block table ("vLLM 前世今生",
 *                         §3.2: fixed 16-token blocks, block table, blocks
 *                         shared between sequences), with grouped-query heads
 *                         ("vLLM" note, section "内核优化"). The result is
 *                         softmax(q·Kᵀ·scale)·V per query head.
 *
 * Memory and layouts (all arrays dense, row-major, no strides):
 *   key, value        [num_tokens, num_kv_heads, head_size]          kv_dtype
 *   k_cache, v_cache  [num_blocks, num_kv_heads, block_size, head_size] cache_dtype
 *                     (one (block, kv head) tile is block_size*head_size
 *                      contiguous elements)
 *   slot_mapping      [num_tokens] int32 or int64; slot = block*block_size + row;
 *                     a negative slot skips its token
 *   q                 [num_seqs, num_heads, head_size]                q_dtype
 *   out               [num_seqs, num_heads, head_size]                out_dtype
 *   block_tables      [num_seqs, max_blocks_per_seq] int32, physical block ids
 *   context_lens      [num_seqs] int32, tokens to attend (the newest included)
 *
 * Query head h reads KV head h / (num_heads / num_kv_heads).
 *
 * Ownership: every pointer is device memory owned by the caller (except those
 * documented as host arrays, read during the call) and must stay valid until
 * the work queued on `stream` has finished. The library never
 * allocates, frees, copies to the host or synchronises; both calls only queue
 * kernels on `stream` (a hipStream_t; NULL is the default stream) and return.
 * They hold no global state besides a thread-local error message and are safe
 * to call from several threads on different streams.
 *
 * Errors: 0 (PA_OK) on success, otherwise a pa_status code, with a message
 * for the calling thread in pa_last_error(). Arguments are validated on the
 * host without reading device memory; nothing is launched when validation
 * fails. Block ids, slots and context lengths are device data and cannot be
 * validated on the host; the kernels keep every access inside the caller's
 * buffers instead: a context length above max_blocks_per_seq*block_size is
 * treated as that maximum, a block id outside [0, num_blocks) reads block 0,
 * and a slot at or past num_blocks*block_size is skipped like a negative one.
 * Such inputs give meaningless results, never a memory fault. Launch
 * failures are reported as PA_ERR_LAUNCH.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_dtype {
  PA_DTYPE_F32 = 0,       /* IEEE binary32 */
  PA_DTYPE_F16 = 1,       /* IEEE binary16 */
  PA_DTYPE_BF16 = 2,      /* bfloat16 */
  PA_DTYPE_FP8_E4M3 = 3,  /* OCP OFP8 E4M3 (bias 7, max 448, NaN = S.1111.111); caches only */
  PA_DTYPE_I32 = 4,       /* int32: index arrays, in tensor descriptors only */
  PA_DTYPE_I64 = 5        /* int64: slot mappings, in tensor descriptors only */
} pa_dtype;

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = 1,         /* a required pointer is NULL */
  PA_ERR_DTYPE = 2,        /* dtype value or combination not supported */
  PA_ERR_SHAPE = 3,        /* a size is negative, zero where it must not be, or inconsistent */
  PA_ERR_UNSUPPORTED = 4,  /* block_size != 16, head_size not 64 or 128, too many query heads per KV head */
  PA_ERR_WORKSPACE = 5,    /* workspace missing, too small or misaligned */
  PA_ERR_LAUNCH = 6,       /* the HIP runtime rejected a kernel launch */
  PA_ERR_CAPACITY = 7,     /* block manager: the pool or a sequence's table row is full */
  PA_ERR_STATE = 8         /* block manager: unknown, duplicate or repeated sequence id */
} pa_status;

/*
 * pa_reshape_and_cache -- write new tokens' K and V into cache slots.
 *
 * For each token t with slot_mapping[t] >= 0 and each KV head:
 *   k_cache[slot / block_size, head, slot % block_size, :] = enc(key[t, head, :], k_scale)
 *   v_cache[...] likewise with value and v_scale.
 * enc copies the bits when cache_dtype == kv_dtype. With cache_dtype ==
 * PA_DTYPE_FP8_E4M3 it widens the element to float32, divides by the scale in
 * float32 (correctly rounded) and rounds to the nearest E4M3 value, ties to
 * even, saturating to +-448; NaN stays NaN, the sign bit is kept. The scales
 * are ignored for non-FP8 caches and must be finite and > 0 for FP8.
 *
 *   key, value      device, [num_tokens, num_kv_heads, head_size], kv_dtype (F32, F16 or BF16)
 *   k_cache, v_cache device, [num_blocks, num_kv_heads, block_size, head_size], cache_dtype
 *                   (== kv_dtype, or FP8_E4M3)
 *   slot_mapping    device, [num_tokens]; int64 if slot_is_int64 else int32
 *   num_tokens      >= 0 (0 queues nothing and returns PA_OK); num_tokens * num_kv_heads
 *                   * head_size * sizeof(kv_dtype) / 16 below 2^31 - 256 (PA_ERR_SHAPE)
 *   block_size      must be 16; head_size must be 64 or 128
 *
 * Slots must be distinct within one call (two tokens writing one slot race).
 */
int pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                         const void* slot_mapping, int slot_is_int64, int64_t num_tokens,
                         int num_kv_heads, int head_size, int64_t num_blocks, int block_size,
                         pa_dtype kv_dtype, pa_dtype cache_dtype, float k_scale, float v_scale,
                         void* stream);

/*
 * pa_decode -- one decode step of paged attention.
 *
 * For every sequence s with n = context_lens[s] and every query head h:
 *   out[s, h, :] = sum_p w_p V_p / sum_p w_p,  w_p = exp(scale * dot(q[s, h], K_p)),
 * over token positions p < n, where K_p, V_p are row p % block_size of KV head
 * h / (num_heads / num_kv_heads) in physical block block_tables[s, p / block_size]
 * (an FP8 cache's codes are multiplied by k_scale / v_scale). n == 0 writes
 * zeros. Table entries at and past ceil(n / block_size) are never read, nor
 * are the rows past n of the last block. Accumulation is float32; out is
 * rounded to out_dtype to nearest, ties to even.
 *
 *   out             device, [num_seqs, num_heads, head_size], out_dtype (q_dtype or F32)
 *   q               device, [num_seqs, num_heads, head_size], q_dtype (F32, F16 or BF16)
 *   k_cache, v_cache device, [num_blocks, num_kv_heads, block_size, head_size], cache_dtype
 *                   (== q_dtype, or FP8_E4M3 with F16 or BF16 queries)
 *   block_tables    device, int32 [num_seqs, max_blocks_per_seq]
 *   context_lens    device, int32 [num_seqs], each <= max_blocks_per_seq * block_size
 *   scale           softmax scale (usually 1/sqrt(head_size)), finite
 *   num_kv_heads    >= 1 and divides num_heads
 *   block_size      must be 16; head_size 64 or 128
 *   workspace       device scratch of at least pa_decode_workspace_bytes(...) bytes,
 *                   256-byte aligned; may be NULL when that size is 0. Its
 *                   contents on entry do not matter; it must not be shared with
 *                   a call running concurrently.
 *   stream          hipStream_t to queue on
 *
 * Schedules. Partitioned: a context longer than one partition (its length
 * chosen on the host from the shapes) is split; each partition writes its
 * running max, sum and unnormalised output to the workspace, and a second
 * kernel merges the partitions. Balanced (the library's own choice for the
 * matrix-core kernel, when num_seqs <= 1024 and the workspace holds
 * pa_decode_workspace_bytes(..., 0) bytes): the blocks of all sequences, laid
 * end to end, are cut into equal ranges, one per wave, whatever the context
 * lengths, so a ragged batch keeps every wave busy to the end; pieces of a
 * sequence cut by a range boundary are merged by a second kernel. With a
 * smaller or NULL workspace the partitioned schedule runs (and may itself
 * need one). Both merge in a fixed order: results are deterministic run to run.
 *
 * Kernel choice: with F16/BF16 queries and a multiple of 4 query heads per
 * KV head, the products of a K/V tile with the group's queries run on the
 * matrix cores (MFMA); otherwise on the vector ALU. Both give the result above
 * within float32 accumulation error. The environment variable PA_DECODE_PATH
 * (read on every call) forces "valu" or "mfma" (the latter only where it
 * applies), for comparison runs; PA_DECODE_LOADS=cached makes the MHA
 * vector kernel read K/V with cached instead of nontemporal loads (likewise).
 */
int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* context_lens, float scale,
              int num_kv_heads, int block_size, int num_seqs, int num_heads, int head_size,
              int max_blocks_per_seq, int64_t num_blocks, pa_dtype q_dtype, pa_dtype cache_dtype,
              pa_dtype out_dtype, float k_scale, float v_scale, void* workspace,
              size_t workspace_bytes, void* stream);

/*
 * pa_prefill -- chunked-prefill attention over the paged cache ("vLLM 前世今生"
 * §5.4 and §7.3: a long prompt is processed in chunks that run next to
 * decode steps; §3.2: the paged cache).
 *
 * Sequence s has context_lens[s] tokens in the cache, the last
 * q_len = query_start_loc[s+1] - query_start_loc[s] of which are its current
 * chunk (their K/V written with pa_reshape_and_cache beforehand). Query row
 * t = query_start_loc[s] + i (i < q_len) sits at position
 * p = context_lens[s] - q_len + i and attends causally to positions 0..p:
 *   out[t, h, :] = sum_{j<=p} w_j V_j / sum_{j<=p} w_j,  w_j = exp(scale * dot(q[t, h], K_j)),
 * with K_j, V_j read through the block table as in pa_decode (FP8 codes times
 * k_scale / v_scale). A chunk of one token is a decode step.
 *
 *   out             device, [num_tokens, num_heads, head_size], out_dtype (q_dtype or F32)
 *   q               device, [num_tokens, num_heads, head_size], F16 or BF16
 *   k_cache, v_cache device, as in pa_decode; cache_dtype == q_dtype or FP8_E4M3
 *   block_tables    device, int32 [num_seqs, max_blocks_per_seq]
 *   context_lens    device, int32 [num_seqs] (chunk included)
 *   query_start_loc device, int32 [num_seqs + 1], non-decreasing, starting at 0
 *   max_query_len   host upper bound of every q_len (sizes the grid)
 *
 * A q_len above max_query_len or above context_lens[s] is cut to the smaller
 * bound; rows beyond it are not written. Accumulation is float32 (weights
 * carried as two 16-bit parts); results agree with the definition within
 * float32 accumulation error. Runs on the matrix cores; no workspace.
 */
int pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
               const int32_t* context_lens, const int32_t* query_start_loc, float scale, int num_kv_heads,
               int block_size, int num_seqs, int num_heads, int head_size, int max_blocks_per_seq,
               int64_t num_blocks, int max_query_len, pa_dtype q_dtype, pa_dtype cache_dtype, pa_dtype out_dtype,
               float k_scale, float v_scale, void* stream);

/*
 * pa_decode_split -- pa_decode with an explicit partition length.
 *
 * partition_blocks = number of 16-token blocks per partition, a multiple of 4
 * in [4, 512] (the partitioned schedule), or 0 for the library's own choice
 * (then identical to pa_decode). Results equal pa_decode's up to float32
 * rounding order. Used to exercise and time given split factors.
 */
int pa_decode_split(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens, float scale,
                    int num_kv_heads, int block_size, int num_seqs, int num_heads, int head_size,
                    int max_blocks_per_seq, int64_t num_blocks, pa_dtype q_dtype,
                    pa_dtype cache_dtype, pa_dtype out_dtype, float k_scale, float v_scale,
                    int partition_blocks, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_workspace_bytes -- workspace size pa_decode / pa_decode_split need
 * for these shapes. Pure function of its arguments; returns 0 for invalid
 * shapes. partition_blocks as in pa_decode_split. With a partition length:
 * the partitioned schedule's need (0 when no sequence can span two
 * partitions). With 0 (the library's choice), which sees no dtype: the larger
 * of the partitioned need and, where the balanced schedule can apply (a
 * multiple of 4 query heads per KV head, num_seqs <= 1024), its need of
 * num_heads * (num_seqs + R) * (head_size + 2) floats plus num_seqs + 1 ints,
 * R being its number of ranges (for this size, the larger count it takes
 * with an FP8 cache; a 16-bit cache takes half as many ranges).
 */
size_t pa_decode_workspace_bytes(int num_seqs, int num_heads, int num_kv_heads, int head_size,
                                 int max_blocks_per_seq, int block_size, int partition_blocks);

/*
 * pa_decode_shared_prefix -- pa_decode for a batch in which groups of
 * sequences share the first physical blocks of their block tables ("vLLM
 * 前世今生" §3.2: sequences that share a prompt prefix map it to the same
 * physical blocks; "vLLM" note, section "前缀缓存": prefix caching). The
 * result is pa_decode's (up to float32 rounding order); only the reading of
 * the shared blocks changes: they are read once per 16 / G sequences of a
 * group (G = num_heads / num_kv_heads) instead of once per sequence.
 *
 *   prefix_groups  host, int32 [num_groups][3]: (first_seq, num_seqs, shared_blocks).
 *                  Group i is sequences first_seq .. first_seq + num_seqs - 1,
 *                  whose block-table entries 0 .. shared_blocks - 1 are equal
 *                  (the first sequence's row is the one read) and whose contexts
 *                  hold at least shared_blocks * block_size tokens. Groups are
 *                  ordered and disjoint; 1 <= shared_blocks <= max_blocks_per_seq.
 *                  Read during the call only.
 *   num_groups     0 .. 16 (0: same as pa_decode)
 *   workspace      at least pa_decode_shared_prefix_workspace_bytes(..., max
 *                  shared_blocks) bytes, 256-byte aligned
 *   others         as in pa_decode
 *
 * The grouped reading applies with F16/BF16 queries, G in {4, 8, 16} and the
 * balanced schedule (num_seqs <= 1024); elsewhere the groups are ignored and
 * every block is read per sequence. A workspace too small for the balanced
 * schedule also leaves the groups unused (pa_decode's partitioned fallback);
 * one that holds the balanced schedule but not the per-part results is
 * refused (PA_ERR_WORKSPACE). The host validates the group list
 * (PA_ERR_SHAPE); that the tables agree and that the contexts are long
 * enough cannot be checked on the host: if they do not, the affected
 * sequences get meaningless values, never an out-of-bounds access.
 */
int pa_decode_shared_prefix(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens, float scale,
                            int num_kv_heads, int block_size, int num_seqs, int num_heads, int head_size,
                            int max_blocks_per_seq, int64_t num_blocks, pa_dtype q_dtype, pa_dtype cache_dtype,
                            pa_dtype out_dtype, float k_scale, float v_scale, const int32_t* prefix_groups,
                            int num_groups, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace pa_decode_shared_prefix needs when no group shares more than
 * max_shared_blocks blocks: pa_decode_workspace_bytes(..., 0) or, where the
 * grouped reading can apply, the balanced schedule's need plus num_seqs ints
 * and num_heads * num_seqs * ceil(max_shared_blocks / 64) * (head_size + 2)
 * floats of per-part results. 0 for invalid shapes.
 */
size_t pa_decode_shared_prefix_workspace_bytes(int num_seqs, int num_heads, int num_kv_heads, int head_size,
                                               int max_blocks_per_seq, int block_size, int max_shared_blocks);

/*
 * pa_decode_append -- one whole decode step: the newest token of every
 * sequence is written into its cache slot, then every sequence attends over
 * its context (the order "vLLM 前世今生" §3.2-3.3 implies for a step: the
 * cache holds the new token's K/V before attention reads it). Same result as
 * pa_reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, ...,
 * num_tokens = num_seqs) followed by pa_decode(...).
 *
 *   key, value      device, [num_seqs, num_kv_heads, head_size], q_dtype: the new
 *                   token of sequence s is row s
 *   slot_mapping    device, [num_seqs]; int64 if slot_is_int64 else int32; a
 *                   negative slot writes nothing. Slot s must be the slot of
 *                   position context_lens[s] - 1 of sequence s (a decode step's
 *                   new token), in a block no other sequence of the batch reads
 *                   (its private last block, as after copy-on-write). If it is
 *                   not, the caches still end as pa_reshape_and_cache leaves
 *                   them, but the output is undefined (a reader of that block
 *                   may see the row before or after the write).
 *   others          as in pa_decode (k_cache, v_cache written as by
 *                   pa_reshape_and_cache; k_scale / v_scale also encode FP8)
 *
 * Where exactly one wave of the decode launch reads the block holding a
 * sequence's new row for a KV head, the decode kernel writes the row itself,
 * by that wave, which waits for its own stores to complete before it loads
 * any block (one launch instead of two): the vector-ALU kernel with one
 * workgroup per (sequence, KV head) -- MHA or two query heads per KV head
 * with F16/BF16 queries, 1, 2, 4 or 8 with F32 queries -- and the matrix-core
 * kernel with 4, 8 or 16 query heads per KV head, in either schedule.
 * Elsewhere the reshape kernel runs first. Every argument is checked before
 * anything is queued; errors as in pa_reshape_and_cache and pa_decode.
 */
int pa_decode_append(void* out, const void* q, const void* key, const void* value, void* k_cache, void* v_cache,
                     const void* slot_mapping, int slot_is_int64, const int32_t* block_tables,
                     const int32_t* context_lens, float scale, int num_kv_heads, int block_size, int num_seqs,
                     int num_heads, int head_size, int max_blocks_per_seq, int64_t num_blocks, pa_dtype q_dtype,
                     pa_dtype cache_dtype, pa_dtype out_dtype, float k_scale, float v_scale, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * pa_decode_scratch -- pa_decode for callers that cannot allocate device
 * memory around a call (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): no workspace argument; the library's own
 * fixed scratch array serves as the workspace. Same arguments, result and
 * schedule choice as pa_decode with a workspace of pa_decode_scratch_bytes()
 * bytes; nothing is allocated or freed.
 *
 * The array lives in the library's device code, one copy per GPU, each held
 * until the process ends; its address on a device is looked up on the first
 * call with that device current, so the call must be made with the device
 * that `stream` belongs to current. Shapes whose workspace need exceeds the
 * array return PA_ERR_WORKSPACE with the sizes in the message (nothing
 * queued). Every call on one GPU uses that GPU's one array: calls that can
 * overlap on one GPU (other streams, other threads) race and must be
 * serialised by the caller; calls queued on one stream are ordered. The array
 * keeps the last call's contents; no call relies on them.
 */
int pa_decode_scratch(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, float scale, int num_kv_heads,
                      int block_size, int num_seqs, int num_heads, int head_size, int max_blocks_per_seq,
                      int64_t num_blocks, pa_dtype q_dtype, pa_dtype cache_dtype, pa_dtype out_dtype, float k_scale,
                      float v_scale, void* stream);

/* Size of pa_decode_scratch's fixed scratch array, in bytes (32 MiB). */
size_t pa_decode_scratch_bytes(void);

/* Partition length (in blocks) pa_decode would choose for these shapes. */
int pa_decode_partition_blocks(int num_seqs, int num_heads, int num_kv_heads, int head_size,
                               int max_blocks_per_seq, int block_size);

/*
 * pa_copy_blocks -- copy whole physical blocks, the device half of
 * copy-on-write ("vLLM 前世今生" §3.2: a block shared by several sequences is
 * copied before one of them writes into it).
 *
 * For i < num_pairs: block dst_blocks[i] of k_cache becomes a copy of block
 * src_blocks[i] (all KV heads, all 16 rows), and the same in v_cache.
 *
 *   k_cache, v_cache   device, [num_blocks, num_kv_heads, block_size, head_size], cache_dtype
 *   src_blocks, dst_blocks  device, int32 [num_pairs]; pairs as emitted by
 *                      pa_bm_append_slots
 *   num_pairs          0 .. 65535 (0 queues nothing)
 *   block_size         must be 16; head_size 64 or 128
 *
 * Destinations must be distinct and no block may be both a source and a
 * destination in one call (the copies run concurrently). A pair with an id
 * outside [0, num_blocks), or with src == dst, copies nothing. Asynchronous on
 * `stream`; must be queued before the reshape that writes into the copies.
 */
int pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_blocks, const int32_t* dst_blocks, int num_pairs,
                   int64_t num_blocks, int num_kv_heads, int head_size, int block_size, pa_dtype cache_dtype,
                   void* stream);

/*
 * Block manager -- host-side bookkeeping of the block pool ("vLLM 前世今生"
 * §3.2 and §3.3; "vLLM" note, section "PagedAttention"): blocks are taken from
 * a free list as sequences grow and returned when they finish (both O(1));
 * a forked sequence shares its parent's blocks (reference counts); appending
 * to a sequence whose last, partly filled block is shared first moves the
 * sequence to a private copy (copy-on-write), reported as a (source,
 * destination) pair for pa_copy_blocks.
 *
 * All functions run on the host, touch no device memory, and are not
 * thread-safe for one manager (callers serialise). Status codes as above;
 * a failing call changes nothing.
 */
typedef struct pa_block_manager pa_block_manager;

/* New manager of blocks 0 .. num_blocks-1 (all free); NULL on bad arguments.
 * block_size must be 16; a sequence may hold at most max_blocks_per_seq blocks. */
pa_block_manager* pa_bm_create(int64_t num_blocks, int block_size, int max_blocks_per_seq);
void pa_bm_destroy(pa_block_manager* bm);
/* Blocks on the free list (-1 for NULL). */
int64_t pa_bm_num_free_blocks(const pa_block_manager* bm);
/* Reference count of a block (0 = free), or -1 for an id outside the pool. */
int pa_bm_block_refcount(const pa_block_manager* bm, int32_t block);
/* Registers an empty sequence (PA_ERR_STATE if the id exists). */
int pa_bm_add_sequence(pa_block_manager* bm, int64_t seq_id);
/* New sequence `child` sharing all of `parent`'s blocks and its length. */
int pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child);
/* Drops a sequence; blocks no other sequence holds return to the free list. */
int pa_bm_free_sequence(pa_block_manager* bm, int64_t seq_id);
/*
 * Appends one token to each of n distinct sequences, in order. slots_out[i]
 * (host, int64 [n]) receives the slot (block * 16 + row) where sequence i's
 * new token is to be written (pa_reshape_and_cache). A sequence at a block
 * boundary takes a fresh block; one whose partly filled last block is shared
 * takes a fresh block too, and the pair (shared, fresh) is appended to
 * cow_src / cow_dst (host, int32, room for n each), their count to *num_cow.
 * PA_ERR_CAPACITY if the free blocks do not suffice or a row would overflow.
 */
int pa_bm_append_slots(pa_block_manager* bm, const int64_t* seq_ids, int n, int64_t* slots_out, int32_t* cow_src,
                       int32_t* cow_dst, int* num_cow);
/* Dense tables for n sequences: tables_out (host, int32 [n, max_blocks]) gets
 * each sequence's blocks padded with -1, lens_out (host, int32 [n]) its length. */
int pa_bm_block_tables(const pa_block_manager* bm, const int64_t* seq_ids, int n, int32_t* tables_out, int max_blocks,
                       int32_t* lens_out);

/*
 * The shared-prefix groups of a batch, as pa_decode_shared_prefix takes them
 * ("vLLM 前世今生" §3.2: forked sequences hold their common prompt in the same
 * physical blocks). seq_ids lists the batch in the order of its block-table
 * rows (as passed to pa_bm_block_tables). A group is a maximal run of
 * consecutive listed sequences that each hold at least min_blocks leading
 * blocks in common with the run's first sequence, counting only blocks that
 * are full in both; groups_out[3g .. 3g+2] = (index of its first sequence in
 * seq_ids, number of sequences >= 2, leading blocks shared by all of them).
 * Runs past max_groups are not reported (their sequences then read their
 * blocks themselves). *num_groups receives the count written. List forks of
 * one prompt next to each other to find them. Errors: PA_ERR_NULL,
 * PA_ERR_SHAPE (min_blocks < 1 or max_groups < 0), PA_ERR_STATE (unknown
 * sequence); nothing is written on error except *num_groups = 0.
 */
int pa_bm_shared_prefix(const pa_block_manager* bm, const int64_t* seq_ids, int n, int min_blocks,
                        int32_t* groups_out, int max_groups, int* num_groups);

/*
 * Tensor descriptors. pa_reshape_and_cache_t and pa_decode_t are
 * pa_reshape_and_cache and pa_decode with every array given as a pa_tensor
 * (pointer, dtype, shape, strides), so that the library itself checks that
 * the arrays agree with one another before anything is queued: ranks, dense
 * row-major strides (a dimension of size 1 may have any stride; an empty
 * tensor's strides are not looked at), element counts below 2^62, equal
 * shapes where the layouts above share a size, and the index dtypes. The
 * sizes the flat calls take (num_tokens, num_seqs, num_heads, head_size,
 * max_blocks_per_seq, num_blocks) come from the shapes; num_kv_heads and
 * block_size must match the caches'. They then forward to the flat call,
 * whose own checks and behaviour apply. Errors: PA_ERR_NULL (a NULL
 * descriptor, or a NULL data pointer in a non-empty tensor), PA_ERR_SHAPE (a
 * rank, stride or size that does not fit), PA_ERR_DTYPE (an index array that
 * is not int32, or a slot mapping neither int32 nor int64), and those of the
 * flat call.
 */
typedef struct pa_tensor {
  void* data;         /* device memory */
  pa_dtype dtype;
  int32_t ndim;       /* 1 to 4 */
  int64_t shape[4];   /* shape[0 .. ndim - 1] */
  int64_t stride[4];  /* in elements */
} pa_tensor;

/*
 *   key, value       [num_tokens, num_kv_heads, head_size], F32, F16 or BF16
 *   k_cache, v_cache [num_blocks, num_kv_heads, block_size, head_size]
 *   slot_mapping     [num_tokens], I32 or I64
 * Other arguments as in pa_reshape_and_cache.
 */
int pa_reshape_and_cache_t(const pa_tensor* key, const pa_tensor* value, const pa_tensor* k_cache,
                           const pa_tensor* v_cache, const pa_tensor* slot_mapping, float k_scale, float v_scale,
                           void* stream);

/*
 *   out, q           [num_seqs, num_heads, head_size]
 *   k_cache, v_cache [num_blocks, num_kv_heads, block_size, head_size]
 *   block_tables     [num_seqs, max_blocks_per_seq], I32
 *   context_lens     [num_seqs], I32
 * Other arguments as in pa_decode (the library's own schedule, as there).
 */
int pa_decode_t(const pa_tensor* out, const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                const pa_tensor* block_tables, const pa_tensor* context_lens, float scale, int num_kv_heads,
                int block_size, float k_scale, float v_scale, void* workspace, size_t workspace_bytes,
                void* stream);

/* Message for the last non-zero status returned on this thread ("" if none). */
const char* pa_last_error(void);

/* Library version, e.g. "0.1.0". */
const char* pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
