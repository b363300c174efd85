/*
 * pkv.h - C ABI of the paged KV cache decode library (libpkv.so) for AMD MI355X (gfx950).
 *
 * The library implements the decode hot path of PagedAttention:
 *   - a host-side block pool: fixed-size KV blocks (8, 16 or 32 tokens), a per-sequence
 *     block table, on-demand allocation, a free queue and reference-counted sharing
 *     ("vLLM ve Triton ile maliyet optimizasyonu", §03 Yöntem, steps 1-3 and the
 *     paragraph on sharing; "vLLM Nedir? PagedAttention ile Production LLM Serving",
 *     sections "PagedAttention" and "Bir istek motorun içinde"), with prefix caching
 *     and copy-on-write (kv_pool_add_seq_prefix, kv_pool_fork, copy_blocks);
 *   - reshape_and_cache: the slot-mapped write of each new token's K/V;
 *   - paged_attention_decode: single-query attention of a batch of sequences whose
 *     K/V are gathered through their block tables, with grouped-query attention, and
 *     paged_attention_decode_plan, its host-side schedule for a step;
 *   - paged_attention_reduce: the merge of per-partition results when the context
 *     is split into partitions;
 *   - paged_attention_prefill: causal multi-query attention for chunked prefill;
 *   - the same write and decode calls over an FP8 (e4m3) cache (*_fp8).
 *
 * General rules
 *   - Every function returns PKV_OK (0) or a negative PKV_E* code; pkv_last_error()
 *     returns a thread-local message for the last failure on the calling thread.
 *   - Device pointers are borrowed: the library never allocates, frees, copies or
 *     synchronises device memory. Kernels are enqueued on the caller's HIP stream
 *     (hipStream_t passed as void*; NULL = the null stream) and run asynchronously.
 *   - All host-side validation happens before any launch: an error return means
 *     nothing was enqueued. Values that live in device memory (slots, block ids,
 *     sequence lengths) are preconditions; the kernels never read or write outside
 *     the buffers whose sizes the arguments describe, but the results of rows that
 *     break a precondition are unspecified.
 *   - The pool object is not thread-safe; use one per thread or lock around it.
 *
 * Cache layout (per layer; the pages do not fix one). BS = block_size, the tokens per
 * block: 16 (the pages' figure, "vLLM ve Triton ile maliyet optimizasyonu", §03 Yöntem,
 * step 1), 8 or 32. x = 16 / element_bytes, i.e. 16 for an FP8 cache, 8 for fp16/bf16
 * and 4 for fp32:
 *   k_cache: [num_blocks][num_kv_heads][head_dim / x][BS][x]
 *   v_cache: [num_blocks][num_kv_heads][head_dim][BS]
 * Token t of a sequence lives in physical block table[t / BS], row t % BS. One
 * (block, KV head) tile of K or V is one contiguous run of BS * head_dim elements;
 * K keeps 16-byte groups of x dimensions per token together, V keeps the BS tokens
 * of each dimension together. Both match the operand layout of the gfx950 matrix
 * instructions, so the kernels load tiles straight into registers; they walk the
 * context in 16-token tiles (one block, half a block at BS = 32, two blocks at BS = 8),
 * except the decode at BS = 32 in the single pass and in partitions of whole blocks,
 * which walks whole blocks (results equal to fp32 summation order, not bit for bit,
 * to those at 8 and 16).
 * A slot is physical_block * BS + row. Every call that takes block_size accepts 8, 16
 * or 32 (EINVAL otherwise); the caches, tables and slots passed must use that size.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------------- */
#define PKV_OK 0
#define PKV_EINVAL (-1)  /* bad argument: null, shape, stride, alignment, range      */
#define PKV_ENOTSUP (-2) /* valid request that this build does not implement          */
#define PKV_ENOMEM (-3)  /* block pool exhausted (the call changed nothing)           */
#define PKV_ENOENT (-4)  /* unknown sequence id                                       */
#define PKV_EHIP (-5)    /* the HIP runtime reported an error at launch               */

/* ---- element types ----------------------------------------------------------- */
#define PKV_F32 0
#define PKV_F16 1
#define PKV_BF16 2
/* FP8 KV cache element: OCP e4m3 (1 sign, 4 exponent bits with bias 7, 3 mantissa
 * bits, no infinities, S.1111.111 = NaN, largest finite 448). A cache type only: for
 * kv_bytes_per_token, kv_pool_create and the *_fp8 entry points below. */
#define PKV_FP8_E4M3 3

/* the default block size (tokens per block) */
#define PKV_BLOCK_SIZE 16

/* partition_size value asking paged_attention_decode for the balanced split */
#define PKV_PARTITION_AUTO (-1)

/* Message for the last failing call on this thread ("" if none). Owned by the
 * library; valid until the next call on this thread. */
const char* pkv_last_error(void);

/* Library version string, e.g. "pkv 0.1.0 gfx950". */
const char* pkv_version(void);

/* ---- kernel timer ----------------------------------------------------------------
 * Not part of the method: a measuring aid. While enabled, every launch of the timed
 * entry points carries a HIP start/stop event pair bound to the kernel itself
 * (hipExtLaunchKernelGGL), so the pair measures that kernel alone without adding
 * packets to the stream. pkv_timer_read(entry, ...) waits for the pairs recorded since
 * the last read (or enable) of that entry, returns their summed milliseconds and count,
 * and resets them. For paged_attention_decode only its main kernel is timed.
 * Enabling or disabling clears every entry. The events belong to the device that was
 * current at their first use; time one device per process. Errors: EINVAL, EHIP. */
#define PKV_TIMER_DECODE 0
#define PKV_TIMER_REDUCE 1
#define PKV_TIMER_CACHE_WRITE 2
#define PKV_TIMER_COPY_BLOCKS 3
#define PKV_TIMER_PREFILL 4
#define PKV_TIMER_MEASURE 5
#define PKV_TIMER_ENTRIES 6
int pkv_timer_enable(int32_t enable);
int pkv_timer_read(int32_t entry, double* total_ms, int64_t* launches);

/* ---- streaming ceilings -----------------------------------------------------------
 * Not part of the method: measuring aids, timed under PKV_TIMER_MEASURE. They read and
 * fold their input into a running XOR per wave, stored to sink[w % sink_len] for wave w
 * (a device uint32 buffer; nothing else is written: with sink_len at least the number of
 * waves and a zeroed sink, the XOR over the sink is that of every 32-bit word read, an
 * invalid block id reading block 0), so the decode kernels' rates can be set against what
 * the same GPU streams with no arithmetic, and the gather against the contiguous read is
 * the cost of reading through a block table ("vLLM ve Triton ile maliyet optimizasyonu",
 * §05 Sınırlar, on the indirection cost of paged reads).
 * pkv_measure_read: bytes (a multiple of 16) of buf, 16-byte aligned, read once in order by
 *   device CUs x waves_per_cu (4 .. 32, a multiple of 4) waves, each with loads_in_flight
 *   (2, 4, 8 or 16) 16-byte loads per lane in flight.
 * pkv_measure_gather: the K and V tiles that paged_attention_decode reads for the batch
 *   (every (block, KV head) tile of every sequence's first ceil(n / block_size) table
 *   entries; head_dim * block_size * element bytes of 1, 2, 4 or 8 KiB). balanced == 0:
 *   the single pass's decomposition, one workgroup of 4 waves per (KV head, sequence) in
 *   its grid order (seq_order as for paged_attention_decode, or NULL), the waves taking
 *   blocks round-robin two in flight. balanced != 0 (16-token blocks): all tiles of the
 *   batch in one list cut into equal runs, one per wave, 8 waves per CU.
 * nontemporal != 0: the loads carry the non-temporal hint, as the decode kernels' tile loads
 *   do (the caches do not keep the lines); 0: plain loads.
 * Errors: EINVAL, ENOTSUP (sizes not built), EHIP. */
int pkv_measure_read(const void* buf, int64_t bytes, int32_t waves_per_cu, int32_t loads_in_flight,
                     int32_t nontemporal, uint32_t* sink, int32_t sink_len, void* stream);
int pkv_measure_gather(const void* k_cache, const void* v_cache, const int32_t* block_tables,
                       const int32_t* seq_lens, int32_t num_seqs, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size, int32_t cache_dtype,
                       int32_t max_blocks_per_seq, int64_t num_blocks, const int32_t* seq_order,
                       int32_t balanced, int32_t nontemporal, uint32_t* sink, int32_t sink_len,
                       void* stream);
/* pkv_measure_rate: what the SIMDs sustain on the kernels' building blocks, with
 * waves_per_simd (1 .. 8) waves on every SIMD of the device (CUs x waves_per_simd
 * workgroups of 4 waves), each running iters iterations of: kind 0, 8 conflict-free 16-byte
 * LDS reads per lane (chunk ((8t + j) * 257 + tid) mod 1024 of a workgroup-local 16 KiB
 * array whose chunk i holds (i, 3i, 5i, 7i), folded by XOR); 1, 8 exponentials (v_exp_f32)
 * in independent chains; 2, 8 FMAs; 3, 4 bf16 16x16x32 matrix products (4 accumulators);
 * 4, kind 3's products with kind 1's exponentials between them; 5, the 4 products with 16
 * FMAs between them; 6, 4 bf16 16x16x16 products (half of kind 3's work per instruction). Used to set the prefill kernel's mix of matrix and vector work
 * against what the hardware overlaps (the prefill steps of "vLLM Nedir? PagedAttention ile
 * Production LLM Serving", section "Chunked prefill"). Errors: EINVAL, EHIP. */
int pkv_measure_rate(int32_t kind, int32_t waves_per_simd, int32_t iters, uint32_t* sink,
                     int32_t sink_len, void* stream);

/* ---- KV bytes per token ------------------------------------------------------------
 * 2 (K and V) x layers x KV heads x head_dim x bytes per element
 * ("Yerel LLM sistemlerinde backpressure ve ölçekleme", section "KV bütçesi": the
 * formula, with 327,680 bytes for an 80-layer, 8-KV-head, head_dim 128 FP16 model;
 * "vLLM Nedir? ...", section "Asıl şişen şey ağırlık değil, KV cache": about 128 KB
 * for 32 layers). PKV_FP8_E4M3 counts one byte per element, half the FP16 figure
 * (same page, the paragraph on KV cache quantisation). Returns -1 for a bad argument. */
int64_t kv_bytes_per_token(int32_t num_layers, int32_t num_kv_heads, int32_t head_dim,
                           int32_t dtype);

/* ==== host block pool ========================================================= */

typedef struct kv_pool kv_pool;

typedef struct {
    int64_t total_blocks;   /* num_blocks                                     */
    int64_t free_blocks;    /* blocks in the free queue                       */
    int64_t used_blocks;    /* blocks with reference count >= 1              */
    int64_t shared_blocks;  /* blocks with reference count >= 2              */
    int64_t alloc_failures; /* appends refused with PKV_ENOMEM so far         */
    int64_t num_seqs;       /* live sequences                                 */
    int64_t cached_blocks;  /* blocks holding a prefix-cache key              */
    int64_t prefix_hit_blocks; /* blocks found by kv_pool_add_seq_prefix so far */
} kv_pool_stats_t;

/* Create a pool of num_blocks physical blocks of block_size (8, 16 or 32) tokens for
 * a model with num_layers layers, num_kv_heads KV heads of head_dim elements of
 * type dtype. One block id addresses the same block in every layer's cache.
 *   free_order: NULL for 0, 1, ..., num_blocks-1, else a permutation of those ids
 *               (copied) giving the initial order of the free queue.
 * The pool holds no device memory: the caller reserves the caches up front (for
 * each layer one K and one V buffer of kv_pool_cache_shape() elements), which is
 * the one-time reservation of "Yerel LLM ...", section "3. VRAM fragmantasyonu".
 * Errors: EINVAL (sizes, block_size, num_blocks * block_size above INT32_MAX, dtype,
 * not a permutation). */
int kv_pool_create(int64_t num_blocks, int32_t block_size, int32_t num_layers,
                   int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                   const int32_t* free_order, kv_pool** out);

/* Free the host state. NULL is a no-op. */
void kv_pool_destroy(kv_pool* pool);

/* kv_bytes_per_token() of the pool's model shape. */
int64_t kv_pool_bytes_per_token(const kv_pool* pool);

/* Shapes (in elements) of one layer's K and V cache in the layout above. */
int kv_pool_cache_shape(const kv_pool* pool, int64_t k_shape[5], int64_t v_shape[4]);

/* Register a new, empty sequence: a request entering the engine, before the scheduling
 * step allocates its slots ("vLLM Nedir? ...", section "Bir istek motorun içinde", steps 1
 * and 2). EINVAL if seq_id is already live. */
int kv_pool_add_seq(kv_pool* pool, int64_t seq_id);

/* Make empty sequence seq_id start with the first n_tokens tokens of src_seq_id by
 * pointing its table at the same physical blocks (reference count + 1 each), as for
 * a shared system prompt or parallel samples ("vLLM Nedir? ...", section
 * "PagedAttention", on block sharing; §03 on sharing). n_tokens must be a multiple
 * of the block size and at most src's length, so a shared block is full and never
 * written again (to share a partly filled block use kv_pool_fork, whose first append
 * copies it).
 * Errors: ENOENT (unknown id), EINVAL (seq not empty, n_tokens not allowed). */
int kv_pool_share_prefix(kv_pool* pool, int64_t seq_id, int64_t src_seq_id, int32_t n_tokens);

/* ---- prefix caching and copy-on-write ----------------------------------------------
 * ("vLLM Nedir? ...", section "Prefix caching"; "vLLM ve Triton ...", §03 on sharing;
 * "Yerel LLM ...", section "4. Prefill ve decode", on eviction.)
 * Every full block of a sequence whose token ids are all known (kv_pool_add_seq_prefix,
 * kv_pool_append_tokens, kv_pool_append_batch_tokens; kv_pool_add_seq counts as an empty
 * prompt with salt 0) gets a key: a 64-bit hash chain over the salt and the token ids of
 * the blocks up to it, with the block's own token ids and its parent's chain hash kept to
 * check a hit. Only the first block with a given key holds it. A block freed to the free
 * queue keeps its key until it is popped for a new use (the free queue is the eviction
 * order); a hit on a free block takes it out of the queue. kv_pool_append,
 * kv_pool_append_batch and kv_pool_share_prefix give tokens without ids: that sequence's
 * later blocks get no key. */

/* Register seq_id with the longest run of cached blocks that starts its prompt: block j
 * (tokens BS j .. BS j + BS - 1) is looked up while it ends before the prompt's last
 * token, so at least one prompt token is always left to compute; the walk stops at the
 * first miss. *n_cached_out = BS x the blocks found (their reference counts + 1). The caller then
 * appends prompt[*n_cached_out ..] with kv_pool_append_tokens and writes only their K/V.
 * salt: blocks are found only under the salt they were stored with (tenant isolation).
 * Errors: EINVAL (seq_id live, n_prompt < 0, NULLs). */
int kv_pool_add_seq_prefix(kv_pool* pool, int64_t seq_id, const int32_t* prompt,
                           int32_t n_prompt, uint64_t salt, int32_t* n_cached_out);

/* child_id (new) shares every block of parent_id, the partly filled last block included
 * (reference counts + 1): parallel sampling and beam search branches. The first append
 * to a shared, partly filled block copies it (copy-on-write, see below).
 * Errors: ENOENT (parent), EINVAL (child live). */
int kv_pool_fork(kv_pool* pool, int64_t parent_id, int64_t child_id);

/* kv_pool_append for tokens with known ids (tokens[0 .. n_tokens)). If the sequence's
 * last block is partly filled and referenced by other tables too, the sequence first
 * moves to a fresh block: copy_out[0] = the old block, copy_out[1] = the new one, and the
 * caller must copy the old block's rows into the new one in every layer (copy_blocks)
 * before writing the new tokens' K/V; otherwise copy_out = {-1, -1}. Full blocks are
 * keyed as described above. ENOMEM (nothing changed) counts the copy's block too.
 * Errors: ENOENT, EINVAL (NULLs, n_tokens < 0), ENOMEM. */
int kv_pool_append_tokens(kv_pool* pool, int64_t seq_id, const int32_t* tokens, int32_t n_tokens,
                          int32_t* slot_mapping_out, int32_t* copy_out);

/* The decode step with token ids: one token (tokens[i]) for each of the n distinct
 * sequences; slot_mapping_out[i] as kv_pool_append_batch. The copies that copy-on-write
 * needs are listed in copies_out[0 .. 2 * *n_copies_out) as (old, new) pairs (at most
 * n). Sequences are served in the order given: when every table that shares a partly
 * filled block writes to it in this step, the last of them writes in place and only the
 * others copy it. All or nothing: ENOMEM (exactly when the free queue is shorter than
 * the blocks the step takes) leaves every sequence unchanged.
 * Errors: ENOENT, EINVAL (duplicates, NULLs), ENOMEM. */
int kv_pool_append_batch_tokens(kv_pool* pool, const int64_t* seq_ids, const int32_t* tokens,
                                int32_t n, int32_t* slot_mapping_out, int32_t* copies_out,
                                int32_t* n_copies_out);

/* allocate_slots: reserve n_tokens new positions at the end of seq_id and write
 * their slot ids to slot_mapping_out[0..n_tokens). A new physical block is popped
 * from the front of the free queue only when the sequence's last block is full
 * (§03 step 3; 17 new tokens in 16-token blocks take 2 blocks: "vLLM Nedir? ...",
 * section "Bir istek motorun içinde", step 2). If the free queue is too short the
 * call returns ENOMEM and changes nothing, so the caller can free (preempt) other
 * sequences and retry. Errors: ENOENT, EINVAL (n_tokens < 0, null output). */
int kv_pool_append(kv_pool* pool, int64_t seq_id, int32_t n_tokens, int32_t* slot_mapping_out);

/* Decode step: one new position for each of the n distinct sequences in seq_ids;
 * slot_mapping_out[i] is the slot of seq_ids[i]. All or nothing: ENOMEM leaves
 * every sequence unchanged. kv_pool_append and this call refuse (EINVAL) a sequence
 * whose last block is shared and partly filled: the *_tokens calls copy it.
 * Errors: ENOENT, EINVAL (duplicate ids, nulls). */
int kv_pool_append_batch(kv_pool* pool, const int64_t* seq_ids, int32_t n,
                         int32_t* slot_mapping_out);

/* Release seq_id: each of its blocks loses one reference; blocks that reach zero
 * are pushed to the back of the free queue in table order ("vLLM Nedir? ...",
 * section "Bir istek motorun içinde", step 5). Errors: ENOENT. */
int kv_pool_free_seq(kv_pool* pool, int64_t seq_id);

/* Length (tokens) of seq_id. Errors: ENOENT, EINVAL. */
int kv_pool_seq_len(const kv_pool* pool, int64_t seq_id, int64_t* len_out);

/* Copy seq_id's block table (at most capacity entries) to blocks_out; *n_out gets
 * the table length. Errors: ENOENT, EINVAL (capacity too small). */
int kv_pool_seq_blocks(const kv_pool* pool, int64_t seq_id, int32_t* blocks_out,
                       int32_t capacity, int32_t* n_out);

/* Copy the free queue, front first (at most capacity entries); *n_out gets its
 * length. Errors: EINVAL (capacity too small). */
int kv_pool_free_queue(const kv_pool* pool, int32_t* blocks_out, int64_t capacity,
                       int64_t* n_out);

/* Reference count of block blk (0 for a free block). Errors: EINVAL. */
int kv_pool_refcount(const kv_pool* pool, int64_t blk, int32_t* ref_out);

/* Dense block tables for the n sequences in seq_ids: the per-request table that maps
 * logical blocks to physical ones and that the attention kernel follows ("vLLM ve Triton
 * ...", §03 Yöntem, step 2). tables_out is int32 [n][max_blocks], row i holding
 * seq_ids[i]'s physical blocks then -1 padding; seq_lens_out[i] is its length. Host memory
 * (pinned or not).
 * Errors: ENOENT, EINVAL (a table longer than max_blocks, nulls). */
int kv_pool_build_tables(const kv_pool* pool, const int64_t* seq_ids, int32_t n,
                         int32_t max_blocks, int32_t* tables_out, int32_t* seq_lens_out);

/* Counters of the pool: every block is either free or used, so free + used = total
 * (equal-sized blocks leave no external fragmentation, "vLLM ve Triton ...", §03 Yöntem,
 * step 3); alloc_failures counts the refused allocations after which the scheduler drops
 * a request ("vLLM Nedir? ...", section "Bir istek motorun içinde", step 2). */
int kv_pool_stats(const kv_pool* pool, kv_pool_stats_t* out);

/* ==== device kernels ========================================================== */

/* reshape_and_cache: for every token t in [0, num_tokens) with s = slot_mapping[t]
 * in [0, num_blocks * BS), copy the raw bits of key[t][g][:] and value[t][g][:] for
 * every KV head g into row s % BS of block s / BS of k_cache / v_cache (layout
 * above). Tokens with a negative slot are skipped. Nothing else is written. This is
 * how a new token's K/V enter the block that on-demand allocation gave it (§03
 * step 3). Duplicate slots in one call are a caller error (which write wins is
 * unspecified); slots at or past num_blocks * BS are ignored.
 *   key, value:   device, dtype, element (t, g, i) at t * key_stride + g * head_dim + i
 *                 (resp. value_stride); 16-byte aligned, strides multiples of x.
 *   slot_mapping: device int32 [num_tokens].
 *   dtype: PKV_F32, PKV_F16 or PKV_BF16 (a bit copy: the type only sets the size).
 * Errors: EINVAL (nulls, alignment, block_size, head_dim not a positive
 * multiple of x, sizes), EHIP. num_tokens == 0 is a no-op.
 * Performance: write a prompt's (or a prefill chunk's) tokens in one call. Once
 * ceil(num_tokens / 16) * num_kv_heads reaches the device's compute units, each group
 * of 16 consecutive tokens is turned around on chip, so that consecutive slots are
 * written as contiguous bytes; a decode step's few scattered tokens take a
 * thread-per-16-bytes form instead. Both write the same bytes. */
int reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                      const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int64_t num_blocks,
                      int64_t key_stride, int64_t value_stride, int32_t dtype, void* stream);

/* paged_attention_decode: for each sequence b with context length n = seq_lens[b]
 * and query head h (KV head g = h / (num_heads / num_kv_heads), contiguous groups):
 *     s_t = scale * q[b][h] . K_b[t],  t < n,  K_b[t] read through block_tables[b]
 *     out[b][h] = sum_t softmax(s)_t V_b[t]
 * i.e. scaled dot-product attention with K/V gathered from scattered blocks (§03,
 * closing paragraphs: the math is unchanged, only the place K and V are read from
 * changes). Softmax is accumulated online in fp32; n counts the token being
 * decoded (write it with reshape_and_cache first). n == 0 gives a zero row.
 *
 *   q:            device [num_seqs][num_heads][head_dim], in_dtype; sequence stride
 *                 q_stride elements (>= num_heads * head_dim, multiple of x).
 *   k_cache/v_cache: device, layout above, num_blocks blocks, in_dtype.
 *   block_tables: device int32 [num_seqs][max_blocks_per_seq]; entries past
 *                 ceil(n / BS) are not read. seq_lens: device int32 [num_seqs].
 *   out:          device [num_seqs][num_heads][head_dim], out_dtype (in_dtype or
 *                 PKV_F32), written with round-to-nearest-even.
 *   partition_size == 0: one pass over the whole context; part_* may be NULL.
 *   partition_size  > 0 (a multiple of 16): the context is cut into partitions of
 *                 partition_size tokens and one workgroup handles each (sequence,
 *                 KV head, partition). A sequence with a single partition writes out
 *                 directly; otherwise each partition p < ceil(n / partition_size)
 *                 writes, for every query head of the group,
 *                   part_out[b][h][p][:] = attention restricted to the partition (fp32),
 *                   part_max[b][h][p]    = a reference logit m_p (natural-log units)
 *                                          within 8 ln 2 of the partition's largest s_t,
 *                   part_sum[b][h][p]    = sum of exp(s_t - m_p) over the partition,
 *                 so that part_max + log(part_sum) is the partition's log-sum-exp;
 *   partition_size == PKV_PARTITION_AUTO (fp16/bf16, num_seqs <= 1024): balanced
 *                 split. All (sequence, KV head, 16-token tile) triples form one list
 *                 that is cut into equal runs, one per wave of the launch, so ragged
 *                 lengths do not leave the device idle. A (sequence, KV head) whose
 *                 tiles all fall in one run writes out; otherwise each run's share
 *                 ("piece" k) writes part_out/part_max/part_sum at index k as above.
 *                 Pieces per (b, h) stay
 *                 <= max_partitions (>= 2 required): each run spans at least
 *                 ceil(T / (max_partitions - 1)) tiles of 16 tokens, T = ceil(
 *                 max_blocks_per_seq * BS / 16).
 *                 paged_attention_reduce must follow, with the same arguments: it
 *                 merges the split rows and writes the zero rows of empty sequences.
 *                 out and part_out must be 16-byte aligned in this mode.
 *   For partition_size > 0, part_* must be non-null with max_partitions >=
 *   ceil(max_blocks_per_seq * BS / partition_size), and paged_attention_reduce()
 *   produces out for the rows with more than one partition.
 *   seq_order:    NULL, or a host array of num_seqs ints, a permutation of 0 .. num_seqs-1
 *                 (paged_attention_decode_plan's output): the order in which the single
 *                 pass hands the sequences to its workgroups (copied into the launch; the
 *                 caller may reuse or free it on return). It only schedules: the results
 *                 are bit-identical with any order or with NULL, where the kernel ranks the
 *                 lengths itself (one extra dependent load and a ranking at every launch).
 *                 Used by the fp16/bf16 single pass with num_seqs <= 256; ignored otherwise.
 * Supported: head_dim in {64, 128}; in_dtype F16/BF16 with num_heads/num_kv_heads
 * <= 16; in_dtype F32 with num_heads/num_kv_heads <= 8 and 16-token blocks.
 * Errors: EINVAL (nulls, alignment, num_heads % num_kv_heads, block_size,
 * partition arguments, seq_order not a permutation, sizes), ENOTSUP (head_dim, group size,
 * dtype pair, F32 with block_size != 16), EHIP.
 * num_seqs == 0 is a no-op. */
int paged_attention_decode(void* out, float* part_out, float* part_max, float* part_sum,
                           const void* q, int64_t q_stride, const void* k_cache,
                           const void* v_cache, const int32_t* block_tables,
                           const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                           int32_t partition_size, int32_t max_partitions, int32_t in_dtype,
                           int32_t out_dtype, const int32_t* seq_order, void* stream);

/* paged_attention_decode_plan: the host half of a decode step's scheduling, computed once
 * per step and passed to every layer's decode call as seq_order. Decode rereads each
 * sequence's whole context every step and is bound by memory bandwidth ("Yerel LLM
 * sistemlerinde backpressure ve ölçekleme", section "4. Prefill ve decode"), and a batch
 * mixes very different context lengths (same page, section "Her istek eşit değildir"), so
 * the work is dealt so that every compute unit streams about as many bytes. From a host copy of the
 * batch's lengths (negative counts as 0): rank the sequences by length, longest first
 * (ties by index), and deal them in serpentine rounds of R = max(1, CUs / num_kv_heads)
 * sequences, CUs of the current HIP device: slot b of round r = b / R, position
 * pos = b - R r, takes rank R r + pos in even rounds and R r + (n_r - 1 - pos) in odd
 * ones (n_r = sequences in that round). Workgroups are dispatched one compute unit after
 * the other, so a unit that holds one of the longest sequences also holds one of the
 * shortest, and the units finish together. order_out: host int32 [num_seqs].
 * Errors: EINVAL (NULLs, num_seqs < 0, num_kv_heads <= 0). */
int paged_attention_decode_plan(const int32_t* seq_lens, int32_t num_seqs, int32_t num_kv_heads,
                                int32_t* order_out);

/* paged_attention_decode_append: the decode step of one new token per sequence in one
 * call: reshape_and_cache of key/value rows b (one token each, num_tokens = num_seqs)
 * into slot_mapping[b], then paged_attention_decode over seq_lens[b] tokens, which
 * include the new one (the write-then-attend order of "vLLM ve Triton ile maliyet
 * optimizasyonu", §03 Yöntem, steps 3-4; the new token attends to itself).
 *   key, value: [num_seqs][num_kv_heads][head_dim] rows of in_dtype, sequence strides
 *               key_stride / value_stride in elements (>= num_kv_heads * head_dim,
 *               multiples of 16 bytes), 16-byte aligned. Borrowed, read only.
 *   slot_mapping: int32 [num_seqs], device. The result equals the two separate calls
 *               when slot_mapping[b] is the slot of position seq_lens[b] - 1 of
 *               sequence b (what kv_pool_append / kv_pool_append_batch return) or is
 *               negative (nothing written). For any other slot the row is still written
 *               (slots outside the pool are skipped), but whether position
 *               seq_lens[b] - 1 then sees the new row or the cache's earlier content is
 *               unspecified.
 * For fp16/bf16 with partition_size >= 0 the write is fused into the decode launch:
 * the wave holding the newest position stores the row into the caches and takes it for
 * the attention from key/value instead of reading it back, placing it where the cache
 * row would be, so the result equals the two calls' bit for bit. With fp32 inputs
 * or PKV_PARTITION_AUTO the write is a separate launch ahead of the decode on the same
 * stream. The other arguments, the outputs and the errors are those of
 * paged_attention_decode (and of reshape_and_cache for the new rows); with
 * partition_size != 0, paged_attention_reduce must follow as for paged_attention_decode. */
int paged_attention_decode_append(void* out, float* part_out, float* part_max, float* part_sum,
                                  const void* q, int64_t q_stride, const void* key,
                                  const void* value, int64_t key_stride, int64_t value_stride,
                                  const int32_t* slot_mapping, void* k_cache, void* v_cache,
                                  const int32_t* block_tables, const int32_t* seq_lens,
                                  int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                  int64_t num_blocks, float scale, int32_t partition_size,
                                  int32_t max_partitions, int32_t in_dtype, int32_t out_dtype,
                                  const int32_t* seq_order, void* stream);

/* paged_attention_reduce: the merge that makes a context split into partitions give the
 * same softmax-weighted sum as one pass over it (the attention math is unchanged by where
 * K and V are read from, "vLLM ve Triton ...", §03 Yöntem, closing paragraphs; long
 * contexts beside short ones, "Yerel LLM ...", section "Her istek eşit değildir", are split
 * so that one sequence does not serialise on one workgroup). For every (b, h) whose sequence has more than one
 * partition (np = ceil(seq_lens[b] / partition_size) > 1; with PKV_PARTITION_AUTO, np
 * is the number of pieces of the balanced split, and rows of empty sequences are
 * written as zeros):
 *     M = max_p part_max,  w_p = exp(part_max[p] - M) * part_sum[p],
 *     out[b][h] = sum_p w_p part_out[p] / sum_p w_p        (p < np only)
 * Rows with np <= 1 are not touched (the decode kernel wrote them). Buffers and
 * num_kv_heads, block_size, max_blocks_per_seq, partition_size, max_partitions are those
 * of the paged_attention_decode call; out_dtype in {F32, F16, BF16}; out and part_out must be
 * 16-byte aligned. Each row is merged in 32-dimension slices, one workgroup per
 * (slice, head, sequence), reading every record once. Errors: EINVAL, ENOTSUP, EHIP. */
int paged_attention_reduce(void* out, const float* part_out, const float* part_max,
                           const float* part_sum, const int32_t* seq_lens, int32_t num_seqs,
                           int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t max_blocks_per_seq,
                           int32_t partition_size, int32_t max_partitions, int32_t out_dtype,
                           void* stream);

/* paged_attention_decode_noalloc: for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). It is
 * paged_attention_decode with partition_size > 0 or PKV_PARTITION_AUTO followed by
 * paged_attention_reduce, with the partition records (part_out, part_max, part_sum) kept
 * in a static device workspace of paged_attention_decode_noalloc_workspace() bytes
 * (64 MiB) instead of caller buffers. The workspace belongs to the library: the runtime
 * reserves it on each device when the library's code is first used there, and it stays
 * reserved until the process ends; the call itself allocates and frees nothing.
 *   Every call on one device shares that device's workspace, so calls that may overlap on
 *   one device (other streams, other threads) race and must be serialised by the caller;
 *   calls on one stream are ordered and safe. Nothing in the workspace needs clearing.
 *   partition_size == 0 is the single pass and uses no workspace.
 *   Records: num_seqs * num_heads rows of P records of (head_dim + 2) floats, with
 *   P = ceil(max_blocks_per_seq * block_size / partition_size) for fixed partitions, and for
 *   PKV_PARTITION_AUTO P = max(2, ceil(T / 4) + 1) (T = ceil(max_blocks_per_seq *
 *   block_size / 16)) lowered to what the workspace holds (longer pieces, same result to
 *   fp32 rounding).
 *   out must be 16-byte aligned. Other arguments, outputs and errors as
 *   paged_attention_decode; EINVAL (nothing enqueued) when the records do not fit, with a
 *   message giving the bytes needed. */
size_t paged_attention_decode_noalloc_workspace(void);
int paged_attention_decode_noalloc(void* out, const void* q, int64_t q_stride, const void* k_cache,
                                   const void* v_cache, const int32_t* block_tables,
                                   const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                                   int32_t partition_size, int32_t in_dtype, int32_t out_dtype,
                                   void* stream);

/* paged_attention_prefill: causal multi-query attention over the paged cache, for
 * chunked prefill: a long prompt is processed in chunks over several steps, each chunk's
 * K/V written to the cache (reshape_and_cache) before its queries attend ("vLLM Nedir?
 * ...", section "Chunked prefill"; "Yerel LLM ...", section "4. Prefill ve decode").
 * Sequence b's queries are rows q_start[b] .. q_start[b+1] - 1 of q: the last
 * L_b = q_start[b+1] - q_start[b] of its n = seq_lens[b] positions. Query i (position
 * p = n - L_b + i) of query head h attends to positions 0 .. p of KV head
 * h / (num_heads / num_kv_heads):
 *     out[r][h] = sum_{t <= p} softmax_t(scale * q[r][h] . K_b[t]) V_b[t]
 * A query with p < 0 (L_b > n) gets a zero row. Single-query rows (L_b = 1) are the
 * decode step; paged_attention_decode is the faster call for those.
 *   q:       device, in_dtype (F16 or BF16), row r at q + r * q_stride elements
 *            (q_stride >= num_heads * head_dim, a multiple of 8), heads dense in a row.
 *   q_start: device int32 [num_seqs + 1], q_start[0] = 0, non-decreasing;
 *            L_b <= max_q_len (rows past max_q_len are not computed).
 *   out:     device [q_start[num_seqs]][num_heads][head_dim], out_dtype (in_dtype or F32),
 *            16-byte aligned.
 *   caches, block_tables, seq_lens as paged_attention_decode (16-bit caches).
 * Supported: head_dim 64 or 128, num_heads / num_kv_heads <= 16; max_q_len up to 65,535
 * query tiles of 8 * floor(32 / G) tokens (G = num_heads / num_kv_heads; EINVAL beyond).
 * The launch stages 96 KiB (head_dim 128) or 32 KiB (64) of LDS per workgroup. The
 * weights enter the value product rounded once to fp16 (relative error at most 2^-11)
 * and V in fp16; with a bf16 cache a second launch on the same stream redoes, with the
 * weights split in two bf16 parts, any workgroup that met a V value of magnitude 2^16 or
 * more (beyond fp16), so the result is defined for every finite input.
 * Errors: EINVAL, ENOTSUP (dtypes, head_dim, group size), EHIP. */
int paged_attention_prefill(void* out, const void* q, int64_t q_stride, const int32_t* q_start,
                            const void* k_cache, const void* v_cache, const int32_t* block_tables,
                            const int32_t* seq_lens, int32_t num_seqs, int32_t max_q_len,
                            int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                            float scale, int32_t in_dtype, int32_t out_dtype, void* stream);

/* copy_blocks: the device half of copy-on-write. For each pair p < n_pairs,
 * (src, dst) = (pairs[2p], pairs[2p + 1]), copy block src onto block dst in the K and
 * the V cache of every layer: block_bytes bytes each, the whole block (the rows past
 * the sequence's length are rewritten before they are read). Pairs with an id outside
 * [0, num_blocks) or src == dst are skipped; two pairs must not share a dst.
 *   k_caches, v_caches: host arrays of num_layers device pointers (16-byte aligned).
 *   pairs: device int32 [n_pairs][2] (kv_pool_append_tokens / _batch_tokens output).
 *   block_bytes: num_kv_heads * BS * head_dim * element bytes (a multiple of 16).
 * Errors: EINVAL (NULLs, alignment, num_layers outside 1..256, block_bytes), EHIP. */
int copy_blocks(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                const int32_t* pairs, int32_t n_pairs, int64_t block_bytes, int64_t num_blocks,
                void* stream);

/* ==== FP8 KV cache ================================================================
 * Storing K and V in FP8 halves the bytes per token, so the same memory holds about
 * twice the context, at some accuracy cost on long contexts ("Yerel LLM sistemlerinde
 * backpressure ve ölçekleme", the paragraph on KV cache quantisation). The page names
 * no format or scaling; here: PKV_FP8_E4M3 codes with one scale per tensor for K
 * (k_scale) and one for V (v_scale), a code c standing for value(c) * scale. Queries,
 * new K/V rows and outputs stay fp16/bf16 (or fp32 out); the layout is the one above
 * with x = 16 (k_cache [num_blocks][Hkv][head_dim/16][BS][16] bytes, v_cache
 * [num_blocks][Hkv][head_dim][BS] bytes). The decode kernels widen the codes to the
 * query type exactly (every e4m3 value is an fp16 and a bf16 value), fold k_scale into
 * the logit scale and v_scale into the output. */

/* reshape_and_cache_fp8: reshape_and_cache into an FP8 cache. Each element x of
 * key (value) is stored as the e4m3 code of the binary32 quotient x / k_scale
 * (x / v_scale), rounded to the nearest finite e4m3 value with ties to the even code:
 * magnitudes above 448 (and infinities) saturate to +-448, NaN gives S.1111.111.
 *   key, value: in_dtype (PKV_F16 or PKV_BF16), strides multiples of 8 elements.
 *   k_scale, v_scale: finite, > 0.
 *   head_dim: a positive multiple of 16.
 * Everything else as reshape_and_cache (its two forms included).
 * Errors: EINVAL, ENOTSUP (in_dtype), EHIP. */
int reshape_and_cache_fp8(const void* key, const void* value, void* k_cache, void* v_cache,
                          const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int64_t num_blocks,
                          int64_t key_stride, int64_t value_stride, int32_t in_dtype,
                          float k_scale, float v_scale, void* stream);

/* paged_attention_decode_fp8: paged_attention_decode over FP8 caches, i.e. with
 * K_b[t] = value(code) * k_scale and V_b[t] = value(code) * v_scale. in_dtype (the
 * query's) is PKV_F16 or PKV_BF16; out_dtype in_dtype or PKV_F32. All three partition
 * modes; the partial results and paged_attention_reduce are unchanged (they already
 * include the scales). Errors as paged_attention_decode, plus EINVAL for a scale that
 * is not finite and positive, ENOTSUP for in_dtype F32. */
int paged_attention_decode_fp8(void* out, float* part_out, float* part_max, float* part_sum,
                               const void* q, int64_t q_stride, const void* k_cache,
                               const void* v_cache, const int32_t* block_tables,
                               const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                               float k_scale, float v_scale, int32_t partition_size,
                               int32_t max_partitions, int32_t in_dtype, int32_t out_dtype,
                               const int32_t* seq_order, void* stream);

/* paged_attention_decode_append_fp8: paged_attention_decode_append over FP8 caches:
 * reshape_and_cache_fp8 of one new row per sequence, then paged_attention_decode_fp8.
 * The new token is attended to as its stored (quantised) value, so the result equals
 * the two calls under the same condition on slot_mapping as
 * paged_attention_decode_append. Fused into the decode launch for partition_size >= 0;
 * a separate cache-write launch with PKV_PARTITION_AUTO. */
int paged_attention_decode_append_fp8(void* out, float* part_out, float* part_max,
                                      float* part_sum, const void* q, int64_t q_stride,
                                      const void* key, const void* value, int64_t key_stride,
                                      int64_t value_stride, const int32_t* slot_mapping,
                                      void* k_cache, void* v_cache, const int32_t* block_tables,
                                      const int32_t* seq_lens, int32_t num_seqs,
                                      int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t max_blocks_per_seq,
                                      int64_t num_blocks, float scale, float k_scale,
                                      float v_scale, int32_t partition_size,
                                      int32_t max_partitions, int32_t in_dtype,
                                      int32_t out_dtype, const int32_t* seq_order, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
