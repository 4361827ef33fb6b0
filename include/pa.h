/*
 * pa.h — PagedAttention decode for AMD MI355X (gfx950): the C ABI of libpa.so.
 *
 * The operations follow the vLLM encyclopedia entry (tonho.wtf): section
 * "como funciona" (KV blocks of a fixed number of tokens, 16 by default; a
 * per-request block table mapping logical to physical blocks with a fill
 * count; a new block only when the previous one is full; reference counts and
 * copy-on-write for parallel samples; everything expressed as fork, append and
 * free; decode attention computed block by block) and section "o que isso
 * custou" (three custom kernels: block write, block read fused with attention,
 * batched block copy).  "KV Cache Administration: PagedAttention &
 * RadixAttention" (techtrendfeed), section "How PagedAttention Works", steps
 * 1-4, and the two other explainers (aitalk.it, briefia.fr) describe the same
 * mechanism with blocks of 16 or 32 tokens.
 *
 * Conventions
 *  - Every entry point returns a pa_status; no exception crosses the ABI.
 *  - Scalar and shape arguments are checked before anything is launched:
 *    PA_ERR_INVALID for null pointers, negative counts, H_q % H_kv != 0, a
 *    partition size that is not a multiple of 32 tokens, too small a workspace;
 *    PA_ERR_UNSUPPORTED for head_dim not in {64, 128}, block_size not in
 *    {16, 32}, or a dtype outside pa_dtype.
 *  - Device entry points take caller-owned device pointers, never allocate or
 *    free device memory, and are asynchronous on `stream` (a hipStream_t passed
 *    as void*; NULL is the default stream).  A launch failure returns
 *    PA_ERR_HIP.  The caller synchronises.
 *  - Element contents (slot values, block-table entries) are the caller's
 *    contract.  Kernels never access memory outside the arrays described by the
 *    size arguments: out-of-range slots and copy pairs are skipped, and
 *    out-of-range block-table entries are read as block 0 (wrong output, no
 *    fault).
 *  - The host pool is single-owner and not thread-safe (one central block
 *    manager, as in the encyclopedia entry's section "como funciona").
 *
 * Cache layout (the pages fix none; this is the library's).  With
 * x = 16 / element_bytes (8 for fp16 and bf16, 4 for fp32), one (block, head)
 * tile is block_size * head_dim contiguous elements, and
 *   K cache [num_blocks][H_kv][head_dim/x][block_size][x]
 *       K(block b, head h, token t, dim i) at [b][h][i/x][r(t)][i%x]
 *       r(t) = (t & 4 ? block_size/2 : 0) + 4*(t >> 3) + (t & 3): inside each
 *       slab the tokens whose index has bit 2 clear come first, in order,
 *       then those with bit 2 set
 *   V cache [num_blocks][H_kv][block_size/x][head_dim][x]
 *       V(block b, head h, token t, dim i) at [b][h][t/x][i][t%x]
 * Both are built from 16-byte vectors: a K vector holds x consecutive dims of
 * one token, a V vector holds x consecutive tokens of one dim, which are the
 * operand shapes of the decode kernel's QK and PV matrix products; the K row
 * order makes each QK operand load read whole 128-byte lines.
 *
 * Slot: slot = physical_block * block_size + offset_in_block.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_pool pa_pool; /* host block pool, below */

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID = 1,
  PA_ERR_UNSUPPORTED = 2,
  PA_ERR_NO_BLOCKS = 3,
  PA_ERR_UNKNOWN_SEQ = 4,
  PA_ERR_HIP = 5,
  PA_ERR_TOO_LARGE = 6 /* beyond pa_decode_noalloc's fixed scratch */
} pa_status;

typedef enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2 } pa_dtype;

/* pa_decode flags */
enum {
  /* Blocks of the batch may be aliased by several sequences (forks, shared
   * prefixes): K/V are read with ordinary cached loads so aliased blocks are
   * served from L2 / Infinity Cache.  Without it K/V are read with
   * non-temporal loads (each block read once per step). */
  PA_DECODE_SHARED_KV = 1
};

/* Static text for a status code; "unknown status" for other values. */
const char* pa_status_str(int status);

/* ABI version of this header (incremented on incompatible change). */
int pa_abi_version(void);

/* ------------------------------------------------------------------------ */
/* Device operations                                                          */
/* ------------------------------------------------------------------------ */

/*
 * pa_write_kv — block write: store the K and V of new tokens into the paged
 * cache (encyclopedia entry, "o que isso custou": the block-write kernel;
 * "como funciona": blocks are filled left to right through the block table).
 *
 *   k_new, v_new  device, [num_tokens][num_kv_heads][head_dim], dtype
 *   k_cache, v_cache  device, layout above, num_blocks blocks
 *   slot_mapping  device, int64 [num_tokens]; token j goes to slot_mapping[j].
 *                 Negative slots and slots >= num_blocks * block_size are
 *                 skipped.  Slots must be distinct (else the winner is
 *                 unspecified).
 * num_tokens == 0 is a no-op.  Bit-exact copy of the element bits.
 */
pa_status pa_write_kv(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                      const int64_t* slot_mapping, int num_tokens, int num_blocks,
                      int num_kv_heads, int head_dim, int block_size, int dtype,
                      void* stream);

/*
 * pa_copy_blocks — batched block copy for copy-on-write (encyclopedia entry,
 * "como funciona": a write into a shared last block copies that block and
 * only it; "o que isso custou": the batched block-copy kernel).
 *
 *   pairs  device, int32 [num_pairs][2] = {src, dst} physical block ids.
 *          For each pair the whole block (all heads, all positions, K and V)
 *          of src is copied to dst.  No dst may equal any src or another dst
 *          of the same call (copies run concurrently).  Pairs with an id
 *          outside [0, num_blocks) are skipped.
 * num_pairs == 0 is a no-op.  Bit-exact.
 */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int num_pairs,
                         int num_blocks, int num_kv_heads, int head_dim, int block_size,
                         int dtype, void* stream);

/*
 * pa_read_probe — a measurement helper, not part of the decode: the read rate
 * the decode's access pattern can reach on this device.  Reads num_tiles
 * tiles of tile_bytes bytes of buf in the order tile_order gives (read i is
 * tile tile_order[i]; entries outside [0, num_tiles) are skipped, so a
 * permutation reads every tile once), with 16-byte loads, non-temporal when
 * nontemporal != 0 as the decode's K/V loads are.  Each of the
 * pa_read_probe_partials() waves of the fixed grid writes the XOR of the
 * 16-byte vectors it read to partials[wave], so the XOR of all partials is the
 * XOR of every tile read.
 *   buf         device memory, num_tiles * tile_bytes bytes, 16-byte aligned
 *   tile_order  device int32 [num_tiles]
 *   partials    device, pa_read_probe_partials() x 16 bytes, 16-byte aligned
 * PA_ERR_INVALID for tile_bytes not a positive multiple of 1024, a negative or
 * larger than INT32_MAX tile count, or a null / misaligned pointer.
 * Asynchronous on `stream`.
 */
int pa_read_probe_partials(void);
pa_status pa_read_probe(const void* buf, int64_t num_tiles, int tile_bytes,
                        const int32_t* tile_order, int nontemporal, void* partials,
                        void* stream);

/*
 * pa_swap_blocks — whole-block copies between two caches of the same
 * geometry, for swapping sequences out to host memory and back (encyclopedia
 * entry, "a ideia": the cache can be swapped to CPU RAM; "como funciona": a
 * preempted sequence returns by swapping in).
 *
 *   src_k, src_v  cache to read, src_blocks blocks, layout above
 *   dst_k, dst_v  cache to write, dst_blocks blocks, same layout
 *   pairs  int32 [num_pairs][2] = {src, dst} block ids (from pa_seq_swap_out
 *          or pa_seq_swap_in).  Pairs outside either cache are skipped; no
 *          dst may repeat within a call.
 * Each of the five arrays may be device memory or pinned host memory
 * (hipHostMalloc); host memory is reached through its device mapping.
 * Anything else (pageable host memory) is PA_ERR_INVALID.  num_pairs == 0 is
 * a no-op.  Bit-exact.  Asynchronous on `stream`: a host cache holds the data
 * once the stream has passed this call.
 */
pa_status pa_swap_blocks(const void* src_k, const void* src_v, int src_blocks, void* dst_k,
                         void* dst_v, int dst_blocks, const int32_t* pairs, int num_pairs,
                         int num_kv_heads, int head_dim, int block_size, int dtype,
                         void* stream);

/*
 * Bytes of workspace pa_decode needs for these sizes; 0 when no sequence can
 * span more than one partition (partition_size == 0 or
 * max_context_len <= partition_size).
 */
size_t pa_decode_workspace_size(int num_seqs, int num_q_heads, int head_dim,
                                int max_context_len, int partition_size);

/*
 * pa_decode — single-query decode attention over block tables (encyclopedia
 * entry, "como funciona": the current token's query times one block's keys
 * gives that slice of the scores, and the output is accumulated against the
 * same block's values; blocks need not be adjacent; "onde isso aparece hoje":
 * K/V shared between query heads as in GQA).
 *
 *   out  device [num_seqs][num_q_heads][head_dim], dtype (written)
 *   q    device [num_seqs][num_q_heads][head_dim], dtype
 *   block_tables  device int32 [num_seqs][max_blocks_per_seq]; entries at
 *        index >= ceil(context_lens[s] / block_size) are never read
 *   context_lens  device int32 [num_seqs]; must be <= max_context_len
 *        (larger values are clamped to it) and <= max_blocks_per_seq*block_size
 *   seq_order  device int32 [num_seqs] or NULL: the order in which sequences
 *        are issued to the GPU (a permutation of 0..num_seqs-1, for example
 *        from pa_decode_order).  A scheduling hint: results do not depend on
 *        it; entries outside [0, num_seqs) are skipped
 *   scale  softmax scale (1/sqrt(head_dim) for standard attention); must be
 *          positive and finite, else PA_ERR_INVALID
 *   partition_size  0: one work unit per (sequence, KV head); otherwise the
 *        context is split into partitions of this many tokens (a multiple of
 *        32) whose partial results (running max, sum, unnormalised output)
 *        are merged by a log-sum-exp reduce in a fixed order
 *   workspace  device, >= pa_decode_workspace_size(...) bytes (may be NULL
 *        when that is 0); contents on entry are ignored
 *   flags  0 or PA_DECODE_SHARED_KV (a cache policy; results are identical)
 *
 * out[s][h] = softmax(scale * q[s][h] . K_s[:, h/G]) V_s[:, h/G], G = H_q/H_kv,
 * where K_s, V_s are the sequence's tokens in logical order.  A sequence with
 * context length 0 gets a zero row.  fp32 accumulation; the PV product of the
 * fp16/bf16 path rounds the softmax weights to the input dtype.  The result is
 * deterministic (no atomics; fixed reduction order).
 */
pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, int max_blocks_per_seq,
                    const int32_t* context_lens, const int32_t* seq_order, int num_seqs,
                    int max_context_len,
                    int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                    int num_blocks, float scale, int partition_size, void* workspace,
                    size_t workspace_bytes, int dtype, int flags, void* stream);

/*
 * pa_decode_noalloc — pa_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, semantics and results as pa_decode
 * (bit-identical: the same kernels), without workspace arguments: the
 * split-K partials go to a device array of PA_NOALLOC_SCRATCH_BYTES (64 MiB)
 * that the library holds on each GPU it runs on until the process ends.  The
 * array's address is looked up once per device, on the first call that needs
 * it with that device current; nothing is allocated or freed, here or later.
 * Make that first call outside graph capture; later calls may be captured
 * into a HIP graph and replayed (the kernels read their inputs and write the
 * array and out at the addresses given at capture).
 *
 * Limit: the call's partials, num_seqs x num_q_heads x slots x
 * (4 x head_dim + 8) bytes with one slot per chunk of partitions that a row
 * spans (at most one per partition), must fit PA_NOALLOC_SCRATCH_BYTES;
 * otherwise PA_ERR_TOO_LARGE and nothing runs.  Any call for which
 * pa_decode_workspace_size() is at most PA_NOALLOC_SCRATCH_BYTES fits (the
 * long-context 70B-class batch of 8 x 64 heads x 131072 tokens in 512-token
 * partitions needs about 11 MB).
 *
 * Every call on one GPU uses that GPU's one array: calls that overlap on a
 * GPU (several streams, several host threads without ordering) race on it
 * and must be serialised by the caller.  Its contents on entry are never
 * read before being written.
 */
#define PA_NOALLOC_SCRATCH_BYTES (64u << 20)
pa_status pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, int max_blocks_per_seq,
                            const int32_t* context_lens, const int32_t* seq_order,
                            int num_seqs, int max_context_len, int num_q_heads,
                            int num_kv_heads, int head_dim, int block_size, int num_blocks,
                            float scale, int partition_size, int dtype, int flags,
                            void* stream);

/*
 * pa_decode_order — the issue order pa_decode_step gives pa_decode (host
 * memory only; no HIP calls).  Sequences whose tables start with the same
 * physical block (forks, shared prefixes) form a group; groups come in
 * decreasing order of their longest context (first appearance breaks ties)
 * and, inside a group, sequences in decreasing context length (index breaks
 * ties).  Keeping sharers together lets a shared block be read from the
 * caches while it is still there; longest first keeps long work from ending
 * the launch.
 *
 *   block_tables  host int32 [num_seqs][max_blocks_per_seq] (entry 0 read
 *                 when context_lens[s] > 0)
 *   context_lens  host int32 [num_seqs]
 *   order_out     host int32 [num_seqs]: a permutation of 0..num_seqs-1
 * PA_ERR_INVALID for negative sizes or a null pointer when num_seqs > 0.
 */
pa_status pa_decode_order(const int32_t* block_tables, int max_blocks_per_seq,
                          const int32_t* context_lens, int num_seqs, int32_t* order_out);

/*
 * Shared-prefix (cascade) decode.  Sequences that hold the same physical
 * blocks for their first L tokens (forks, parallel samples, beams, prefix
 * cache hits; encyclopedia entry, "como funciona": shared prefixes are mapped,
 * not copied) can have that part attended in one pass for all of them: their
 * queries fill two 16-column matrix-core tiles (32 / G sequences of G query
 * heads each; column c: member c / G, query head c % G), so one read of each
 * K/V block serves the whole group.
 * The rest of every context runs as in pa_decode, and the split-K reduce
 * merges both parts.  Same result as pa_decode up to floating-point rounding
 * order.
 *
 * pa_cascade_plan (host memory only): groups sequences whose tables start
 * with the same block (as pa_decode_order); a group's prefix L is the run of
 * identical leading table entries, capped by the shortest member's context,
 * rounded down to a multiple of 32, and kept only when >= max(min_prefix, 32)
 * and the group has two or more members; groups are cut into column groups
 * of 32 / G members (none when G > 16).  Outputs: prefix_len_out[num_seqs]
 * (L, or 0 for sequences outside any group), groups_out[num_seqs][3] =
 * {first member, member count, L}, members_out[num_seqs] (sequence indices),
 * *num_groups_out, *max_prefix_out (largest L), *max_members_out (largest
 * member count) and *max_rest_out (largest context_lens[s] - prefix_len[s]).
 *
 * pa_decode_cascade: pa_decode plus that plan in device memory
 * (num_groups == 0 is plain pa_decode) and its three host values; max_rest
 * must be at least the largest context_lens[s] - prefix_len[s] (the reduce
 * runs only when that part spans several work-groups' worth of partitions).
 * A plan may also be built by hand: every member of a group must hold the
 * group's first member's blocks for its first L tokens, L <= its context, and
 * prefix_len[s] must equal its group's L (0 outside groups).  An L that is
 * not a multiple of 32 is taken rounded down to one; the tokens cut off run
 * with the rest of each context.
 * Groups of at most 16 / G members run one 16-column tile per load, larger
 * ones two.  fp32 runs the plain path.  The workspace must hold
 * pa_decode_cascade_workspace_size(...) bytes, which is non-zero even for an
 * unsplit decode (the two parts meet in the reduce).
 */
pa_status pa_cascade_plan(const int32_t* block_tables, int max_blocks_per_seq,
                          const int32_t* context_lens, int num_seqs, int block_size,
                          int num_q_heads, int num_kv_heads, int min_prefix,
                          int32_t* prefix_len_out, int32_t* groups_out, int32_t* members_out,
                          int* num_groups_out, int* max_prefix_out, int* max_members_out,
                          int* max_rest_out);
size_t pa_decode_cascade_workspace_size(int num_seqs, int num_q_heads, int head_dim,
                                        int max_context_len, int partition_size);
pa_status pa_decode_cascade(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, int max_blocks_per_seq,
                            const int32_t* context_lens, const int32_t* seq_order, int num_seqs,
                            int max_context_len, int num_q_heads, int num_kv_heads,
                            int head_dim, int block_size, int num_blocks, float scale,
                            int partition_size, const int32_t* prefix_len,
                            const int32_t* groups, const int32_t* members, int num_groups,
                            int max_prefix, int max_members, int max_rest, void* workspace,
                            size_t workspace_bytes, int dtype, int flags, void* stream);

/*
 * pa_decode_step — one decode iteration of a batch as the central manager
 * hands it to the GPU (encyclopedia entry, "como funciona": the manager ships
 * the block tables with each iteration's input): append one position to each
 * of seqs[0..num_seqs) in the pool, build slots, copy-on-write pairs, lengths
 * and block tables in `host_staging`, copy them to `dev_staging` with one
 * asynchronous host-to-device copy, then run pa_copy_blocks (if any pair),
 * the block write of k_new / v_new (device [num_seqs][H_kv][d]) into the new
 * positions, and pa_decode of q into out (device [num_seqs][H_q][d]).  The
 * decode issues the sequences in pa_decode_order's order and sets
 * PA_DECODE_SHARED_KV itself whenever the pool holds a block with
 * refcount > 1; then, if the workspace holds
 * pa_decode_cascade_workspace_size(...) bytes, shared prefixes of 512 tokens
 * or more go through the cascade (pa_cascade_plan).
 *
 * For fp16 / bf16 the block write runs inside the decode launch: the wave
 * that ends each context takes the appended token from k_new / v_new for its
 * last group and stores it in its slot (fp32 runs pa_write_kv first).  All
 * work is on `stream`.  Not for graph capture (the pool step runs on the
 * host).
 *
 *   tokens        host int32 [num_seqs] token id of each new position, or NULL;
 *                 with ids the append is pa_seq_append_tokens, so sequences
 *                 that a prefix index tracks keep feeding it (without, it is
 *                 pa_seq_append_batch, which ends that tracking)
 *   host_staging  pinned host memory (hipHostMalloc), >=
 *                 pa_decode_step_staging_size() bytes, 16-byte aligned; a
 *                 small kernel on `stream` reads it through its device
 *                 mapping (an asynchronous copy if it has none), so it must
 *                 not be rewritten until the stream has passed this call
 *                 (alternate two buffers and wait on an event)
 *   dev_staging   device memory of the same size; holds the step's metadata
 *                 until the step's kernels have run
 *   workspace     as for pa_decode, sized for the longest context after the
 *                 append
 * Every argument is checked before the pool changes: on any error status the
 * pool and the device are untouched (PA_ERR_NO_BLOCKS when the pool cannot
 * cover the batch, PA_ERR_INVALID when a table would exceed
 * max_blocks_per_seq or the workspace is too small).  The caller owns all
 * memory; nothing is allocated.
 */
size_t pa_decode_step_staging_size(int num_seqs, int max_blocks_per_seq);
pa_status pa_decode_step(pa_pool* pool, const int64_t* seqs, int num_seqs,
                         const int32_t* tokens, const void* k_new,
                         const void* v_new, void* k_cache, void* v_cache, int num_blocks,
                         int num_kv_heads, int head_dim, int block_size, const void* q,
                         void* out, int num_q_heads, float scale, int partition_size,
                         int max_blocks_per_seq, void* host_staging, void* dev_staging,
                         size_t staging_bytes, void* workspace, size_t workspace_bytes,
                         int dtype, void* stream);

/*
 * pa_beam_decode_step — one beam-search iteration in one call:
 * pa_seq_beam_step(old_beams, parents, new_beams, tokens) in the pool (tokens:
 * host int32 [n_new] or NULL, as there), then, as in
 * pa_decode_step (same staging and fused block write), the staging
 * copy, pa_copy_blocks of its pairs, the block write of k_new / v_new (device
 * [n_new][H_kv][d], in new_beams order) and pa_decode of q into out (device
 * [n_new][H_q][d]).  Staging sized by
 * pa_decode_step_staging_size(n_new, max_blocks_per_seq).  Shapes, buffers,
 * table capacity and workspace are checked before the pool changes; the
 * pool step's own rules (and its PA_ERR_NO_BLOCKS behaviour) are those of
 * pa_seq_beam_step.  n_new == 0 retires the old beams and launches nothing.
 */
pa_status pa_beam_decode_step(pa_pool* pool, const int64_t* old_beams, int n_old,
                              const int64_t* parents, const int64_t* new_beams, int n_new,
                              const int32_t* tokens, const void* k_new, const void* v_new,
                              void* k_cache, void* v_cache,
                              int num_blocks, int num_kv_heads, int head_dim, int block_size,
                              const void* q, void* out, int num_q_heads, float scale,
                              int partition_size, int max_blocks_per_seq, void* host_staging,
                              void* dev_staging, size_t staging_bytes, void* workspace,
                              size_t workspace_bytes, int dtype, void* stream);

/* ------------------------------------------------------------------------ */
/* Host block pool (host memory only; no HIP calls)                          */
/* ------------------------------------------------------------------------ */
/*
 * Policy (the pages give the operations, not an order; this one is fixed so
 * that tables are reproducible): the free list is FIFO, initialised to
 * free_order (or 0..num_blocks-1 when NULL); a block whose refcount drops to
 * zero goes to the back; free releases a sequence's blocks in logical order;
 * an append takes a new block when the sequence's fill is a multiple of
 * block_size, and on its first token copies the last block when that block is
 * partly filled and held by another sequence (the appending sequence copies;
 * the last holder writes in place).  Appends are all-or-nothing.
 */
pa_status pa_pool_create(int num_blocks, int block_size, const int32_t* free_order,
                         pa_pool** out);
void pa_pool_destroy(pa_pool* pool);

/* New empty sequence.  PA_ERR_INVALID if seq_id exists. */
pa_status pa_seq_create(pa_pool* pool, int64_t seq_id);

/* child maps every block of parent (refcount + 1 each) and copies its fill.
 * PA_ERR_UNKNOWN_SEQ if parent is unknown, PA_ERR_INVALID if child exists. */
pa_status pa_seq_fork(pa_pool* pool, int64_t parent, int64_t child);

/*
 * Append num_tokens positions to seq.  slots_out [num_tokens] receives the
 * slot of each new position; pairs_out [1][2] receives at most one
 * {src, dst} copy-on-write pair, *num_pairs_out its count.  The caller must
 * run pa_copy_blocks on the pairs before writing into the returned slots.
 * PA_ERR_NO_BLOCKS leaves the pool unchanged.
 */
pa_status pa_seq_append(pa_pool* pool, int64_t seq, int num_tokens, int64_t* slots_out,
                        int32_t* pairs_out, int* num_pairs_out);

/*
 * Append tokens_each positions to each of seqs[0..n) in that order (ids must be
 * distinct).  slots_out [n][tokens_each]; pairs_out [n][2] (at most one pair
 * per sequence).  All-or-nothing over the whole batch.
 */
pa_status pa_seq_append_batch(pa_pool* pool, const int64_t* seqs, int n, int tokens_each,
                              int64_t* slots_out, int32_t* pairs_out, int* num_pairs_out);

/* Release every block of seq in logical order (host blocks if it is swapped
 * out) and forget seq.  PA_ERR_UNKNOWN_SEQ if seq is unknown. */
pa_status pa_seq_free(pa_pool* pool, int64_t seq);

/*
 * pa_seq_beam_step — one beam-search step (encyclopedia entry, "como
 * funciona": beam candidates share intermediate blocks and the sharing
 * pattern changes every step, like a process tree).  The new beams
 * new_beams[j] become forks of parents[j] (each parent one of old_beams; a
 * parent may have several children or none), then every old beam is freed
 * (new ids may reuse old ids), then one position is appended to each new beam
 * in the order given (pa_seq_append_batch, or pa_seq_append_tokens when
 * tokens[n_new] is not NULL): slots_out [n_new], pairs_out [n_new][2] and
 * *num_pairs_out are its copy-on-write pairs (run pa_copy_blocks before
 * pa_write_kv).  Everything is checked before anything changes
 * (PA_ERR_UNKNOWN_SEQ for an unknown old beam; PA_ERR_INVALID for a repeated,
 * swapped or foreign id); the fork-and-retire part cannot fail after that.  If
 * the append finds too few blocks it returns PA_ERR_NO_BLOCKS with the new
 * beams in place and nothing appended.
 */
pa_status pa_seq_beam_step(pa_pool* pool, const int64_t* old_beams, int n_old,
                           const int64_t* parents, const int64_t* new_beams, int n_new,
                           const int32_t* tokens, int64_t* slots_out, int32_t* pairs_out,
                           int* num_pairs_out);

/*
 * Swapping whole sequences (encyclopedia entry, "como funciona": eviction
 * takes all of a sequence's blocks or none; a preempted sequence returns by
 * swap-in from CPU RAM or by recomputation, the latter being pa_seq_free plus
 * a new prefill).
 *
 * pa_pool_set_host_blocks: give the pool num_host_blocks host block ids
 * [0, num_host_blocks), free list FIFO in increasing order.  Resets the host
 * area; PA_ERR_INVALID while any sequence is swapped out.
 *
 * pa_seq_swap_out: move seqs[0..n) (distinct, not swapped) to host blocks, all
 * or nothing.  Each distinct GPU block that the batch's tables name, in order
 * of first appearance (sequence order, then logical order), gets one host
 * block (blocks shared inside the batch stay shared on the host).  Every table
 * entry then names its host block and gives up its GPU reference, released in
 * the same order.  pairs_out [cap][2] receives {gpu block, host block} per
 * distinct block and *num_pairs_out their count: run pa_swap_blocks(device ->
 * host) with them before anything else writes the released GPU blocks.
 * PA_ERR_NO_BLOCKS (nothing changes) if the host free list is too short;
 * PA_ERR_INVALID if cap is too small, a sequence is already swapped or ids
 * repeat; PA_ERR_UNKNOWN_SEQ for an unknown id (checked first).
 *
 * pa_seq_swap_in: the mirror image for swapped seqs: each distinct host block
 * gets a new GPU block (FIFO; refcount = references from the batch), host
 * references are released in order, pairs_out receives {host block, GPU
 * block}: run pa_swap_blocks(host -> device) before decoding them.
 * PA_ERR_NO_BLOCKS (nothing changes) if the GPU free list is too short.
 *
 * A swapped sequence cannot be appended to, forked or put in
 * pa_pool_block_tables (PA_ERR_INVALID); pa_seq_block_table returns its host
 * block ids; pa_seq_free releases them.
 */
pa_status pa_pool_set_host_blocks(pa_pool* pool, int num_host_blocks);
pa_status pa_seq_swap_out(pa_pool* pool, const int64_t* seqs, int n, int32_t* pairs_out,
                          int cap, int* num_pairs_out);
pa_status pa_seq_swap_in(pa_pool* pool, const int64_t* seqs, int n, int32_t* pairs_out,
                         int cap, int* num_pairs_out);
/* 1 if seq is swapped out, 0 if on the GPU, -1 if unknown. */
int pa_seq_is_swapped(const pa_pool* pool, int64_t seq);
/* stats_out[3] = {free host blocks, host blocks in use, swapped sequences}. */
pa_status pa_pool_host_stats(const pa_pool* pool, int64_t* stats_out);

/* ------------------------------------------------------------------------ */
/* Prefix reuse (host memory only; no HIP calls)                              */
/* ------------------------------------------------------------------------ */
/*
 * An index attached to the pool finds the blocks that already hold a
 * request's prompt prefix, so only the rest is computed (aitalk.it,
 * "RadixAttention: un albero che non dimentica" and the chain-hashing
 * paragraph of "Due strati, non due rivali"; "KV Cache Administration",
 * "How RadixAttention Works", "How vLLM Implements Prefix Caching", "Cache
 * salting prevents cross-tenant reuse").  Both kinds give the same reuse when
 * nothing is evicted; they differ in structure and eviction unit:
 *
 *   PA_PREFIX_HASH   key of block i = SHA-256(key of block i-1 (32 zero bytes
 *                    for i = 0) ‖ LE32(block_size) ‖ token ids as LE32 ‖
 *                    LE32(|e|) ‖ e), where e = LE32(|salt|) ‖ salt ‖ extra
 *                    for block 0 and e = extra after it (pa_prefix_block_hash).
 *                    Eviction: single blocks, least recently idle first,
 *                    deepest first among blocks idle since the same call.
 *   PA_PREFIX_RADIX  compressed trie over token ids at block granularity, one
 *                    root per (salt, extra).  Eviction: whole leaves no
 *                    sequence holds or sits in, least recently used first
 *                    (deeper first among equals); inner nodes go only after
 *                    all their children.
 *
 * The index holds one reference on every block it indexes, so a cached block
 * outlives its requests; it is evicted only when an allocation finds the free
 * list short (pa_pool_stats counts it as used; "shared" counts sequence
 * references only).  Only full blocks are indexed.  A block is indexed as
 * soon as it is full: its K/V must be written (pa_write_kv on the slots
 * returned) before work that reads a later request's hits, which in-order
 * use of one stream gives.
 */
enum { PA_PREFIX_HASH = 1, PA_PREFIX_RADIX = 2 };

/* SHA-256 (FIPS 180-4) of data[0..len) into out[32]. */
pa_status pa_sha256(const void* data, size_t len, uint8_t* out);

/* Chain key of one block (see PA_PREFIX_HASH): parent[32] (NULL = zeros),
 * tokens[n], extra[extra_len] -> out[32]. */
pa_status pa_prefix_block_hash(const uint8_t* parent, const int32_t* tokens, int n,
                               const void* extra, int extra_len, uint8_t* out);

/* Attach an index of `kind` to a pool that has no sequences yet
 * (PA_ERR_INVALID otherwise; PA_ERR_UNSUPPORTED for an unknown kind). */
pa_status pa_pool_enable_prefix_cache(pa_pool* pool, int kind);

/*
 * New sequence for a prompt tokens[0..n): the longest run of its full blocks
 * that ends before its last token and is found in the index is mapped (no K/V
 * to compute; *cached_tokens_out = that run's tokens, a multiple of
 * block_size), fresh blocks are taken for the rest, and slots_out
 * [n - cached] receives the slots of tokens cached..n-1 for pa_write_kv.
 * The new full blocks are indexed.  salt (tenant) and extra (for example an
 * adapter id) are part of every key: different salts never share blocks.
 * All or nothing: PA_ERR_NO_BLOCKS (nothing changes, not even recency) when
 * free plus evictable blocks cannot cover the new blocks; PA_ERR_INVALID
 * without an index or for an existing id.
 */
pa_status pa_seq_create_cached(pa_pool* pool, int64_t seq, const int32_t* tokens, int n,
                               const void* salt, int salt_len, const void* extra, int extra_len,
                               int* cached_tokens_out, int64_t* slots_out);

/*
 * pa_seq_append_batch with token ids tokens[n][tokens_each]: a sequence
 * created by pa_seq_create_cached keeps feeding the index, which indexes each
 * block as it fills.  Plain pa_seq_append_batch, pa_seq_swap_out and
 * pa_seq_free end that tracking for a sequence; pa_seq_fork passes it on.
 */
pa_status pa_seq_append_tokens(pa_pool* pool, const int64_t* seqs, int n, const int32_t* tokens,
                               int tokens_each, int64_t* slots_out, int32_t* pairs_out,
                               int* num_pairs_out);

/* stats_out[6] = {indexed blocks, blocks eviction could free now, blocks
 * found (cumulative), blocks looked up (cumulative), blocks evicted
 * (cumulative), tree nodes (radix; 0 for hash)}; all 0 without an index. */
pa_status pa_prefix_stats(const pa_pool* pool, int64_t* stats_out);

/* Copy seq's block table into out[0..cap); *num_blocks_out, *num_tokens_out get
 * its length and fill (also when cap is too small).  PA_ERR_UNKNOWN_SEQ for an
 * unknown seq; PA_ERR_INVALID if cap is too small (nothing copied). */
pa_status pa_seq_block_table(const pa_pool* pool, int64_t seq, int32_t* out, int cap,
                             int* num_blocks_out, int* num_tokens_out);

/* Dense tables for a batch: out [n][maxb] padded with -1, lens_out [n].
 * PA_ERR_UNKNOWN_SEQ for an unknown sequence; PA_ERR_INVALID for a swapped-out
 * one or a table longer than maxb. */
pa_status pa_pool_block_tables(const pa_pool* pool, const int64_t* seqs, int n, int32_t* out,
                               int maxb, int32_t* lens_out);

/* Refcount of a physical block, or -1 if out of range. */
int pa_pool_refcount(const pa_pool* pool, int32_t block);

/* Current free list, front first: out[0..cap), *n_out = its length (also
 * when cap is too small, which returns PA_ERR_INVALID and copies nothing). */
pa_status pa_pool_free_list(const pa_pool* pool, int32_t* out, int cap, int* n_out);

/* stats_out[5] = {free blocks, used blocks, shared blocks (refcount > 1),
 * tokens held by live sequences, copy-on-write pairs issued so far}.
 * PA_ERR_INVALID for a null pointer. */
pa_status pa_pool_stats(const pa_pool* pool, int64_t* stats_out);

/*
 * Per-token KV bytes: 2 (K and V) x layers x KV heads x head_dim x element
 * bytes (encyclopedia entry, "o problema": the OPT-13B case; briefia.fr,
 * section "L'ampleur du cache KV": the factors).  0 for a bad dtype.
 */
size_t pa_kv_bytes_per_token(int num_layers, int num_kv_heads, int head_dim, int dtype);

#ifdef __cplusplus
}
#endif
#endif /* PA_H */
