/*
 * pagedkv.h - C ABI of libpagedkv: paged KV-cache decode attention, cache writes
 * and a host-side block allocator for AMD Instinct MI355X (gfx950).
 *
 * Sources for what is computed (restated, not quoted):
 *   [P1] ksqn.cn "大模型推理性能优化：PagedAttention与Continuous Batching原理与实践"
 *   [P2] hihuo.com "vLLM 原理：PagedAttention 和 Continuous Batching"
 *   [P3] blog.gitcode.com "如何通过PagedAttention实现LLM高性能推理：实战指南"
 *
 * Every symbol is extern "C"; arguments are plain pointers, integers and one
 * small descriptor struct.  Device pointers are HIP device addresses owned by
 * the caller; `stream` is a hipStream_t passed as void* (NULL = the default
 * stream).  Device calls only enqueue work on that stream and return; the
 * library never allocates, frees or synchronises device memory.
 *
 * Errors: every call returns pa_status (or a documented sentinel) and never
 * aborts.  Host validation covers what the host can see: null pointers,
 * negative sizes, unsupported shapes, 16-byte alignment, workspace size,
 * 32-bit index range.  Values that only the device sees (block IDs, slots,
 * context lengths) are preconditions; a violation gives unspecified results
 * but never an out-of-bounds access: the kernels clamp or skip such entries
 * as stated per call.  A launch failure returns PA_ERR_HIP.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = 1,  /* null pointer, negative size, misalignment, bad struct field */
    PA_ERR_UNSUPPORTED = 2,  /* valid request outside the compiled shapes / dtypes        */
    PA_ERR_OOM = 3,          /* allocator: not enough free blocks; state unchanged          */
    PA_ERR_STATE = 4,        /* allocator: unknown / duplicate / already-freed sequence     */
    PA_ERR_HIP = 5,          /* a HIP runtime call or kernel launch failed                  */
    PA_ERR_TOO_LARGE = 6     /* the request needs more than a fixed-size static buffer holds */
} pa_status;

typedef enum pa_dtype { PA_DTYPE_F32 = 0, PA_DTYPE_BF16 = 1 } pa_dtype;

/*
 * The physical cache: one K array and one V array, each holding num_blocks
 * blocks of block_size token slots for num_kv_heads heads of head_dim values
 * ([P1] section 2.2: fixed-size pages scattered through one pool; [P2]
 * PagedAttention > 工作原理 > 1. 页表管理: a per-sequence page table).
 *
 * Supported: block_size in {8, 16, 32, 64}; head_dim in {64, 128}; dtype in
 * {F32, BF16}.  Smaller blocks waste fewer slots at
 * sequence ends but mean more table entries per token ([P1] section 3.4 on
 * --block-size).
 *
 * Layout (the library's own choice; the pages fix only the logical picture).
 * Let s = element bytes, X = 16 / s (elements per 16-byte group), E = X / 4,
 * TT = min(block_size, 16) tokens per tile, TPB = block_size / TT.  A block is
 * cut into TPB tiles of TT tokens; tiles are ordered block -> tile -> kv head
 * (the Hkv heads' tiles of one tile slot are adjacent), each tile holding
 * TT * head_dim elements.  Element (block b, head h, token slot o, dim d) sits at
 *
 *   K: ((((b*TPB + o/TT)*Hkv + h)*(D/X) + d/X)*TT + o%TT)*X + d%X
 *   V: ((b*TPB + o/TT)*Hkv + h)*TT*D
 *      + ((((d/(16E))*(TT/4) + (o%TT)/4)*16 + d%16)*E + (d/16)%E)*4 + o%4
 *
 * so a K 16-byte group is X consecutive dims of one token, and a V 16-byte
 * group is 4 consecutive tokens of E dims spaced 16 apart.  One wavefront
 * reading a 16-token tile with one 16-byte load per lane per 1 KiB touches one
 * contiguous KiB per instruction (with blocks of 8, two runs of 512 bytes, one
 * per block).
 *
 * A slot is b * block_size + o.  Bytes per array: pa_cache_bytes().
 */
typedef struct pa_cache_desc {
    int32_t num_blocks;    /* N > 0                                   */
    int32_t block_size;    /* B: 8, 16, 32 or 64 tokens per block     */
    int32_t num_kv_heads;  /* Hkv > 0                                 */
    int32_t head_dim;      /* D: 64 or 128                            */
    int32_t dtype;         /* pa_dtype                                */
} pa_cache_desc;

/* Human-readable name of a status code (static storage; never NULL). */
const char* pa_status_string(pa_status s);

/* ABI version of this header: (major << 16) | minor. */
int32_t pa_abi_version(void);

/* Bytes of ONE cache array (K or V) for the descriptor; 0 if the descriptor is invalid. */
size_t pa_cache_bytes(const pa_cache_desc* desc);

/*
 * pa_reshape_and_cache - write new tokens' keys and values into their slots.
 *
 * The scatter that pairs with the attention gather ([P1] section 2.2) and the
 * cache update after each forward step ([P2] 调度流程, step 4).
 *   k, v          device, [num_tokens, Hkv, D] row-major, dtype of the cache, 16-B aligned
 *   slot_mapping  device, [num_tokens] int64; slot = block * B + offset; -1 = skip
 *   k_cache, v_cache  device, the cache arrays (layout above), 16-B aligned
 * Token t's bits are copied unchanged; every other byte of the cache is left
 * as it was.  Preconditions: no two tokens share a non-negative slot; slots
 * are < N * B (larger slots are skipped).  num_tokens == 0 is a no-op.
 */
pa_status pa_reshape_and_cache(const pa_cache_desc* desc, const void* k, const void* v,
                               const int64_t* slot_mapping, int32_t num_tokens,
                               void* k_cache, void* v_cache, void* stream);

/*
 * pa_copy_blocks - copy whole physical blocks (K and V, every head and slot).
 *
 * Used for copy-on-write of a block shared between sequences ([P2]
 * PagedAttention > 优势 > 3. 支持共享 names the sharing; the copy before a write
 * is this library's reading).
 *   pairs  device, [num_pairs][2] int32 (src, dst)
 * Pairs run concurrently: no block may be the dst of one pair and the src or
 * dst of another.  Pairs with an ID outside [0, N) are skipped.
 */
pa_status pa_copy_blocks(const pa_cache_desc* desc, void* k_cache, void* v_cache,
                         const int32_t* pairs, int32_t num_pairs, void* stream);

/*
 * pa_update_block_tables - apply (row, column, block) updates to a device
 * block-table array [rows][max_blocks_per_seq] int32.
 *   updates  device, [num_updates][3] int32; entries with row or column out of
 *            range are skipped.  Later duplicates of one (row, column) race.
 * Lets a caller keep the tables resident in HBM and send only the entries the
 * allocator changed in a step ([P2] 工作原理 > 2. 按需分配: a new page only when a
 * token crosses a page boundary).
 */
pa_status pa_update_block_tables(int32_t* block_tables, int32_t num_rows,
                                 int32_t max_blocks_per_seq, const int32_t* updates,
                                 int32_t num_updates, void* stream);

/*
 * pa_append_tokens - every write of one decode step: the copy-on-write block
 * copies, the block-table updates, the new tokens' scatter (the writes that
 * follow each forward step, [P2] 调度流程 step 4; the sharing that copy-on-write
 * preserves, [P2] 优势 > 3. 支持共享) and the upload of the context lengths the
 * next decode call reads.  One launch when cow_pairs is NULL; with cow_pairs the
 * copies run as a first launch, so pass NULL for a step that copies nothing.
 *   k, v, slot_mapping, num_tokens   as for pa_reshape_and_cache
 *   cow_pairs      [num_tokens][2] int32 (src, dst) or NULL: before token t is
 *                  written, block src is copied onto block dst (whole block, K and
 *                  V); (-1, -1) or an ID outside [0, N) = no copy
 *   block_tables   device, [num_rows][max_blocks_per_seq] int32, updated in place
 *   table_updates  [num_updates][3] int32 (row, column, block) or NULL; entries
 *                  outside the table are skipped; no two may name one entry
 *   lens_in, lens_out, num_lens   lens_out[i] = lens_in[i] for i < num_lens
 *                  (lens_out device; NULL/0 = nothing)
 * slot_mapping, cow_pairs, table_updates and lens_in may be device memory or
 * pinned host memory (each element is read once), so a step's host-built
 * metadata needs no separate copy.  The result equals pa_copy_blocks (all valid
 * pairs), pa_update_block_tables, then pa_reshape_and_cache, under those calls'
 * preconditions; any number of a sequence's tokens may be written in one call.
 */
pa_status pa_append_tokens(const pa_cache_desc* desc, const void* k, const void* v,
                           const int64_t* slot_mapping, const int32_t* cow_pairs,
                           int32_t num_tokens, void* k_cache, void* v_cache,
                           int32_t* block_tables, int32_t num_rows, int32_t max_blocks_per_seq,
                           const int32_t* table_updates, int32_t num_updates,
                           const int32_t* lens_in, int32_t* lens_out, int32_t num_lens,
                           void* stream);

/* Decode flags (the `flags` argument of the pa_paged_attn_decode calls). */
enum {
    /* Read K/V tiles with ordinary loads, which keep them in L2 and the
     * last-level cache.  Set it when blocks are shared between the batch's
     * sequences (a forked or prefix-cached prompt), so that a shared block is
     * read from HBM once per call.  Without it tiles are read with
     * non-temporal loads, which do not displace cached data and stream a
     * batch of private contexts faster. */
    PA_DECODE_KEEP_CACHED = 1
};

/*
 * Decode attention.
 *
 * For each sequence i and query head j, with L = context_lens[i],
 * G = Hq / Hkv and kv head h = j / G:
 *   out[i, j, :] = sum_t softmax_t(scale * <q[i,j,:], K_i[t,h,:]>) * V_i[t,h,:]
 * over t < L, where K_i[t] / V_i[t] are read from block block_tables[i][t / B],
 * slot t % B ([P1] sections 2 and 2.2: decode attends over every cached token
 * of the sequence, gathered from its scattered blocks; section 2.3 item 3:
 * ragged lengths).  L == 0 gives zeros.  No causal, sliding or bias mask.
 * scale is any finite value (zero gives uniform weights over the L tokens; a
 * negative scale is accepted); NaN or infinity gives PA_ERR_INVALID_ARG.
 *
 *   out            device, [num_seqs, Hq, D], dtype of the cache, 16-B aligned
 *   q              device, [num_seqs, Hq, D], dtype of the cache, 16-B aligned
 *   block_tables   device, [num_seqs, max_blocks_per_seq] int32; only columns
 *                  < ceil(L / B) are read (others may hold anything)
 *   context_lens   device, [num_seqs] int32; values are clamped to
 *                  [0, max_blocks_per_seq * B]
 *   num_units      number of work units the tiles of the batch are split into
 *                  (each unit is one wavefront); 0 = a default sized to the GPU.
 *                  The split decides the order of floating-point reductions,
 *                  so results are bit-reproducible for a given
 *                  (context_lens, num_units) and independent of block IDs.
 *   flags          0 or PA_DECODE_KEEP_CACHED; other bits give
 *                  PA_ERR_INVALID_ARG.  Results do not depend on it.
 *   workspace      device scratch of at least pa_decode_workspace_bytes()
 *                  bytes, 16-B aligned, owned by the caller.  It holds partial
 *                  results and, in its last 4 * num_units bytes, one arrival
 *                  count per unit.  Zero-fill it once after allocating it: the
 *                  counts must be zero when a call starts, and every completed
 *                  pa_paged_attn_decode call leaves them zero.  Pass the same
 *                  workspace_bytes on every call that uses one workspace (the
 *                  counts are found from its end), and order those calls on one
 *                  stream.  _partial and _merge below never touch the counts and
 *                  need no initial contents.
 * Block IDs outside [0, N) in a column that is read are replaced by 0.
 * Supported: bf16 with G in {1, 2, 4, 8, 16}; f32 with any G.  Outputs are
 * rounded to the output dtype nearest-even from fp32 accumulators.
 */
size_t pa_decode_workspace_bytes(const pa_cache_desc* desc, int32_t num_q_heads,
                                 int32_t num_units);

/* The num_units the library uses for num_units == 0 on the current device. */
int32_t pa_decode_default_units(void);

pa_status pa_paged_attn_decode(const pa_cache_desc* desc, void* out, const void* q,
                               const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* context_lens,
                               int32_t num_seqs, int32_t num_q_heads,
                               int32_t max_blocks_per_seq, float scale, int32_t num_units,
                               void* workspace, size_t workspace_bytes, uint32_t flags,
                               void* stream);

/*
 * pa_paged_attn_decode enqueues one kernel.  It gathers and attends: each wave
 * takes a range of 16-token tiles.  A row is a kv head (bf16 with G > 1) or a
 * query head (otherwise).  With num_units >= rows every row is cut into the
 * same num_units / rows ranges, of equal cost where a sequence costs its tile
 * count plus one; with fewer units the batch's tiles, row after row, are cut
 * into num_units ranges of equal tile count.  A wave writes the sequences it
 * holds whole to `out` and leaves partial (max, sum, accumulator) records for
 * sequences cut by range ends.  The holder of a cut sequence's pieces that
 * finishes last (found with the workspace's arrival counts) merges the records
 * with the log-sum-exp rule, in piece order ([P1] section 2.2 names only the
 * gather; the split and the merge are this library's).
 *
 * The same work as two kernels, same arguments: _partial (gather and attend,
 * records only) then _merge (a second kernel merges every cut sequence) on one
 * stream gives outputs bit-identical to pa_paged_attn_decode; it lets a caller
 * time the stages apart.
 */
pa_status pa_paged_attn_decode_partial(const pa_cache_desc* desc, void* out, const void* q,
                                       const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, const int32_t* context_lens,
                                       int32_t num_seqs, int32_t num_q_heads,
                                       int32_t max_blocks_per_seq, float scale,
                                       int32_t num_units, void* workspace,
                                       size_t workspace_bytes, uint32_t flags, void* stream);
pa_status pa_paged_attn_decode_merge(const pa_cache_desc* desc, void* out, const void* q,
                                     const void* k_cache, const void* v_cache,
                                     const int32_t* block_tables, const int32_t* context_lens,
                                     int32_t num_seqs, int32_t num_q_heads,
                                     int32_t max_blocks_per_seq, float scale, int32_t num_units,
                                     void* workspace, size_t workspace_bytes, uint32_t flags, void* stream);

/*
 * pa_decode_step - one decode step of a layer in one launch: the writes of
 * pa_append_tokens and the attention of pa_paged_attn_decode together.  After
 * each forward step every running sequence appends its new token and the next
 * step attends over it ([P2] 调度流程; [P1] section 2: decode runs one step per
 * token and is the bottleneck), so both happen every step; here the token is
 * taken into attention straight from k_new / v_new and written to the cache by
 * the same waves that read its tile, with no separate write launch.
 *   k_new, v_new   device, [num_seqs, Hkv, D]: sequence i's new token (position
 *                  lens_in[i] - 1), dtype of the cache, 16-B aligned
 *   slot_mapping   [num_seqs] int64, device or pinned host: the slot of that
 *                  position (its offset must be (lens_in[i] - 1) % B); -1 = the
 *                  sequence writes no token this step (attended as cached)
 *   cow_pairs      [num_seqs][2] int32 (src, dst) or NULL, device or pinned host:
 *                  sequence i's last block is copied from src onto dst (= the
 *                  block of its slot) before its token is written; (-1, -1) = none
 *   lens_in        [num_seqs] int32, device or pinned host: context lengths
 *                  including the new token; copied into context_lens
 *   block_tables, context_lens   device, as in pa_paged_attn_decode; updated in
 *                  place: block_tables[i][(lens_in[i] - 1) / B] = slot / B and
 *                  context_lens = lens_in, as the next call expects them
 *   workspace      pa_decode_step_workspace_bytes(desc, Hq, num_units, num_seqs)
 *                  bytes, zero-filled once (the same rules as for
 *                  pa_paged_attn_decode's workspace; a workspace sized for the
 *                  step also serves pa_paged_attn_decode with the same bytes)
 * Results: cache bytes, tables and lengths equal those of pa_append_tokens(k_new,
 * v_new, slot_mapping, cow_pairs, the table entries above, lens_in -> context_lens)
 * and out equals, bit for bit, the pa_paged_attn_decode call that follows it
 * (same num_units and flags).  Inside the launch, workgroup 0 writes the lengths
 * and table entries and every other workgroup waits (bounded) until it has; other
 * arguments and errors as in pa_paged_attn_decode.
 */
size_t pa_decode_step_workspace_bytes(const pa_cache_desc* desc, int32_t num_q_heads,
                                      int32_t num_units, int32_t num_seqs);
pa_status pa_decode_step(const pa_cache_desc* desc, void* out, const void* q, const void* k_new,
                         const void* v_new, const int64_t* slot_mapping, const int32_t* cow_pairs,
                         const int32_t* lens_in, void* k_cache, void* v_cache,
                         int32_t* block_tables, int32_t* context_lens, int32_t num_seqs,
                         int32_t num_q_heads, int32_t max_blocks_per_seq, float scale,
                         int32_t num_units, void* workspace, size_t workspace_bytes,
                         uint32_t flags, void* stream);

/*
 * pa_paged_attn_decode_noalloc - pa_paged_attn_decode for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc.  It takes no workspace: partial records and
 * arrival counts live in one static device buffer of the library,
 * PA_DECODE_NOALLOC_SCRATCH_BYTES bytes per GPU, held until the process ends.
 * Arguments, results (bit for bit, for the same num_units) and errors are those of
 * pa_paged_attn_decode, plus:
 *   - PA_ERR_TOO_LARGE when pa_decode_workspace_bytes(desc, num_q_heads,
 *     num_units) exceeds the buffer (nothing is launched then);
 *   - the first call on a device looks the buffer up (hipGetSymbolAddress) and
 *     zero-fills it with a kernel on `stream`; no call allocates or frees memory;
 *   - every call on one GPU shares that GPU's buffer: calls that overlap in time
 *     on one GPU (different streams, threads or processes' graphs) race and give
 *     unspecified results.  Calls ordered on one stream are safe; each completed
 *     call leaves the arrival counts at zero for the next.
 */
#define PA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
pa_status pa_paged_attn_decode_noalloc(const pa_cache_desc* desc, void* out, const void* q,
                                       const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, const int32_t* context_lens,
                                       int32_t num_seqs, int32_t num_q_heads,
                                       int32_t max_blocks_per_seq, float scale,
                                       int32_t num_units, uint32_t flags, void* stream);

/*
 * Chunked-prefill attention over the paged cache.
 *
 * The prompt is processed in one pass before decoding ([P1] section 2), long
 * prompts a chunk at a time; generation is autoregressive, so a prompt token
 * attends to itself and to every earlier token ([P1] section 2.1).  Sequence s
 * brings c_s = query_start[s+1] - query_start[s] query rows (its chunk) and holds
 * L_s = context_lens[s] >= c_s tokens in the cache, the chunk's own keys and
 * values last (write them first with pa_reshape_and_cache).  Chunk token i sits
 * at position L_s - c_s + i:
 *   out[row, j, :] = sum_{p <= L_s - c_s + i} softmax_p(scale * <q[row, j], K_p>) V_p
 * with row = query_start[s] + i, query head j reading KV head j / G.
 *
 *   out, q         device, [num_tokens, Hq, D] row-major, bf16, 16-B aligned
 *   block_tables   device, [num_seqs, max_blocks_per_seq] int32 (as in decode)
 *   query_start    device, [num_seqs + 1] int32, non-decreasing, 0 <= values
 *                  <= num_tokens; sequences with c_s = 0 are skipped
 *   context_lens   device, [num_seqs] int32, clamped to [0, max_blocks_per_seq * B]
 *   max_query_len  host; every c_s must be <= it (it sizes the grid: rows past
 *                  it may be left unwritten)
 * scale: any finite value, zero and negative included (NaN or infinity gives
 * PA_ERR_INVALID_ARG).
 * Rows of a chunk longer than its cache (positions below 0) are written as
 * zeros; rows whose query_start entries are out of range are not written.
 * Block IDs outside [0, N) in a column that is read are replaced by 0.
 * Supported: bf16 with G in {1, 2, 4, 8, 16} and D in {64, 128}
 * (PA_ERR_UNSUPPORTED otherwise).  Accumulation is fp32, P is rounded to bf16
 * before the PV product, and outputs are rounded nearest-even.  No workspace.
 * A row's bits do not depend on how its prompt is cut into chunks, nor on the
 * other rows or sequences of the call; a NaN in a visible key, value or query
 * propagates to the row.
 */
pa_status pa_paged_attn_prefill(const pa_cache_desc* desc, void* out, const void* q,
                                const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, const int32_t* query_start,
                                const int32_t* context_lens, int32_t num_seqs,
                                int32_t num_tokens, int32_t num_q_heads,
                                int32_t max_blocks_per_seq, int32_t max_query_len, float scale,
                                void* stream);

/*
 * Whole-block copies between two pools of the same block geometry (desc's
 * num_kv_heads, block_size, head_dim, dtype; desc->num_blocks is not used):
 * for k < num_pairs, block pairs[2k] of (src_k, src_v), a pool of src_blocks
 * blocks, is copied onto block pairs[2k+1] of (dst_k, dst_v), a pool of
 * dst_blocks blocks.  Either pool may be device memory or pinned host memory
 * (hipHostMalloc / torch pin_memory); pairs may be device or pinned host
 * memory.  Pairs naming a block outside its pool are skipped.  Destination
 * blocks must be distinct and must not be sources of the same call.  This is
 * the data half of swapping (pa_seq_swap_out / pa_seq_swap_in give the pairs).
 */
pa_status pa_swap_blocks(const pa_cache_desc* desc, const void* src_k, const void* src_v,
                         int32_t src_blocks, void* dst_k, void* dst_v, int32_t dst_blocks,
                         const int32_t* pairs, int32_t num_pairs, void* stream);

/*
 * Host block allocator ("block manager", [P1] section 2.2; sample structure in
 * [P3] section 2.2).  Host memory only; not thread-safe; one instance per
 * cache.  Semantics:
 *   - free blocks form a FIFO queue, initialised from initial_free_order
 *     (a permutation of 0..N-1) or 0..N-1 when it is NULL;
 *   - add(seq, n): a new sequence holds ceil(n / B) blocks taken from the head
 *     of the queue ([P2] PagedAttention 的思路: 500 tokens -> 32 pages);
 *     all-or-nothing: PA_ERR_OOM leaves the state unchanged;
 *   - append(seq): reserve the slot of the next token; a new block is taken
 *     only when the token falls past the last block ([P2] 工作原理 > 2.
 *     按需分配); when the target block is held by more than one sequence the
 *     writer moves to a fresh block and (cow_src, cow_dst) name the block
 *     copy the caller must do first (copy-on-write); otherwise -1, -1;
 *   - fork(parent, child): child shares all of parent's blocks ([P2]
 *     优势 > 3. 支持共享: parallel sampling and beam search);
 *   - free(seq): drop one reference per block in logical order; blocks that
 *     reach zero join the tail of the queue ([P2] 工作原理 > 3. 及时释放).
 * Sequence IDs are arbitrary int64 values.  PA_ERR_STATE: unknown seq, a seq
 * that already exists (add, fork child).  State is unchanged by any error.
 */
typedef struct pa_allocator pa_allocator;

pa_status pa_alloc_create(int32_t num_blocks, int32_t block_size,
                          const int32_t* initial_free_order, pa_allocator** out);
void      pa_alloc_destroy(pa_allocator* a);
int32_t   pa_alloc_num_free(const pa_allocator* a);                       /* -1 if a == NULL */
int32_t   pa_alloc_num_seqs(const pa_allocator* a);                       /* -1 if a == NULL */
int32_t   pa_alloc_refcount(const pa_allocator* a, int32_t block);        /* -1 if out of range */
/* Copy the free queue, head first, into out[0..cap); *n = its full length. */
pa_status pa_alloc_free_list(const pa_allocator* a, int32_t* out, int32_t cap, int32_t* n);

pa_status pa_seq_add(pa_allocator* a, int64_t seq, int32_t num_tokens);
pa_status pa_seq_append(pa_allocator* a, int64_t seq, int64_t* slot,
                        int32_t* cow_src, int32_t* cow_dst);
/*
 * Append one token to each of seqs[0..n) in order.  slots[k] and
 * cow_pairs[2k], cow_pairs[2k+1] receive the k-th result (-1, -1 when no
 * copy is needed); new_blocks[k] is the block newly placed in the k-th
 * sequence's table (a fresh page or a copy-on-write target), else -1, and
 * new_cols[k] its table column.  Stops at the first failure:
 * *num_done = appends completed (earlier ones stay applied), and the status
 * is that of the failing append (PA_ERR_OOM / PA_ERR_STATE).
 */
pa_status pa_seq_append_batch(pa_allocator* a, const int64_t* seqs, int32_t n, int64_t* slots,
                              int32_t* cow_pairs, int32_t* new_blocks, int32_t* new_cols,
                              int32_t* num_done);
pa_status pa_seq_fork(pa_allocator* a, int64_t parent, int64_t child);
pa_status pa_seq_free(pa_allocator* a, int64_t seq);
/* Slots of positions start .. start+count-1 (must lie inside the sequence). */
pa_status pa_seq_slots(const pa_allocator* a, int64_t seq, int32_t start, int32_t count,
                       int64_t* out);
pa_status pa_seq_info(const pa_allocator* a, int64_t seq, int32_t* num_tokens,
                      int32_t* num_blocks);
/* Copy the block table (logical order) into out[0..cap); PA_ERR_INVALID_ARG if cap is short. */
pa_status pa_seq_block_table(const pa_allocator* a, int64_t seq, int32_t* out, int32_t cap);
/*
 * Decode metadata for seqs[0..n): block_tables [n][max_blocks_per_seq]
 * (unused columns set to -1) and context_lens [n] (host arrays).
 * PA_ERR_INVALID_ARG if a table is longer than max_blocks_per_seq.
 */
pa_status pa_batch_metadata(const pa_allocator* a, const int64_t* seqs, int32_t n,
                            int32_t max_blocks_per_seq, int32_t* block_tables,
                            int32_t* context_lens);

/*
 * Prefix caching: prompts that open with the same tokens share those tokens'
 * pages instead of computing them again ([P2] 优势 > 3. 支持共享; [P1] sections
 * 3.4 and 5.2 item 4).  The pages give no mechanism; this one:
 *   - a full block is identified by key_i = FNV-1a-64(le64(key_{i-1}) ||
 *     le32(its B tokens)), key_{-1} = 0 (equal keys are taken as equal
 *     prefixes; a 64-bit collision would share a wrong block);
 *   - add_prefix(seq, tokens, n) admits a prompt of n tokens: its leading full
 *     blocks whose keys are cached are reused (reference + 1; a cached block
 *     with no holder leaves the free queue), never the block of token n - 1,
 *     and the rest is taken from the queue as in add.  *num_cached_tokens =
 *     reused blocks * B: those tokens' K/V are already in the cache.  OOM when
 *     the queue, less the reused blocks in it, is short; nothing changes then;
 *   - register_blocks(seq, tokens, n): tokens are the sequence's first n tokens
 *     (n <= its length) and their K/V are written.  Each full block among them
 *     is considered once per sequence, in order: it becomes the cached block
 *     for its key unless that key is cached already (the duplicate stays
 *     uncached).  A forked child inherits its parent's progress;
 *   - a cached block whose last holder lets go joins the free queue's tail
 *     like any block and stays findable; any allocation that takes it from
 *     the head evicts it (its key is forgotten).
 * Calls that pass no tokens (pa_seq_add, appends) never look blocks up.
 */
pa_status pa_seq_add_prefix(pa_allocator* a, int64_t seq, const int32_t* tokens,
                            int32_t num_tokens, int32_t* num_cached_tokens);
pa_status pa_seq_register_blocks(pa_allocator* a, int64_t seq, const int32_t* tokens,
                                 int32_t num_tokens);
/*
 * Swapping ([P2] Preemption（抢占）: Recompute or Swap, "move the KV cache to the
 * CPU"; [P1] section 3.4 on --swap-space).  A host pool of num_host_blocks
 * blocks (its own FIFO queue, IDs 0..n-1, initially empty pool) holds swapped
 * sequences; the caller owns the host memory and copies with pa_swap_blocks.
 *   - set_host_pool: (re)size the host pool; PA_ERR_STATE while any sequence is
 *     swapped out;
 *   - swap_out(seq): all-or-nothing; takes one host block per table entry from
 *     the host queue's head and writes (device block, host block) pairs in
 *     logical order into pairs[2k], pairs[2k+1]; the device references are
 *     dropped as in free (a shared block stays for its other holders).  The
 *     sequence keeps its length and prefix-cache progress;
 *   - swap_in(seq): all-or-nothing; fresh device blocks from the queue's head
 *     (evicting cached blocks as any allocation does), (host block, device
 *     block) pairs in logical order; the host blocks return to the host queue's
 *     tail in logical order;
 *   - a swapped sequence accepts only swap_in, free (its host blocks return),
 *     seq_info and is_swapped; everything else returns PA_ERR_STATE.
 * PA_ERR_INVALID_ARG when cap is below the sequence's block count.
 */
pa_status pa_alloc_set_host_pool(pa_allocator* a, int32_t num_host_blocks);
int32_t   pa_alloc_num_free_host(const pa_allocator* a);             /* -1 if a == NULL */
/* Copy the host queue, head first, into out[0..cap); *n = its full length. */
pa_status pa_alloc_host_free_list(const pa_allocator* a, int32_t* out, int32_t cap, int32_t* n);
/* A swapped sequence's host blocks in logical order (PA_ERR_STATE if not swapped). */
pa_status pa_seq_host_blocks(const pa_allocator* a, int64_t seq, int32_t* out, int32_t cap);
int32_t   pa_seq_is_swapped(const pa_allocator* a, int64_t seq);     /* 1, 0, or -1 if unknown */
pa_status pa_seq_swap_out(pa_allocator* a, int64_t seq, int32_t* pairs, int32_t cap,
                          int32_t* num_pairs);
pa_status pa_seq_swap_in(pa_allocator* a, int64_t seq, int32_t* pairs, int32_t cap,
                         int32_t* num_pairs);

/* Blocks looked up and reused by add_prefix so far, and blocks cached now. */
pa_status pa_alloc_prefix_stats(const pa_allocator* a, int64_t* lookups, int64_t* hits,
                                int32_t* cached_blocks);
/* 1 and *key when the block is cached, 0 when not, -1 if out of range. */
int32_t   pa_alloc_block_cached(const pa_allocator* a, int32_t block, uint64_t* key);

/*
 * Continuous-batching scheduler: the host side of a serving loop over its own
 * allocator ([P2] vLLM 的调度 > 调度流程 and Preemption（抢占）; [P1] section 2.3).
 * Each pa_sched_step, in this order:
 *   1. requests that have produced their whole output release their blocks;
 *   2. the requests added since the last step join the waiting queue's tail;
 *   3. swapped-out requests come back first, in swap-out order, while their blocks fit;
 *   4. waiting requests are admitted first come, first served while the whole
 *      prompt fits (the first that does not fit blocks the queue; none is admitted
 *      while a swapped request waits); with prefix caching, admission reuses the
 *      cached full blocks of the prompt's opening and prefill starts after them;
 *   5. every request whose prompt was complete before this step appends one
 *      decode token, in running order; when no block is free the running request
 *      admitted last is preempted (it may be the requester): swapped out when the
 *      host pool holds its blocks, else freed and queued at the waiting queue's
 *      head to recompute its prompt plus the tokens it has generated;
 *   6. every running request whose prompt is not fully written gets its next chunk
 *      of at most `chunk` prompt tokens, in running order (after the appends, so a
 *      request preempted in this step holds no chunk of it); with prefix caching
 *      each chunk's full blocks are then offered to the cache;
 *   7. with prefix caching, each decode token that completes a block offers it.
 * The plan says what the caller writes and attends: prompt chunks (slots), decode
 * tokens (slots, copy-on-write pairs) and swap copies.  The caller runs a step's
 * device work as: swap-in copies, prompt writes and prefill, swap-out copies,
 * decode writes and decode.
 *
 *   pa_sched_create    num_host_blocks > 0 enables swap preemption; prefix_caching
 *                      != 0 makes requests carry token IDs.
 *   pa_sched_allocator the scheduler's allocator (owned by it; valid until destroy),
 *                      for block tables and statistics; do not add or free through it.
 *   pa_sched_add_requests  n requests (ids returned in rids, consecutive from 0 in
 *                      creation order); they join the queue at the next step.
 *                      prompt_tokens: the prompts concatenated (prefix caching only,
 *                      else NULL); out_tokens: NULL or the out_lens[k] tokens each
 *                      request generates, concatenated (prefix caching: the ID of the
 *                      token appended at position prompt_len + g; a replayed trace
 *                      knows them, a live loop passes them with pa_sched_push_tokens
 *                      as it samples them).
 *   pa_sched_push_tokens  append a token ID to each named request's known outputs.
 *   pa_sched_step      run one step; *plan points into the scheduler's own arrays,
 *                      valid until the next step or destroy.  PA_ERR_STATE (nothing
 *                      changed) when prefix caching needs a decode token's ID that
 *                      was not given.
 *   pa_sched_running / pa_sched_waiting  the running (running order) and waiting
 *                      (queue order) requests; returns the count, fills up to cap.
 * Not thread-safe: one scheduler thread.
 */
typedef struct pa_scheduler pa_scheduler;

typedef struct pa_sched_plan {
    int64_t step;                       /* steps run before this one */
    int32_t num_finished, num_arrived, num_admitted, num_preempted;
    int32_t num_prefill, num_decode, num_decode_cows, num_swapped_in, num_swapped_out;
    int64_t num_prefill_tokens;
    const int64_t* finished;            /* [num_finished] */
    const int64_t* arrived;             /* [num_arrived] */
    const int64_t* admitted;            /* [num_admitted] */
    const int32_t* admitted_cached;     /* [num_admitted] prompt tokens already cached */
    const int64_t* preempted;           /* [num_preempted] recomputed later */
    const int64_t* prefill_rid;         /* [num_prefill] chunk's request */
    const int32_t* prefill_start;       /* [num_prefill] its first position */
    const int32_t* prefill_count;       /* [num_prefill] its tokens */
    const int64_t* prefill_slots;       /* [num_prefill_tokens] chunk after chunk */
    const int64_t* decode_rid;          /* [num_decode] */
    const int64_t* decode_pos;          /* [num_decode] position of the new token */
    const int64_t* decode_slot;         /* [num_decode] */
    const int32_t* decode_cow;          /* [num_decode][2] (src, dst), -1 -1 = none */
    const int64_t* swapped_in;          /* [num_swapped_in] */
    const int32_t* swapped_in_pairs;    /* [num_swapped_in] pairs of each */
    const int32_t* swap_in;             /* (host, device) block pairs, request after request */
    const int64_t* swapped_out;         /* [num_swapped_out] */
    const int32_t* swapped_out_pairs;   /* [num_swapped_out] */
    const int32_t* swap_out;            /* (device, host) block pairs */
} pa_sched_plan;

pa_status pa_sched_create(int32_t num_blocks, int32_t block_size,
                          const int32_t* initial_free_order, int32_t chunk,
                          int32_t prefix_caching, int32_t num_host_blocks, pa_scheduler** out);
void      pa_sched_destroy(pa_scheduler* s);
pa_allocator* pa_sched_allocator(pa_scheduler* s);
pa_status pa_sched_add_requests(pa_scheduler* s, int32_t n, const int32_t* prompt_lens,
                                const int32_t* out_lens, const int32_t* prompt_tokens,
                                const int32_t* out_tokens, int64_t* rids);
pa_status pa_sched_push_tokens(pa_scheduler* s, const int64_t* rids, const int32_t* tokens,
                               int32_t n);
pa_status pa_sched_step(pa_scheduler* s, pa_sched_plan* plan);
int32_t   pa_sched_running(const pa_scheduler* s, int64_t* rids, int32_t* prompts,
                           int32_t* lengths, int32_t cap);
int32_t   pa_sched_waiting(const pa_scheduler* s, int64_t* rids, int32_t cap);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
