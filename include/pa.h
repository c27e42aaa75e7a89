/*
 * pa.h -- C ABI of libpa.so: one paged-attention step on AMD Instinct MI355X
 * (gfx950).
 *
 * The step follows the attention layer of a continuous-batching inference
 * step as the pages describe it:
 *   [P1] "vLLM 推理流程分析" (blog.chen3feng.top): §5.1.2 _prepare_inputs
 *        (positions, query_start_loc, seq_lens, compute_slot_mapping), §6.1
 *        attention dispatch (write the new K/V first, then attend), §6.2 the
 *        paged FlashAttention call, §6.3 the KV-cache write
 *        (reshape_and_cache_flash with slot_mapping, kv_cache_dtype, k_scale,
 *        v_scale), §10.1-10.2 the cache's life over prefill and decode.
 *   [P5] "vLLM 源码完全拆解（十六）：把十五篇机制拼成一张可执行的源码阅读地图"
 *        (pinghaoyang.com.cn): third walk-through path (slot = physical block
 *        * S + offset; paging changes where K/V are fetched, not the
 *        attention definition; partitioned evaluation with a rescaling
 *        merge), fourth walk-through path (query_start_loc as a prefix sum of
 *        per-request token counts; the metadata consistency checks).
 *
 * Conventions shared by every call
 * --------------------------------
 * - All sizes are element counts unless a name ends in _bytes.
 * - "device" pointers are HIP device memory on the current device; "host"
 *   pointers are ordinary CPU memory.  The library never takes ownership of
 *   a buffer, never frees one, and keeps no pointer after a call returns.
 * - Calls that launch work are asynchronous on the given stream (NULL means
 *   the default stream).  Work enqueued by one call on a stream sees the
 *   effects of earlier calls on that stream (so pa_write_kv then
 *   pa_attention on one stream attends over the freshly written rows, as
 *   [P1] §6.1 orders them).
 * - Errors are reported through pa_status only; nothing is thrown across
 *   the ABI.  On any status other than PA_OK and PA_ERR_HIP the call has
 *   enqueued no work, and pa_last_error() (per thread) describes the
 *   problem.  PA_ERR_HIP means a HIP runtime call failed; when a call
 *   launches several kernels and a later launch fails, the kernels queued
 *   before it stay queued (for pa_write_kv_attention this can be part of
 *   the KV update).  Every argument and workspace check is done before the
 *   first launch.
 * - The library is thread-compatible: concurrent calls on different streams
 *   are allowed; the workspace passed to pa_attention must not be shared by
 *   calls that may run concurrently.
 * - HIP graphs: every launching call may be captured into a HIP graph
 *   (stream capture).  pa_attention and pa_write_kv_attention then store
 *   their work lists at capture in a pinned host arena of the library (8 MiB
 *   per device, created by the first call on the device made outside
 *   capture, never reused, kept until the process ends) that the graph's
 *   kernels read at every replay; without room there, the lists are written
 *   into the workspace by copy kernels inside the graph.  A replay
 *   recomputes the captured batch on the current contents of the device
 *   buffers.  The batch's shape (the host mirrors, num_tokens and the hint)
 *   is fixed at capture; the device arrays, the pool, query/key/value and
 *   the block-table contents are read at replay.  The workspace and every
 *   buffer must stay allocated while the graph is replayed.  With
 *   PA_VALIDATE set a captured call returns PA_ERR_UNSUPPORTED (the checks
 *   read the block table back synchronously), and launches are not timed
 *   by pa_profile_enable while captured.
 *
 * KV pool layout (chosen for gfx950, differs from the pages' layout)
 * ------------------------------------------------------------------
 * The pool is two arrays, k_cache and v_cache, each holding num_blocks
 * blocks of block_size token slots for num_kv_heads heads of head_dim
 * elements.  Slot s lives in block s / block_size at offset s % block_size.
 * Within a block each kv head owns one contiguous tile:
 *   k_cache: [num_blocks][num_kv_heads][head_dim / E][block_size][E]
 *            E = 16 / sizeof(element) (4 fp32, 8 bf16, 16 fp8): the key
 *            row of a slot is cut into 16-byte chunks; chunk c of all
 *            block_size slots is contiguous.
 *   v_cache: [num_blocks][num_kv_heads][head_dim][block_size]
 *            (the tile is stored dimension-major).
 * pa_kv_elem_offset() returns the element index of any (block, offset,
 * head, dim) and is the authoritative definition of this layout.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The same type as hipStream_t (an opaque HIP stream handle). */
struct ihipStream_t;
typedef struct ihipStream_t *pa_stream_t;

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1,  /* a null pointer, negative size or inconsistent shape  */
  PA_ERR_UNSUPPORTED = 2,  /* a valid request the library does not implement      */
  PA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required           */
  PA_ERR_VALIDATION = 4,   /* metadata failed the consistency checks (PA_VALIDATE) */
  PA_ERR_HIP = 5,          /* a HIP runtime call failed                            */
  PA_ERR_CAPACITY = 6      /* the block pool has too few free blocks               */
} pa_status;

/* Element types.  pa_dtype is a plain 32-bit integer (not an enum type), so
 * that every value a caller passes is well defined on both sides of the
 * ABI; the calls reject values other than these constants with
 * PA_ERR_INVALID_ARG or PA_ERR_UNSUPPORTED. */
enum {
  PA_F32 = 0,       /* IEEE binary32                                          */
  PA_BF16 = 1,      /* bfloat16                                               */
  PA_FP8_E4M3 = 2   /* OCP FP8 E4M3FN (bias 7, max 448, no inf), pool only    */
};
typedef int32_t pa_dtype;

/* A KV pool ([P1] §6.2: key_cache / value_cache, one per K and V).
 * Supported: block_size 16; head_dim 64 or 128; kv_dtype F32, BF16 or
 * FP8_E4M3.  k_scale / v_scale are the per-tensor dequantisation scales of
 * an FP8 pool (stored code * scale = value) and are ignored otherwise. */
typedef struct pa_kv_pool {
  void *k_cache;            /* device, pa_kv_cache_bytes() bytes */
  void *v_cache;            /* device, pa_kv_cache_bytes() bytes */
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  pa_dtype kv_dtype;
  float k_scale;
  float v_scale;
} pa_kv_pool;

/* One step's ragged batch ([P1] §5.1.3 common attention metadata).
 * Request i owns query rows query_start_loc[i] .. query_start_loc[i+1]-1 of
 * the flat token stream (its c_i new tokens) and has seq_lens[i] tokens in
 * total including them, so new token t sits at position
 * seq_lens[i] - c_i + t.  block_table row i lists the physical blocks of
 * logical blocks 0, 1, ...; only its first ceil(seq_lens[i] / block_size)
 * entries are ever read.  The host mirrors must hold the same values as the
 * device arrays (the caller builds them on the CPU anyway); the library
 * reads them to plan the launch without a device-to-host copy. */
typedef struct pa_batch {
  int32_t num_seqs;                     /* N >= 0                              */
  int32_t num_tokens;                   /* T = query_start_loc[N]              */
  const int32_t *query_start_loc;       /* device [N + 1]                      */
  const int32_t *seq_lens;              /* device [N]                          */
  const int32_t *block_table;           /* device [N][bt_stride]               */
  int32_t bt_stride;                    /* elements between block_table rows   */
  const int32_t *query_start_loc_host;  /* host   [N + 1], same values         */
  const int32_t *seq_lens_host;         /* host   [N],     same values         */
  int32_t num_common_prefix_blocks;     /* shared-prefix hint, see below (0: none) */
} pa_batch;

/* num_common_prefix_blocks ([P1] §4.4: the scheduler reports the number of
 * blocks common to all requests; §5.1.3: cascade attention): n > 0
 * states that the first n block-table entries of every request that has new
 * tokens are the same n physical blocks, and that these blocks lie wholly in
 * every such request's history (16 * n <= seq_lens[i] - c_i).  The library
 * may then compute the rows' attention over those 16 * n keys once for all
 * rows that share them and combine it with the rest by the partition rule of
 * [P5] third walk-through path; the result equals the one without the hint
 * up to rounding.  The hint is ignored (no error) where it cannot be used: a
 * request violating the history condition, rows the library handles with
 * its prefill kernel, or pool / query types without that path.  A hint whose
 * blocks are not actually shared gives wrong results; with PA_VALIDATE set,
 * pa_attention checks the block tables and returns PA_ERR_VALIDATION. */

/* ---------------------------------------------------------------------- */

/* a0 -- step metadata on the host ([P1] §5.1.2; [P5] fourth walk-through
 * path).  query_start_loc[0] = 0, query_start_loc[i+1] = query_start_loc[i]
 * + num_scheduled[i]; seq_lens[i] = num_computed[i] + num_scheduled[i].
 * All pointers are host memory; query_start_loc has num_seqs + 1 entries.
 * PA_ERR_INVALID_ARG for negative counts or a total above INT32_MAX. */
pa_status pa_prepare_metadata(int32_t num_seqs, const int32_t *num_computed,
                              const int32_t *num_scheduled, int32_t *query_start_loc,
                              int32_t *seq_lens);

/* a1 -- slot derivation on the device ([P1] §5.1.2 compute_slot_mapping;
 * [P5] third walk-through path).  For every new token t of request i, with
 * p = seq_lens[i] - c_i + t:
 *   slot_mapping[query_start_loc[i] + t] =
 *       block_table[i][p / block_size] * block_size + p % block_size.
 * slot_mapping: device int64 [batch->num_tokens], written.  block_size must
 * be 16.  The host mirrors of the batch are used to size the launch. */
pa_status pa_slot_mapping(const pa_batch *batch, int32_t block_size, int64_t *slot_mapping,
                          pa_stream_t stream);

/* a2 -- KV scatter ([P1] §6.3 reshape_and_cache_flash).  For every token n
 * with slot_mapping[n] >= 0, stores key[n] and value[n] (each
 * [num_kv_heads][head_dim], in_dtype) into that slot of the pool.  Same
 * dtype: a bit copy (F32 -> F32, BF16 -> BF16).  FP8 pool (in_dtype F32 or
 * BF16): y = x / scale in IEEE fp32, then the nearest E4M3FN value with ties
 * to even, |y| > 448 saturating to +-448, NaN -> 0x7F.  Negative slots are
 * skipped (padding tokens); slots at or beyond num_blocks * block_size are
 * skipped as well (and reported under PA_VALIDATE).  Duplicate non-negative
 * slots within one call leave the slot holding one of the rows.
 * key, value: device [num_tokens][num_kv_heads][head_dim]; slot_mapping:
 * device int64 [num_tokens]. */
pa_status pa_write_kv(const pa_kv_pool *pool, const void *key, const void *value,
                      pa_dtype in_dtype, const int64_t *slot_mapping, int32_t num_tokens,
                      pa_stream_t stream);

/* Device workspace pa_attention and pa_write_kv_attention need for this
 * batch (bytes), or 0 when the arguments are invalid (pa_last_error() says
 * why).  The attention backend plans a batch on the host and runs it in a
 * caller-provided workspace ([P5] fourth walk-through path: the backend's
 * metadata builder prepares the plan and workspace before the kernels run);
 * the size depends only on the pool's shape and the batch's host mirrors
 * (the split-K partial results (m, l, o) of the rows whose keys are cut
 * into several pieces, plus room for the work lists), so the query and the
 * call always agree.  Host only: launches nothing. */
size_t pa_attention_workspace_bytes(const pa_kv_pool *pool, const pa_batch *batch,
                                    int32_t num_q_heads);

/* a3..a7 -- attention over the paged pool ([P1] §6.2 flash_attn_varlen_func
 * with block_table and causal=True; [P5] third walk-through path).  For
 * every new token n = query_start_loc[i] + t of request i and query head h:
 *   visible keys j = 0 .. p (p = seq_lens[i] - c_i + t) when causal,
 *                    0 .. seq_lens[i] - 1 when not;
 *   s_j = softmax_scale * (query[n][h] . K_j[h / g]),  g = num_q_heads / num_kv_heads;
 *   output[n][h] = sum_j softmax(s)_j * V_j[h / g],
 * with K_j / V_j read from the pool through block_table (FP8 pools are
 * dequantised with k_scale / v_scale).  softmax_scale must be finite and
 * positive (normally 1/sqrt(head_dim)).  Accumulation is fp32; the output is
 * rounded to q_dtype.  Supported: q_dtype F32 with an F32 pool; q_dtype
 * BF16 with a BF16 or FP8 pool; num_q_heads a multiple of num_kv_heads with
 * g <= 16.
 * query, output: device [num_tokens][num_q_heads][head_dim] (q_dtype).
 * workspace: device, at least pa_attention_workspace_bytes() bytes, 256-byte
 * aligned; its contents need no initialisation and are scratch after the
 * call.  Requests with c_i = 0 are skipped. */
pa_status pa_attention(const pa_kv_pool *pool, const pa_batch *batch, const void *query,
                       pa_dtype q_dtype, int32_t num_q_heads, float softmax_scale,
                       int32_t causal, void *output, void *workspace, size_t workspace_bytes,
                       pa_stream_t stream);

/* a1 + a2 + a3..a7 in one call: the attention whose forward includes the KV
 * cache update ([P1] §6.1: a backend may write the new K/V inside its own
 * forward instead of through a separate cache-update step).  The result is
 * that of
 *   pa_slot_mapping(batch, 16, slot_mapping);
 *   pa_write_kv(pool, key, value, q_dtype, slot_mapping, num_tokens);
 *   pa_attention(pool, batch, query, q_dtype, ...);
 * on the same stream: the pool receives exactly the same bytes, and the
 * attention reads the new keys as the pool holds them (quantised for FP8
 * pools).  The output may differ from pa_attention's in the last bits,
 * because the kernels may add a request's newest key in another order.
 * key, value: device [num_tokens][num_kv_heads][head_dim] in q_dtype (BF16
 * for BF16 and FP8 pools, F32 for F32 pools).  slot_mapping: device int64
 * [num_tokens], written with the slots of the new tokens, or NULL.  The
 * other arguments, the workspace (pa_attention_workspace_bytes() covers both
 * calls) and the errors are those of pa_attention; on an error other than
 * PA_ERR_HIP nothing is written.  A request's new tokens must go to slots that no other request
 * of the batch reads (a block receiving new tokens belongs to one request,
 * as any KV-cache manager arranges); otherwise the result is undefined. */
pa_status pa_write_kv_attention(const pa_kv_pool *pool, const pa_batch *batch, const void *query,
                                const void *key, const void *value, pa_dtype q_dtype,
                                int32_t num_q_heads, float softmax_scale, int32_t causal,
                                int64_t *slot_mapping, void *output, void *workspace,
                                size_t workspace_bytes, pa_stream_t stream);

/* pa_write_kv_attention for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, result, pool bytes and errors as
 * pa_write_kv_attention, without the workspace: the call's work lists and
 * split-K partials live in a static device array of the library
 * (pa_noalloc_scratch_bytes() bytes, 32 MiB; each device the library runs
 * on holds its own copy until the process ends).  The call allocates no
 * device, pinned or managed memory and creates no stream (its host-side
 * plan uses ordinary host memory); the work lists reach the array through
 * kernels that carry them as arguments.  A batch whose plan needs more than
 * the array returns PA_ERR_WORKSPACE before anything is launched (all five
 * reference workloads fit; the largest, 128 decode rows over a shared
 * prefix, needs about 20 MiB).  No part of the array needs to start at zero:
 * every byte a kernel reads was written earlier in the same call.  Every
 * call on one device shares that device's array and it keeps the last
 * call's contents, so calls that may overlap on one device (other streams,
 * other threads) race and give undefined results; serialise them. */
pa_status pa_write_kv_attention_noalloc(const pa_kv_pool *pool, const pa_batch *batch,
                                        const void *query, const void *key, const void *value,
                                        pa_dtype q_dtype, int32_t num_q_heads, float softmax_scale,
                                        int32_t causal, int64_t *slot_mapping, void *output,
                                        pa_stream_t stream);

/* Bytes of the static scratch pa_write_kv_attention_noalloc uses per device. */
size_t pa_noalloc_scratch_bytes(void);

/* ---------------------------------------------------------------------- */
/* Host block pool (the KV-cache manager on either side of the step).
 *
 * [P1] §4.2-4.3 (allocate_slots for running and waiting requests,
 * get_computed_blocks for prefix-cache hits), §8.1 (free: every block's
 * reference count drops, a block at zero returns to the free queue), §10
 * (a request's blocks over prefill, decode and prefix reuse); [P5] second
 * walk-through path (a free block keeps its contents for prefix hits until
 * it is reused; the cache key covers the parent prefix and extra identity).
 *
 * Policy where the pages leave it open: the free queue starts in ascending
 * block order and hands out from its head; a freed request returns its
 * blocks last block first; a block handed out again leaves the hash map.
 * Block hash: FNV-1a 64 over the little-endian bytes of the parent block's
 * hash (0 for a request's first block), extra_key, and the block's
 * block_size token ids as int32; lookups also compare the stored key.
 *
 * The manager is host memory only and never touches the device; calls on
 * one manager are serialised by an internal lock.  Request ids are the
 * caller's.  Errors: PA_ERR_INVALID_ARG for bad arguments or an unknown
 * request; PA_ERR_CAPACITY when allocate_slots cannot be satisfied (then
 * nothing changes). */
typedef struct pa_kv_manager pa_kv_manager;

/* A manager of blocks 0 .. num_blocks-1 of block_size tokens, all free. */
pa_status pa_kv_manager_create(int32_t num_blocks, int32_t block_size, pa_kv_manager **manager);
void pa_kv_manager_destroy(pa_kv_manager *manager);

/* Blocks in the free queue (reference count 0, cached or not); -1 for NULL. */
int32_t pa_kv_manager_num_free_blocks(pa_kv_manager *manager);

/* get_computed_blocks: the longest run of leading full blocks of token_ids
 * (num_tokens host int32 ids) whose contents are cached under extra_key.
 * The block holding the last token is never reported, so a step always
 * computes at least one token.  Writes up to max_blocks ids to blocks (host)
 * and their number to *num_blocks; takes no reference (allocate_slots does). */
pa_status pa_kv_manager_get_computed_blocks(pa_kv_manager *manager, const int32_t *token_ids,
                                            int32_t num_tokens, uint64_t extra_key,
                                            int32_t *blocks, int32_t max_blocks,
                                            int32_t *num_blocks);

/* allocate_slots: request_id will hold num_tokens tokens after the step.  A
 * request without blocks first takes computed_blocks (from
 * get_computed_blocks; each gets a reference and leaves the free queue).
 * Then blocks are taken from the head of the free queue until the request
 * has ceil(num_tokens / block_size).  The new blocks' ids (the ones to
 * zero, new_block_ids_to_zero in [P1] §4.4) go to new_blocks (host, room
 * for max_new) and their number to *num_new.  All or nothing:
 * PA_ERR_CAPACITY leaves every count unchanged. */
pa_status pa_kv_manager_allocate_slots(pa_kv_manager *manager, int64_t request_id,
                                       int32_t num_tokens, const int32_t *computed_blocks,
                                       int32_t num_computed_blocks, int32_t *new_blocks,
                                       int32_t max_new, int32_t *num_new);

/* Enters the request's full blocks among its first num_tokens tokens
 * (token_ids, host) into the prefix cache under extra_key.  A block already
 * cached, or whose key another block already holds, is left as it is. */
pa_status pa_kv_manager_cache_blocks(pa_kv_manager *manager, int64_t request_id,
                                     const int32_t *token_ids, int32_t num_tokens,
                                     uint64_t extra_key);

/* free: drops the request's reference on each of its blocks, last block
 * first; blocks reaching zero join the tail of the free queue (still
 * cached).  The request is forgotten. */
pa_status pa_kv_manager_free(pa_kv_manager *manager, int64_t request_id);

/* The request's block ids in logical order (its block-table row). */
pa_status pa_kv_manager_block_ids(pa_kv_manager *manager, int64_t request_id, int32_t *blocks,
                                  int32_t max_blocks, int32_t *num_blocks);

/* Reference count of one block. */
pa_status pa_kv_manager_ref_count(pa_kv_manager *manager, int32_t block, int32_t *ref_count);

/* Zeroes every byte of the listed blocks in k_cache and v_cache (all kv
 * heads), as the model runner clears newly allocated blocks ([P1] §5.1.1,
 * _zero_block_ids).  block_ids: device int32 [num_ids]; ids outside the pool
 * are skipped. */
pa_status pa_zero_blocks(const pa_kv_pool *pool, const int32_t *block_ids, int32_t num_ids,
                         pa_stream_t stream);

/* Bytes of each of k_cache and v_cache for this pool's shape and dtype. */
size_t pa_kv_cache_bytes(const pa_kv_pool *pool);

/* Element index (not byte offset) of (block, offset, head, dim) in k_cache
 * (which = 0) or v_cache (which = 1); -1 for out-of-range arguments. */
int64_t pa_kv_elem_offset(const pa_kv_pool *pool, int32_t which, int64_t block, int32_t offset,
                          int32_t head, int32_t dim);

/* Human-readable name of a status code (static storage). */
const char *pa_status_string(pa_status status);

/* Detail of the last failing call on this thread (empty if none). */
const char *pa_last_error(void);

/* Kernel timing for measurement.  While enabled, every kernel the library
 * launches is bracketed by a pair of HIP events recorded on the stream it
 * runs on.  pa_profile_read() waits for the recorded events and returns,
 * for the kernel named `kernel`, the number of launches and their summed
 * duration in milliseconds since the last reset.  Enabling or disabling
 * resets the records.  Launches captured into a HIP graph are not timed.
 * Work that rides in another kernel's launch is timed with that launch: the
 * one-call scatter of prefill rows in "k_decode" when no "k_write_new" runs,
 * the copy of the later launches' work lists into the workspace in
 * "k_decode", the merge of split-K partials in "k_extend" when no "k_merge"
 * runs. */
pa_status pa_profile_enable(int32_t enable);
pa_status pa_profile_read(const char *kernel, int32_t *launches, double *total_ms);

/* Placement check (diagnostic, for measurement; allocates, launches on the
 * null stream and waits for the device).  The planners rely on dispatch
 * placements that HIP does not promise; when one fails the results stay
 * exact and only the speed suffers.  Three probe launches, shaped like the
 * library's own, record each workgroup's hardware ids on the current device:
 *   one_wave_alone:   4 x CUs one-wave workgroups using over 256 registers
 *                     per lane (the matrix-core decode kernel's paired form,
 *                     sized for one wave on every SIMD): fraction of them
 *                     alone on their SIMD;
 *   two_wave_paired:  8 x CUs one-wave workgroups of two waves per SIMD (its
 *                     two-wave form): fraction of u < 4 x CUs whose partner
 *                     u + 4 x CUs runs on u's SIMD;
 *   xcd_round_robin:  2 x CUs 512-thread workgroups holding 160 KB of LDS
 *                     (the extend kernels): fraction of workgroups b on XCD
 *                     b % 8.
 * compute_units and xcds (distinct XCD ids seen) describe the device.
 * out: host struct, filled on PA_OK.  Errors: PA_ERR_INVALID_ARG (NULL out),
 * PA_ERR_HIP (no device, or a launch or copy failed). */
typedef struct pa_placement {
  int32_t compute_units;
  int32_t xcds;
  float one_wave_alone;
  float two_wave_paired;
  float xcd_round_robin;
} pa_placement;

pa_status pa_placement_check(pa_placement *out);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
