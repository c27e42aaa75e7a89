// Internal declarations shared by the translation units of libpa.so.
// Not part of the ABI (include/pa.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "../../include/pa.h"

namespace pa {

constexpr int kBlock = 16;           // tokens per pool block (the only size supported)
constexpr int kKeysPerIter = 64;     // keys one wave scores per iteration (4 blocks)
constexpr int kWavesPerGroup = 4;    // waves per workgroup in the split-K kernels

// One unit of token-parallel (split-K) attention: keys [kv_begin, kv_end),
// walked through the block table of request `req`, for the query rows of the
// item's kind:
//  * kind 0 (ntok = 1): row `token` of the flat stream.  When `wpos` >= 0
//    (attention that includes the KV update) the row is its request's only
//    new token, at position wpos inside this unit's key range: the unit first
//    stores the token's K/V rows into the pool, then attends.
//  * kind 1: the ntok consecutive rows token .. token + ntok - 1 of request
//    `req` (a short chunk, such as the draft tokens of a verify step); `wpos`
//    is the key limit (exclusive) of the last of them, and with a causal mask
//    row t sees keys below wpos - (ntok - 1 - t).
//  * kind 2 (shared prefix): the rows row_token[token .. token + ntok - 1] of
//    the prefix row list, over keys [kv_begin, kv_end) of the common prefix,
//    walked through the block-table row `prefix_bt` (no mask: the prefix lies
//    in every row's history); row t's partial goes to slot
//    row_slot0[token + t] + part.
// The matrix-core kernel gives each (row, q head) pair one MFMA column, so
// ntok x g <= 32.  Kinds 0 and 1: when `part` < 0 the range is every row's
// whole visible range and the kernel writes the final output; otherwise row
// t's partial (m, l, o) goes to slot part + t * stride.
struct DecodeItem {
  int32_t token;
  int32_t req;
  int32_t kv_begin;
  int32_t kv_end;
  int32_t part;
  int32_t wpos;
  int16_t ntok;
  int16_t kind;
  int32_t stride;
};
static_assert(sizeof(DecodeItem) == 32, "decode items are 32 bytes");

// New tokens whose K/V rows the plan-driven scatter writes: `count` (1..16)
// consecutive tokens of request `req`, flat rows tok0 .., positions pos0 ..,
// all in logical block pos0 / 16.
struct WriteSeg {
  int32_t req;
  int32_t tok0;
  int32_t pos0;
  int32_t count;
};

struct WriteArgs {
  const void *key;        // [T][Hkv][D] input rows
  const void *value;
  const WriteSeg *segs;
  const int32_t *block_table;
  int64_t *slots_out;     // [T] or null
  void *k_cache;
  void *v_cache;
  int32_t n_segs;
  int32_t bt_stride;
  int32_t num_blocks;
  int32_t num_kv_heads;
  float k_scale;          // pool scales (fp8 encode), 1 otherwise
  float v_scale;
  int32_t *release;       // or null: release flag of the stream's previous staging buffer
};

// Merge of the partials of one token: slots [first, first + count).
struct MergeItem {
  int32_t token;
  int32_t first;
  int32_t count;
  int32_t pad;
};

// One workgroup of an MFMA extend kernel: columns [col0, col0 + kExtCols)
// (key-split kernel) or [col0, col0 + kWideCols) (wide kernel) of request
// `req`, where column k is (token t = k / g, q head hg = k % g) of kv head
// `kvh`; the request's new tokens start at stream row `tok0`, there are `c`
// of them and the request holds `L` tokens in total.  Wide items only: the
// item covers keys [key0, key1) of the columns' visible ranges (key0 a
// multiple of 64); with slot0 >= 0 it is one key piece of its columns and
// writes partial (m, l, o) of token t (0-based within the request) at
// partial slot slot0 + t * slot_stride, else the output.  The wide kernel
// also runs key-split items (mode 1), so that one launch can mix both.
struct ExtendItem {
  int32_t req;
  int32_t kvh;
  int32_t tok0;
  int32_t c;
  int32_t L;
  int32_t col0;
  int32_t key0;
  int32_t key1;
  int32_t slot0;
  int32_t slot_stride;
  int32_t mode;           // wide kernel: 0 = wide item, 1 = key-split item (kExtCols columns)
  int32_t wnew;           // key-split items, attention with the KV update: 1 when this item
                          // writes its request's new K/V rows of kv head kvh itself
};

// One workgroup of the shared-prefix (cascade) pass: columns [col0, col0 +
// kExtCols) of the prefix rows of kv head `kvh`, where column k is (prefix row
// k / g, q head k % g), over keys [key0, key1) of the common prefix; the
// result is the partial (m, l, o) at slot row_slot0[row] + kc.
struct PrefixItem {
  int32_t kvh;
  int32_t col0;
  int32_t key0;
  int32_t key1;
  int32_t kc;
  int32_t pad[3];
};

struct DecodeArgs {
  const void *q;          // [T][Hq][D]
  void *out;              // [T][Hq][D]
  const void *k_cache;
  const void *v_cache;
  const int32_t *block_table;
  const DecodeItem *items;
  // > 0 (matrix-core kernel): wave (b, kv head), b < pair_stride, runs item b
  // and then item pair_stride + b when it exists; 0: one item per wave
  int32_t pair_stride;
  float *part_ml;         // [slots][Hq][2]  (m in log2 units, l)
  float *part_o;          // [slots][Hq][D]
  int32_t n_items;
  int32_t bt_stride;
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t g;              // q heads per kv head handled by this launch
  int32_t h0;             // first q head (within each kv head's group) of this launch
  int32_t g_total;        // num_q_heads / num_kv_heads
  float scale_log2;       // softmax_scale * log2(e) (* k_scale for fp8 pools)
  float v_scale;          // 1 for non-fp8 pools
  int32_t zero;           // always 0 (used to keep per-step loads inside the loop)
  int32_t causal;         // kind 1 items: rows see keys up to their own position
  // kind 2 items (shared prefix)
  const int32_t *row_token;   // flat row of each prefix row
  const int32_t *row_slot0;   // first partial slot of each prefix row
  const int32_t *prefix_bt;   // block-table row whose leading entries are the common prefix
  int32_t max_cols;       // largest ntok x g over the items (matrix-core kernel: <= 32)
  // KV update of items with wpos >= 0 (null knew: no update in this launch)
  const void *knew;       // [T][Hkv][D] new K rows (query dtype)
  const void *vnew;
  int64_t *slots_out;     // [T] or null
  void *k_store;          // the pool arrays, writable
  void *v_store;
  float enc_k_scale;      // pool scales for the fp8 encode, 1 otherwise
  float enc_v_scale;
  int32_t *release;       // or null: release flag of the stream's previous staging buffer
  // The new rows of other requests (prefill chunks) scattered by extra
  // one-wave workgroups after the decode ones (matrix-core kernel, attention
  // with the KV update): workgroup n_dec + u writes segment u / num_kv_heads
  // of wseg for kv head u % num_kv_heads, from knew / vnew.
  const WriteSeg *wseg;
  int32_t n_wseg_units;   // 0: none
  // The later launches' work lists moved from the staging buffer (host
  // memory) into the workspace by one-wave workgroups after those: workgroup
  // n_dec + n_wseg_units + c copies 16-byte vectors 256 c .. 256 c + 255 of
  // copy_vecs from copy_src to copy_dst.
  const uint4 *copy_src;
  uint4 *copy_dst;
  int32_t copy_vecs;
  int32_t n_copy_units;   // 0: none
};
constexpr int kCopyVecsPerUnit = 256;

// The merge launch's arguments.  Up to kMergeInline items also travel in the
// arguments themselves (in device memory when the kernel starts, where the
// work lists are read over PCIe from pinned host memory): measured 0.4-0.9 us
// off the merge launch of the decode workloads.
constexpr int kMergeInline = 224;
struct MergeArgs {
  void *out;
  const float *part_ml;
  const float *part_o;
  const MergeItem *items;
  int32_t n_items;
  int32_t num_q_heads;
  int32_t inline_items;   // 1: the items are inl[0 .. n_items)
  int32_t pad;
  MergeItem inl[kMergeInline];
};
static_assert(sizeof(MergeArgs) <= 4096, "kernel arguments of at most 4 KB");

struct ExtendArgs {
  const void *q;
  void *out;
  const void *k_cache;
  const void *v_cache;
  const int32_t *block_table;
  const ExtendItem *items;
  // shared-prefix pass only
  const PrefixItem *pitems;
  const int32_t *row_token;   // token (flat row) of each prefix row
  const int32_t *row_slot0;   // first partial slot of each prefix row
  const int32_t *prefix_bt;   // block-table row whose leading entries are the common prefix
  float *part_ml;             // [slots][Hq][2]
  float *part_o;              // [slots][Hq][D]
  int32_t prefix_cols;        // prefix rows x g
  int32_t n_items;
  int32_t bt_stride;
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t g;
  int32_t causal;
  float scale_log2;
  float k_scale;
  float v_scale;
  // KV update by items with wnew (null knew: none in this launch)
  const void *knew;           // [T][Hkv][D] new K rows (bf16)
  const void *vnew;
  int64_t *slots_out;         // [T] or null
  void *k_store;              // the pool arrays, writable
  void *v_store;
  float enc_k_scale;          // pool scales for the fp8 encode, 1 otherwise
  float enc_v_scale;
  int32_t *release;           // or null: release flag of the stream's previous staging buffer
  // The merge of the split-K partials (of an earlier launch of the call)
  // carried by extra workgroups after the extend items: workgroup n_items + b
  // merges units 8 b .. 8 b + 7, unit u being q head u % num_q_heads of
  // merge item u / num_q_heads, into `out`.
  const MergeItem *mitems;
  int32_t n_merge_units;      // 0: none
};

constexpr int kExtCols = 128;        // columns per extend workgroup (4 x 32, keys split over 2 waves)
constexpr int kWideCols = 256;       // columns per wide extend workgroup (8 x 32, every wave every key)

// Launchers (return hipSuccess or the launch error).
hipError_t launch_slot_mapping(const pa_batch &b, int64_t *slots, int max_c, hipStream_t s);
hipError_t launch_write_kv(const pa_kv_pool &p, const void *key, const void *value,
                           pa_dtype in_dtype, const int64_t *slots, int32_t num_tokens,
                           hipStream_t s);
hipError_t launch_plan_copy(void *dst, const void *src, size_t bytes, hipStream_t s);
hipError_t launch_write_new(const pa_kv_pool &p, pa_dtype in_dtype, const WriteArgs &a,
                            hipStream_t s);
hipError_t launch_decode(const pa_kv_pool &p, pa_dtype q_dtype, const DecodeArgs &a,
                         int g_tmpl, hipStream_t s);
// split-K decode on the matrix cores (bf16 and fp8 pools)
hipError_t launch_decode_mfma(const pa_kv_pool &p, const DecodeArgs &a, hipStream_t s);
hipError_t launch_merge(pa_dtype q_dtype, int head_dim, const MergeArgs &a, hipStream_t s);
// all extend items (wide and key-split) in one launch
hipError_t launch_extend_wide(const pa_kv_pool &p, const ExtendArgs &a, hipStream_t s);
hipError_t launch_prefix(const pa_kv_pool &p, const ExtendArgs &a, hipStream_t s);

// Records the error detail for pa_last_error() and returns `st`.
pa_status pa_set_error(pa_status st, const char *fmt, ...);

// Placement probe: 4 x cus, 8 x cus and 2 x cus workgroups, each writing its
// (HW_ID, XCC_ID) pair at ids[2 * workgroup].
hipError_t launch_placement_probe(int cus, uint32_t *one_ids, uint32_t *two_ids, uint32_t *wide_ids,
                                  hipStream_t s);

hipError_t launch_zero_blocks(const pa_kv_pool &p, const int32_t *block_ids, int32_t n, hipStream_t s);

// Kernel timing hooks (no-ops unless profiling is enabled).
void prof_begin(const char *name, hipStream_t s);
void prof_end(hipStream_t s);

}  // namespace pa
