// Slot derivation and KV scatter kernels.
//
// Slot derivation follows "vLLM 推理流程分析" §5.1.2 (compute_slot_mapping):
// the new token at position p of request i goes to slot
// block_table[i][p / S] * S + p % S, with p = seq_len - c + t.
// The scatter follows §6.3 of the same page (reshape_and_cache_flash: write
// each token's K and V rows at its slot, converting to fp8 when the cache is
// fp8).  The pool tiles are laid out for gfx950 (see include/pa.h):
//   K tile of (block, head): [head_dim / E][16 slots][E elements]  (16-byte chunks)
//   V tile of (block, head): [head_dim][16 slots]
#include <algorithm>
#include <cstring>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// One workgroup per request; threads walk the request's new tokens.
__global__ __launch_bounds__(256) void k_slot_mapping(const int32_t *__restrict__ qsl,
                                                      const int32_t *__restrict__ seq_lens,
                                                      const int32_t *__restrict__ bt,
                                                      int32_t bt_stride,
                                                      int64_t *__restrict__ slots) {
  const int i = blockIdx.x;
  const int start = qsl[i];
  const int c = qsl[i + 1] - start;
  const int first_pos = seq_lens[i] - c;
  const int32_t *row = bt + (int64_t)i * bt_stride;
  for (int t = threadIdx.x; t < c; t += blockDim.x) {
    const int p = first_pos + t;
    const int b = p / kBlock;
    const int o = p - b * kBlock;
    slots[start + t] = (int64_t)row[b] * kBlock + o;
  }
}

hipError_t launch_slot_mapping(const pa_batch &b, int64_t *slots, int max_c, hipStream_t s) {
  if (b.num_seqs == 0 || b.num_tokens == 0) return hipSuccess;
  const int threads = max_c >= 256 ? 256 : (max_c <= 64 ? 64 : 128);
  prof_begin("k_slot_mapping", s);
  hipLaunchKernelGGL(k_slot_mapping, dim3(b.num_seqs), dim3(threads), 0, s, b.query_start_loc,
                     b.seq_lens, b.block_table, b.bt_stride, slots);
  prof_end(s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// KV scatter.  One thread per (token, kv head, 16-byte pool chunk of K): it
// reads the token's slot and the matching input elements of K and V once and
// writes the K chunk (16 contiguous bytes) and the same dims of V (one
// element per dim row of the dimension-major V tile).  Threads of one token
// and head are consecutive, so input rows are read contiguously; a decode
// step needs a single round trip per token.
// IN / KV are the input and pool element kinds.
// ---------------------------------------------------------------------------
template <int IN, int KV, int D>
__global__ __launch_bounds__(256) void k_write_kv(const void *__restrict__ key,
                                                  const void *__restrict__ value,
                                                  const int64_t *__restrict__ slots,
                                                  int32_t num_tokens, int32_t num_kv_heads,
                                                  int64_t capacity, void *__restrict__ kc,
                                                  void *__restrict__ vc, float k_scale,
                                                  float v_scale) {
  constexpr int IB = KvTraits<IN>::bytes;   // input element bytes
  constexpr int PB = KvTraits<KV>::bytes;   // pool element bytes
  constexpr int NCH = D * PB / 16;          // chunks per key row
  constexpr int TILE = D * kBlock * PB;     // bytes of one (block, head) tile

  const int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)num_tokens * num_kv_heads * NCH;
  if (w >= total) return;
  const int c = (int)(w % NCH);
  const int64_t th = w / NCH;               // token * num_kv_heads + head
  const int h = (int)(th % num_kv_heads);
  const int64_t n = th / num_kv_heads;
  const int64_t slot = slots[n];
  const KvChunkIn<IN, KV> in = load_kv_chunk<IN, KV>((const char *)key + th * D * IB,
                                                     (const char *)value + th * D * IB, c);
  if (slot < 0 || slot >= capacity) return;  // padding token / out-of-range slot
  const int64_t blk = slot / kBlock;
  const int off = (int)(slot - blk * kBlock);
  store_kv_chunk<IN, KV, D>(in, kc, vc, (blk * num_kv_heads + h) * (int64_t)TILE, off, c, k_scale,
                            v_scale);
}

// The same scatter with the slots derived on the fly (a1 + a2 in one pass),
// for the new tokens the step's plan lists as block segments: up to 16
// consecutive tokens of one request whose positions fall in one logical
// block.  Token n of the segment at position p goes to slot
// block_table[req][p / 16] * 16 + p % 16, which is also stored to slots_out[n]
// when that pointer is set.  One workgroup per (segment, kv head) fills the
// segment's slots of the head's K and V tiles (scatter_segment).  Used by the
// attention call that includes the KV update when no split-K launch carries
// the segments.
template <int IN, int KV, int D>
__global__ __launch_bounds__(256) void k_write_new(const WriteArgs a) {
  const StagingRelease staging_release{a.release};
  __shared__ __attribute__((aligned(16))) uint8_t vt[D * kBlock * KvTraits<KV>::bytes];
  const int h = (int)(blockIdx.x % (unsigned)a.num_kv_heads);
  const int si = (int)(blockIdx.x / (unsigned)a.num_kv_heads);
  const WriteSeg sg = a.segs[si];
  scatter_segment<IN, KV, D, 256>(sg.req, sg.tok0, sg.pos0, sg.count, h, a.num_kv_heads, a.key, a.value,
                                  a.block_table, a.bt_stride, a.num_blocks, a.k_cache, a.v_cache, a.k_scale,
                                  a.v_scale, a.slots_out, vt, threadIdx.x);
}

template <int IN, int KV>
static hipError_t write_dispatch_d(const pa_kv_pool &p, const void *key, const void *value,
                                   const int64_t *slots, int32_t T, hipStream_t s) {
  const int64_t chunks = (int64_t)T * p.num_kv_heads * (p.head_dim * KvTraits<KV>::bytes / 16);
  const dim3 grid((unsigned)((chunks + 255) / 256));
  const int64_t cap = (int64_t)p.num_blocks * p.block_size;
  prof_begin("k_write_kv", s);
  if (p.head_dim == 128)
    hipLaunchKernelGGL((k_write_kv<IN, KV, 128>), grid, dim3(256), 0, s, key, value, slots, T,
                       p.num_kv_heads, cap, p.k_cache, p.v_cache, p.k_scale, p.v_scale);
  else
    hipLaunchKernelGGL((k_write_kv<IN, KV, 64>), grid, dim3(256), 0, s, key, value, slots, T,
                       p.num_kv_heads, cap, p.k_cache, p.v_cache, p.k_scale, p.v_scale);
  prof_end(s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Plan copy for launches captured into a HIP graph: the work lists travel as
// kernel arguments (captured by value into the graph node) and are written
// into the caller's workspace, so every replay rebuilds the same lists
// without any host buffer that the library might reuse later.
// ---------------------------------------------------------------------------
constexpr int kPieceWords = 992;     // 3968 bytes of payload per launch

struct PlanPiece {
  uint32_t words[kPieceWords];
};

__global__ __launch_bounds__(256) void k_plan_copy(const PlanPiece piece, uint32_t *__restrict__ dst,
                                                   int32_t nwords) {
  for (int i = threadIdx.x; i < nwords; i += blockDim.x) dst[i] = piece.words[i];
}

hipError_t launch_plan_copy(void *dst, const void *src, size_t bytes, hipStream_t s) {
  const size_t words = bytes / 4;
  for (size_t w0 = 0; w0 < words; w0 += kPieceWords) {
    const int n = (int)std::min<size_t>(kPieceWords, words - w0);
    PlanPiece piece;
    memcpy(piece.words, (const uint32_t *)src + w0, (size_t)n * 4);
    hipLaunchKernelGGL(k_plan_copy, dim3(1), dim3(256), 0, s, piece, (uint32_t *)dst + w0, n);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Zeroing of newly allocated blocks ("vLLM 推理流程分析" §5.1.1, the model
// runner clears the blocks the scheduler lists in new_block_ids_to_zero, so
// that no stale K/V of an earlier owner can be read).  A block's tiles of all
// kv heads are contiguous in each of k_cache and v_cache; one workgroup per
// (block, array) clears them with 16-byte stores.  Ids outside the pool are
// skipped.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_zero_blocks(const int32_t *__restrict__ ids, int32_t num_blocks,
                                                     int64_t block_bytes, char *__restrict__ kc,
                                                     char *__restrict__ vc) {
  const int32_t b = ids[blockIdx.x];
  if (b < 0 || b >= num_blocks) return;
  char *base = (blockIdx.y == 0 ? kc : vc) + (int64_t)b * block_bytes;
  for (int64_t o = threadIdx.x * 16; o < block_bytes; o += blockDim.x * 16)
    *(uint4 *)(base + o) = make_uint4(0, 0, 0, 0);
}

hipError_t launch_zero_blocks(const pa_kv_pool &p, const int32_t *block_ids, int32_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int elem = p.kv_dtype == PA_F32 ? 4 : p.kv_dtype == PA_BF16 ? 2 : 1;
  const int64_t block_bytes = (int64_t)p.num_kv_heads * p.head_dim * p.block_size * elem;
  prof_begin("k_zero_blocks", s);
  hipLaunchKernelGGL(k_zero_blocks, dim3((unsigned)n, 2), dim3(256), 0, s, block_ids, p.num_blocks,
                     block_bytes, (char *)p.k_cache, (char *)p.v_cache);
  prof_end(s);
  return hipGetLastError();
}

hipError_t launch_write_kv(const pa_kv_pool &p, const void *key, const void *value,
                           pa_dtype in_dtype, const int64_t *slots, int32_t T, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (p.kv_dtype == PA_F32) return write_dispatch_d<KV_F32, KV_F32>(p, key, value, slots, T, s);
  if (p.kv_dtype == PA_BF16) return write_dispatch_d<KV_BF16, KV_BF16>(p, key, value, slots, T, s);
  if (in_dtype == PA_BF16) return write_dispatch_d<KV_BF16, KV_FP8>(p, key, value, slots, T, s);
  return write_dispatch_d<KV_F32, KV_FP8>(p, key, value, slots, T, s);
}

template <int IN, int KV>
static hipError_t write_new_d(const pa_kv_pool &p, const WriteArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)a.n_segs * p.num_kv_heads));
  prof_begin("k_write_new", s);
  if (p.head_dim == 128) hipLaunchKernelGGL((k_write_new<IN, KV, 128>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((k_write_new<IN, KV, 64>), grid, dim3(256), 0, s, a);
  prof_end(s);
  return hipGetLastError();
}

hipError_t launch_write_new(const pa_kv_pool &p, pa_dtype in_dtype, const WriteArgs &a, hipStream_t s) {
  if (a.n_segs == 0) return hipSuccess;
  if (p.kv_dtype == PA_F32) return write_new_d<KV_F32, KV_F32>(p, a, s);
  if (p.kv_dtype == PA_BF16) return write_new_d<KV_BF16, KV_BF16>(p, a, s);
  if (in_dtype == PA_BF16) return write_new_d<KV_BF16, KV_FP8>(p, a, s);
  return write_new_d<KV_F32, KV_FP8>(p, a, s);
}

}  // namespace pa
