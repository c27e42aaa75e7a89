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
// for the tokens the step's plan lists: token n of request req at position
// pos goes to slot block_table[req][pos / 16] * 16 + pos % 16, which is also
// stored to slots_out[n] when that pointer is set.  Used by the attention
// call that includes the KV update.
template <int IN, int KV, int D>
__global__ __launch_bounds__(256) void k_write_new(const WriteArgs a) {
  constexpr int IB = KvTraits<IN>::bytes;
  constexpr int PB = KvTraits<KV>::bytes;
  constexpr int NCH = D * PB / 16;
  constexpr int TILE = D * kBlock * PB;

  const int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)a.n_toks * a.num_kv_heads * NCH;
  if (w >= total) return;
  const int c = (int)(w % NCH);
  const int64_t wh = w / NCH;               // list entry * num_kv_heads + head
  const int h = (int)(wh % a.num_kv_heads);
  const WriteTok t = a.toks[wh / a.num_kv_heads];
  const int64_t slot =
      (int64_t)a.block_table[(int64_t)t.req * a.bt_stride + t.pos / kBlock] * kBlock + t.pos % kBlock;
  if (a.slots_out && h == 0 && c == 0) a.slots_out[t.token] = slot;
  const int64_t th = (int64_t)t.token * a.num_kv_heads + h;
  const KvChunkIn<IN, KV> in = load_kv_chunk<IN, KV>((const char *)a.key + th * D * IB,
                                                     (const char *)a.value + th * D * IB, c);
  if (slot < 0 || slot >= a.capacity) return;
  const int64_t blk = slot / kBlock;
  const int off = (int)(slot - blk * kBlock);
  store_kv_chunk<IN, KV, D>(in, a.k_cache, a.v_cache, (blk * a.num_kv_heads + h) * (int64_t)TILE,
                            off, c, a.k_scale, a.v_scale);
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
  const int64_t threads = (int64_t)a.n_toks * p.num_kv_heads * (p.head_dim * KvTraits<KV>::bytes / 16);
  const dim3 grid((unsigned)((threads + 255) / 256));
  prof_begin("k_write_new", s);
  if (p.head_dim == 128) hipLaunchKernelGGL((k_write_new<IN, KV, 128>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((k_write_new<IN, KV, 64>), grid, dim3(256), 0, s, a);
  prof_end(s);
  return hipGetLastError();
}

hipError_t launch_write_new(const pa_kv_pool &p, pa_dtype in_dtype, const WriteArgs &a, hipStream_t s) {
  if (a.n_toks == 0) return hipSuccess;
  if (p.kv_dtype == PA_F32) return write_new_d<KV_F32, KV_F32>(p, a, s);
  if (p.kv_dtype == PA_BF16) return write_new_d<KV_BF16, KV_BF16>(p, a, s);
  if (in_dtype == PA_BF16) return write_new_d<KV_BF16, KV_FP8>(p, a, s);
  return write_new_d<KV_F32, KV_FP8>(p, a, s);
}

}  // namespace pa
