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
  constexpr int E = 16 / PB;                // pool elements per 16-byte chunk
  constexpr int NCH = D / E;                // chunks per key row
  constexpr int TILE = D * kBlock * PB;     // bytes of one (block, head) tile
  static_assert(IN != KV_FP8, "fp8 is a pool format only");
  static_assert(KV == KV_FP8 || IN == KV, "same-dtype copy or fp8 encode");

  const int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)num_tokens * num_kv_heads * NCH;
  if (w >= total) return;
  const int c = (int)(w % NCH);
  const int64_t th = w / NCH;               // token * num_kv_heads + head
  const int h = (int)(th % num_kv_heads);
  const int64_t n = th / num_kv_heads;
  const int64_t slot = slots[n];
  // input elements c*E .. c*E+E-1 of the token's K and V rows
  const char *ks = (const char *)key + (th * D + (int64_t)c * E) * IB;
  const char *vs = (const char *)value + (th * D + (int64_t)c * E) * IB;
  constexpr int NV = E * IB / 16;           // 16-byte input vectors per chunk
  uint4 kin[NV], vin[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    kin[i] = ((const uint4 *)ks)[i];
    vin[i] = ((const uint4 *)vs)[i];
  }
  if (slot < 0 || slot >= capacity) return;  // padding token / out-of-range slot
  const int64_t blk = slot / kBlock;
  const int off = (int)(slot - blk * kBlock);
  const int64_t tile = (blk * num_kv_heads + h) * (int64_t)TILE;
  char *kdst = (char *)kc + tile + (int64_t)c * (kBlock * 16) + off * 16;
  char *vdst = (char *)vc + tile + ((int64_t)c * E * kBlock + off) * PB;  // row c*E, column off
  if constexpr (KV != KV_FP8) {
    *(uint4 *)kdst = kin[0];
    const uint32_t *vw = (const uint32_t *)vin;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if constexpr (KV == KV_F32) ((uint32_t *)vdst)[e * kBlock] = vw[e];
      else ((uint16_t *)vdst)[e * kBlock] = (uint16_t)(vw[e / 2] >> (16 * (e & 1)));
    }
  } else {
    const uint32_t *kw = (const uint32_t *)kin, *vw = (const uint32_t *)vin;
    auto elem = [](const uint32_t *words, int e) -> float {
      if constexpr (IN == KV_BF16) return __uint_as_float((words[e / 2] >> (16 * (e & 1))) << 16);
      else return __uint_as_float(words[e]);
    };
    uint32_t out[4] = {0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < E; ++e) {
      out[e / 4] |= e4m3_encode(elem(kw, e) / k_scale) << (8 * (e & 3));
      ((uint8_t *)vdst)[e * kBlock] = (uint8_t)e4m3_encode(elem(vw, e) / v_scale);
    }
    *(uint4 *)kdst = make_uint4(out[0], out[1], out[2], out[3]);
  }
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

}  // namespace pa
