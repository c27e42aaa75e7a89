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
// KV scatter.  A workgroup takes 16 consecutive tokens of one kv head.
//  K: thread (chunk c, token n) copies / encodes the 16-byte pool chunk c of
//     token n, so the 16 threads of a chunk write 256 contiguous bytes when
//     the tokens' slots are consecutive within a block (prefill).
//  V: the 16 rows are staged in LDS; thread (dim e, token n) writes one
//     element of pool row e, token-fastest, so consecutive slots coalesce.
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

  __shared__ float vstage[kBlock][D + 1];

  const int h = blockIdx.y;
  const int n0 = blockIdx.x * kBlock;
  const int tid = threadIdx.x;

  // ---- K ----
  for (int w = tid; w < NCH * kBlock; w += 256) {
    const int c = w / kBlock, nn = w % kBlock, n = n0 + nn;
    if (n >= num_tokens) continue;
    const int64_t slot = slots[n];
    if (slot < 0 || slot >= capacity) continue;
    const int64_t blk = slot / kBlock;
    const int off = (int)(slot - blk * kBlock);
    char *dst = (char *)kc + (blk * num_kv_heads + h) * (int64_t)TILE + (int64_t)c * (kBlock * 16) +
                off * 16;
    const char *src = (const char *)key + (((int64_t)n * num_kv_heads + h) * D + (int64_t)c * E) * IB;
    if constexpr (KV != KV_FP8) {
      *(uint4 *)dst = *(const uint4 *)src;
    } else {
      uint32_t out[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t word = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int e = q * 4 + b;
          float x;
          if constexpr (IN == KV_BF16) x = __uint_as_float((uint32_t)((const uint16_t *)src)[e] << 16);
          else x = ((const float *)src)[e];
          word |= e4m3_encode(x / k_scale) << (8 * b);
        }
        out[q] = word;
      }
      *(uint4 *)dst = make_uint4(out[0], out[1], out[2], out[3]);
    }
  }

  // ---- V: stage the 16 rows as floats (exact for fp32 and bf16 inputs) ----
  for (int w = tid; w < kBlock * D; w += 256) {
    const int nn = w / D, e = w % D, n = n0 + nn;
    float x = 0.0f;
    if (n < num_tokens) {
      const int64_t idx = ((int64_t)n * num_kv_heads + h) * D + e;
      if constexpr (IN == KV_BF16) x = __uint_as_float((uint32_t)((const uint16_t *)value)[idx] << 16);
      else x = ((const float *)value)[idx];
    }
    vstage[nn][e] = x;
  }
  __syncthreads();
  for (int w = tid; w < kBlock * D; w += 256) {
    const int e = w / kBlock, nn = w % kBlock, n = n0 + nn;
    if (n >= num_tokens) continue;
    const int64_t slot = slots[n];
    if (slot < 0 || slot >= capacity) continue;
    const int64_t blk = slot / kBlock;
    const int off = (int)(slot - blk * kBlock);
    const int64_t idx = ((blk * num_kv_heads + h) * D + e) * kBlock + off;  // element index
    const float x = vstage[nn][e];
    if constexpr (KV == KV_F32) {
      ((float *)vc)[idx] = x;
    } else if constexpr (KV == KV_BF16) {
      ((uint16_t *)vc)[idx] = (uint16_t)(__float_as_uint(x) >> 16);  // exact: x came from bf16
    } else {
      ((uint8_t *)vc)[idx] = (uint8_t)e4m3_encode(x / v_scale);
    }
  }
}

template <int IN, int KV>
static hipError_t write_dispatch_d(const pa_kv_pool &p, const void *key, const void *value,
                                   const int64_t *slots, int32_t T, hipStream_t s) {
  const dim3 grid((T + kBlock - 1) / kBlock, p.num_kv_heads);
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
