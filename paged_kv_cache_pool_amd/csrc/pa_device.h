// Device helpers for the gfx950 kernels of libpa.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// The first kernel a call launches releases the staging buffer of the
// previous call on its stream: while any of its workgroups runs, every
// earlier kernel of the stream has completed.  The lanes of wave 0 of
// workgroup 0 store the flag when they leave the kernel (the same value, a
// wave-uniform condition; a vector store to pinned host memory at system
// scope).  At the exit no load follows the store, so the compiler keeps
// loading the kernel's uniform metadata through the scalar path.
struct StagingRelease {
  int32_t *flag;
  __device__ __forceinline__ ~StagingRelease() {
    if (flag != nullptr && blockIdx.x == 0 && __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 0)
      __hip_atomic_store(flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

enum KvKind { KV_F32 = 0, KV_BF16 = 1, KV_FP8 = 2 };

template <int KV> struct KvTraits;
template <> struct KvTraits<KV_F32> { static constexpr int bytes = 4; };
template <> struct KvTraits<KV_BF16> { static constexpr int bytes = 2; };
template <> struct KvTraits<KV_FP8> { static constexpr int bytes = 1; };

__device__ __forceinline__ float bf16_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// acc + a.lo * b.lo + a.hi * b.hi with bf16 pairs (v_dot2_f32_bf16; products
// exact, fp32 accumulation).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// Two OCP E4M3FN codes (bytes 2*hi_word, 2*hi_word+1 of w) -> two exact floats.
__device__ __forceinline__ f32x2_t fp8x2_to_f32(uint32_t w, bool hi_word) {
  return hi_word ? __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true)
                 : __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
}

// OCP E4M3FN encoder (software, integer arithmetic), written from the format:
// 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, exponent field 0
// subnormal (m * 2^-9), largest finite magnitude 448 (code 0x7E), code 0x7F
// (and 0xFF) NaN, no infinity.  Rounding: nearest, ties to even; magnitudes
// of 448 or more saturate to 448; NaN encodes as 0x7F.  Branch-free: the
// normal, subnormal, saturated and NaN codes are all formed and one is
// selected (early returns made the compiler emit four nested branches per
// element, each with its exec-mask bookkeeping).
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  // normal codes (2^-6 <= |y| < 448): exponent 1..15 and the top 3 mantissa
  // bits, rounded half to even on the 20 dropped bits (a carry into the
  // exponent is the correct next code)
  const uint32_t code_n = (((a >> 23) - 120u) << 3) | ((a >> 20) & 7u);
  const uint32_t rem = a & 0xfffffu;
  const uint32_t up = (rem > 0x80000u ? 1u : 0u) | (rem == 0x80000u ? (code_n & 1u) : 0u);
  // subnormal codes (|y| < 2^-6): |y| / 2^-9 rounded to the nearest integer,
  // ties to even (0..8; 8 is the smallest normal, whose code is also 8)
  const uint32_t code_s = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  uint32_t code = a < 0x3c800000u ? code_s : code_n + up;
  code = a >= 0x43e00000u ? 0x7eu : code;       // >= 448 (incl. inf)
  return a > 0x7f800000u ? 0x7fu : (sign | code);
}

// ---------------------------------------------------------------------------
// Pool encoding of new K/V elements.  Every writer of new rows (the scatter
// kernel, its plan-driven variant and the decode kernel's own-token write)
// derives the stored bits with pool_bits(), so the pool bytes do not depend on
// which of them wrote a token.  IN / KV are the input and pool element kinds.
// ---------------------------------------------------------------------------

// Input element bits (a bf16 or an fp32 word, zero-extended) as a float.
template <int IN>
__device__ __forceinline__ float in_to_f32(uint32_t raw) {
  if constexpr (IN == KV_BF16) return __uint_as_float(raw << 16);
  else return __uint_as_float(raw);
}

// Stored bits of one element: the input bits for a same-dtype pool, the
// E4M3FN code of x / scale (fp32 division) for an fp8 pool.
template <int IN, int KV>
__device__ __forceinline__ uint32_t pool_bits(uint32_t raw, float scale) {
  static_assert(IN != KV_FP8, "fp8 is a pool format only");
  static_assert(KV == KV_FP8 || IN == KV, "same-dtype copy or fp8 encode");
  if constexpr (KV == KV_FP8) return e4m3_encode(in_to_f32<IN>(raw) / scale);
  else return raw;
}

// The value the attention kernels compute with for stored bits (fp8: the
// code's own value; the per-tensor scale is applied outside the dot products).
template <int KV>
__device__ __forceinline__ float pool_value(uint32_t bits) {
  if constexpr (KV == KV_FP8) return fp8x2_to_f32(bits, false).x;
  else return in_to_f32<KV>(bits);
}

// One 16-byte pool chunk of a new token's K and V rows for one kv head: the
// elements c*E .. c*E+E-1 of the head's input rows (E = 16 / pool element
// bytes).  The K chunk is 16 contiguous bytes of the chunk-major K tile; the
// same dims of V go to rows c*E .. of the dimension-major V tile, one element
// per row.
template <int IN, int KV> struct KvChunkIn {
  static constexpr int IB = KvTraits<IN>::bytes;
  static constexpr int E = 16 / KvTraits<KV>::bytes;
  static constexpr int NV = E * IB / 16;   // 16-byte input vectors per chunk
  uint4 k[NV], v[NV];
};

template <int IN, int KV>
__device__ __forceinline__ KvChunkIn<IN, KV> load_kv_chunk(const void *key_row, const void *value_row,
                                                           int c) {
  using In = KvChunkIn<IN, KV>;
  In r;
  const uint4 *ks = (const uint4 *)((const char *)key_row + (int64_t)c * In::E * In::IB);
  const uint4 *vs = (const uint4 *)((const char *)value_row + (int64_t)c * In::E * In::IB);
#pragma unroll
  for (int i = 0; i < In::NV; ++i) {
    r.k[i] = ks[i];
    r.v[i] = vs[i];
  }
  return r;
}

// Input element e of a chunk (zero-extended bits).
template <int IN, int KV>
__device__ __forceinline__ uint32_t chunk_elem(const uint4 *words4, int e) {
  const uint32_t *words = (const uint32_t *)words4;
  if constexpr (KvTraits<IN>::bytes == 2) return (words[e / 2] >> (16 * (e & 1))) & 0xffffu;
  else return words[e];
}

// The 16 stored bytes of a K chunk.
template <int IN, int KV>
__device__ __forceinline__ uint4 k_chunk_bits(const KvChunkIn<IN, KV> &in, float k_scale) {
  constexpr int PB = KvTraits<KV>::bytes;
  constexpr int E = 16 / PB;
  uint32_t out[4] = {0, 0, 0, 0};
#pragma unroll
  for (int e = 0; e < E; ++e)
    out[e * PB / 4] |= pool_bits<IN, KV>(chunk_elem<IN, KV>(in.k, e), k_scale) << (8 * ((e * PB) & 3));
  return make_uint4(out[0], out[1], out[2], out[3]);
}

// Stored bits of element e of a V chunk.
template <int IN, int KV>
__device__ __forceinline__ uint32_t v_elem_bits(const KvChunkIn<IN, KV> &in, int e, float v_scale) {
  return pool_bits<IN, KV>(chunk_elem<IN, KV>(in.v, e), v_scale);
}

// Stores chunk c of slot offset `off` of the (block, head) tiles whose byte
// offset in k_cache / v_cache is `tile`.
template <int IN, int KV, int D>
__device__ __forceinline__ void store_kv_chunk(const KvChunkIn<IN, KV> &in, void *kc, void *vc,
                                               int64_t tile, int off, int c, float k_scale,
                                               float v_scale) {
  constexpr int PB = KvTraits<KV>::bytes;
  constexpr int E = 16 / PB;
  constexpr int S = 16;                      // slots per block
  char *kdst = (char *)kc + tile + (int64_t)c * (S * 16) + off * 16;
  char *vdst = (char *)vc + tile + ((int64_t)c * E * S + off) * PB;  // row c*E, column off
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t vb = v_elem_bits<IN, KV>(in, e, v_scale);
    if constexpr (PB == 4) ((uint32_t *)vdst)[e * S] = vb;
    else if constexpr (PB == 2) ((uint16_t *)vdst)[e * S] = (uint16_t)vb;
    else ((uint8_t *)vdst)[e * S] = (uint8_t)vb;
  }
  *(uint4 *)kdst = k_chunk_bits<IN, KV>(in, k_scale);
}

// One block segment of the scatter of new rows, for one kv head h: tokens
// tok0 .. tok0 + count - 1 (count <= 16) of request req, at positions pos0 ..
// in logical block pos0 / 16, go to slots block_table[req * bt_stride + pos0 /
// 16] * 16 + pos0 % 16 + t (also stored to slots_out when it is set and
// h == 0); a block id outside the pool leaves the pool untouched.  NT threads
// (tid 0 .. NT - 1) of one workgroup; vt: LDS for the head's V tile.
//  K: one thread per (token, 16-byte chunk), one 16-byte store each (the
//     chunks of consecutive slots are contiguous in the chunk-major tile);
//  V: the tokens' elements are first placed in LDS in the tile's own
//     dimension-major layout, then the tile is written as 16-byte vectors;
//     a vector that also covers slots outside the segment is written
//     element by element, leaving the other slots untouched.
// The input rows are read before the block id: they depend on the segment
// only, so both reads are in flight together and the workgroup waits for one
// round trip instead of two.
template <int IN, int KV, int D, int NT>
__device__ __forceinline__ void scatter_segment(int req, int tok0, int pos0, int count, int h, int num_kv_heads,
                                                const void *key, const void *value, const int32_t *block_table,
                                                int64_t bt_stride, int num_blocks, void *k_cache, void *v_cache,
                                                float k_scale, float v_scale, int64_t *slots_out, uint8_t *vt,
                                                int tid) {
  constexpr int S = 16;                          // slots per block
  constexpr int IB = KvTraits<IN>::bytes;
  constexpr int PB = KvTraits<KV>::bytes;
  constexpr int E = 16 / PB;                     // elements per 16 bytes of the pool
  constexpr int NCH = D / E;                     // chunks per key row
  constexpr int TILE = D * S * PB;               // bytes of one (block, head) tile
  constexpr int NVEC = TILE / 16;                // 16-byte vectors per tile
  constexpr int NIT = (S * NCH + NT - 1) / NT;   // chunks per thread
  const int off0 = pos0 % S;
  KvChunkIn<IN, KV> in[NIT];
#pragma unroll
  for (int k = 0; k < NIT; ++k) {
    const int w = tid + NT * k;
    if (w < count * NCH) {
      const int t = w / NCH, c = w % NCH;
      const int64_t th = (int64_t)(tok0 + t) * num_kv_heads + h;
      in[k] = load_kv_chunk<IN, KV>((const char *)key + th * D * IB, (const char *)value + th * D * IB, c);
    }
  }
  asm volatile("" ::: "memory");                 // the rows' reads are issued before the block id's
  const int blk = block_table[(int64_t)req * bt_stride + pos0 / S];
  const bool in_pool = blk >= 0 && blk < num_blocks;   // else the slots are not written
  const int64_t tile = ((int64_t)blk * num_kv_heads + h) * TILE;
#pragma unroll
  for (int k = 0; k < NIT; ++k) {
    const int w = tid + NT * k;
    if (w >= count * NCH) continue;
    const int t = w / NCH, c = w % NCH;
    if (in_pool)
      *(uint4 *)((char *)k_cache + tile + c * (S * 16) + (off0 + t) * 16) = k_chunk_bits<IN, KV>(in[k], k_scale);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t b = v_elem_bits<IN, KV>(in[k], e, v_scale);
      uint8_t *p = vt + ((c * E + e) * S + off0 + t) * PB;
      if constexpr (PB == 4) *(uint32_t *)p = b;
      else if constexpr (PB == 2) *(uint16_t *)p = (uint16_t)b;
      else *p = (uint8_t)b;
    }
  }
  if (slots_out && h == 0 && tid < count) slots_out[tok0 + tid] = (int64_t)blk * S + off0 + tid;
  __syncthreads();
  if (!in_pool) return;                          // (uniform: every thread returns)
  // a vector holds E consecutive slots of one dim row
  char *vdst = (char *)v_cache + tile;
  for (int w = tid; w < NVEC; w += NT) {
    const int s0 = (w * E) % S;                  // first slot of the vector
    if (s0 >= off0 && s0 + E <= off0 + count) {
      *(uint4 *)(vdst + w * 16) = *(const uint4 *)(vt + w * 16);
    } else if (s0 + E > off0 && s0 < off0 + count) {
      for (int e = 0; e < E; ++e) {
        const int sl = s0 + e;
        if (sl < off0 || sl >= off0 + count) continue;
        const int o = w * 16 + e * PB;
        if constexpr (PB == 4) *(uint32_t *)(vdst + o) = *(const uint32_t *)(vt + o);
        else if constexpr (PB == 2) *(uint16_t *)(vdst + o) = *(const uint16_t *)(vt + o);
        else vdst[o] = (char)vt[o];
      }
    }
  }
}

// Wave-wide reductions (64 lanes).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__device__ __forceinline__ int readlane(int x, int lane) {
  return __builtin_amdgcn_readlane(x, lane);
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load the compiler may neither hoist nor batch with its neighbours
// (used for LDS data that is re-read every step instead of kept in registers).
__device__ __forceinline__ uint4 load16_volatile(const void *p) {
  const u32x4_t v = *(const volatile u32x4_t *)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}

}  // namespace pa

namespace pa {

// DPP lane movements (gfx9 encodings).
constexpr int kDppQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppRowHalfMirror = 0x141; // lane i of 8 <- lane 7 - i
constexpr int kDppRowMirror = 0x140;     // lane i of 16 <- lane 15 - i

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// All 16 lanes of each row end with the row's max / sum (butterfly over the
// row: lane ^ 1, lane ^ 2, the other quad, the other half-row).
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp_f32<kDppQuadSwap1>(x));
  x = fmaxf(x, dpp_f32<kDppQuadSwap2>(x));
  x = fmaxf(x, dpp_f32<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp_f32<kDppRowMirror>(x));
  return x;
}

__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_f32<kDppQuadSwap1>(x);
  x += dpp_f32<kDppQuadSwap2>(x);
  x += dpp_f32<kDppRowHalfMirror>(x);
  x += dpp_f32<kDppRowMirror>(x);
  return x;
}

__device__ __forceinline__ float lane_f32(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// Wave-wide max / sum, result uniform (row results combined through readlane).
__device__ __forceinline__ float wave_max_dpp(float x) {
  x = row_max16(x);
  return fmaxf(fmaxf(lane_f32(x, 0), lane_f32(x, 16)), fmaxf(lane_f32(x, 32), lane_f32(x, 48)));
}

__device__ __forceinline__ float wave_sum_dpp(float x) {
  x = row_sum16(x);
  return (lane_f32(x, 0) + lane_f32(x, 16)) + (lane_f32(x, 32) + lane_f32(x, 48));
}

// Merge of partitions: one wave per (token, q head).  Every lane reads one
// partition's (m, l) (64 per round), so the maximum and the weights come from
// one wave reduction instead of a chain of dependent loads; the partial
// outputs are then summed with the weights.  Partials first .. first + count
// - 1 of q head qh (m in log2 units, l, o with v_scale applied) -> output row
// `token`.  Lanes are split into PPI groups of D / 4 lanes; group s takes
// partials r = s, s + PPI, ... and each of its lanes 4 dims of them (one float4
// per partial), so one load instruction reads PPI whole partials and each lane
// keeps U of them in flight.
template <int D, bool F32OUT>
__device__ __forceinline__ void merge_unit(int first, int count, int token, int qh, int num_q_heads,
                                           const float *part_ml, const float *part_o, void *out, int lane) {
  constexpr int LPP = D / 4;                     // lanes per partial
  constexpr int PPI = 64 / LPP;                  // partials per load instruction
  constexpr int U = 8;
  const float *ml = part_ml + ((int64_t)first * num_q_heads + qh) * 2;
  const int64_t ml_stride = (int64_t)num_q_heads * 2;

  const int sub = lane / LPP, d4 = lane % LPP;
  const float *po = part_o + ((int64_t)first * num_q_heads + qh) * D + 4 * d4;
  const int64_t po_stride = (int64_t)num_q_heads * D;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  float m = -INFINITY, l = 0.0f;
  if (count <= PPI * U && count <= 64) {
    // few partials (the usual case): every read (the partial outputs and both
    // (m, l) layouts) is issued at once, so the merge waits for one round trip
    float4 v[U];
    float mr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = sub + u * PPI;
      const int rc = r < count ? r : 0;          // in range; its weight is dropped below
      v[u] = *(const float4 *)(po + rc * po_stride);
      mr[u] = r < count ? ml[rc * ml_stride] : -INFINITY;
    }
    const float m_lane = lane < count ? ml[lane * ml_stride] : -INFINITY;
    const float l_lane = lane < count ? ml[lane * ml_stride + 1] : 0.0f;
    m = wave_max_dpp(m_lane);
    l = wave_sum_dpp(m_lane != -INFINITY ? fmaf(__builtin_amdgcn_exp2f(m_lane - m), l_lane, 0.0f) : 0.0f);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w = mr[u] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mr[u] - m);
      acc.x = fmaf(w, v[u].x, acc.x);
      acc.y = fmaf(w, v[u].y, acc.y);
      acc.z = fmaf(w, v[u].z, acc.z);
      acc.w = fmaf(w, v[u].w, acc.w);
    }
  } else {
    // m = max_r m_r, l = sum_r 2^(m_r - m) l_r (a partial without keys has m_r = -inf)
    for (int r0 = 0; r0 < count; r0 += 64)
      if (r0 + lane < count) m = fmaxf(m, ml[(r0 + lane) * ml_stride]);
    m = wave_max_dpp(m);
    for (int r0 = 0; r0 < count; r0 += 64) {
      const int r = r0 + lane;
      if (r < count) {
        const float mr = ml[r * ml_stride];
        if (mr != -INFINITY) l = fmaf(__builtin_amdgcn_exp2f(mr - m), ml[r * ml_stride + 1], l);
      }
    }
    l = wave_sum_dpp(l);

    // O = sum_r 2^(m_r - m) o_r / l
    for (int r0 = sub; r0 < count; r0 += PPI * U) {
      float4 v[U];
      float mr[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = r0 + u * PPI;
        const int rc = r < count ? r : r0;         // in range; its weight is dropped below
        v[u] = *(const float4 *)(po + rc * po_stride);
        mr[u] = r < count ? ml[rc * ml_stride] : -INFINITY;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float w = mr[u] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mr[u] - m);
        acc.x = fmaf(w, v[u].x, acc.x);
        acc.y = fmaf(w, v[u].y, acc.y);
        acc.z = fmaf(w, v[u].z, acc.z);
        acc.w = fmaf(w, v[u].w, acc.w);
      }
    }
  }
  // sum the PPI groups (lanes d4, d4 + LPP, ...)
#pragma unroll
  for (int o = LPP; o < 64; o <<= 1) {
    acc.x += __shfl_xor(acc.x, o, 64);
    acc.y += __shfl_xor(acc.y, o, 64);
    acc.z += __shfl_xor(acc.z, o, 64);
    acc.w += __shfl_xor(acc.w, o, 64);
  }
  if (sub != 0) return;
  const float inv = 1.0f / l;
  const int64_t idx = ((int64_t)token * num_q_heads + qh) * D + 4 * d4;
  if constexpr (F32OUT) {
    *(float4 *)((float *)out + idx) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  } else {
    uint2 w2;
    w2.x = (uint32_t)f32_to_bf16(acc.x * inv) | ((uint32_t)f32_to_bf16(acc.y * inv) << 16);
    w2.y = (uint32_t)f32_to_bf16(acc.z * inv) | ((uint32_t)f32_to_bf16(acc.w * inv) << 16);
    *(uint2 *)((uint16_t *)out + idx) = w2;
  }
}

}  // namespace pa
