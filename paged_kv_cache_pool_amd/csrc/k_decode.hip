// Token-parallel split-K attention over the paged pool (decode tokens, and
// any query row the plan does not give to the MFMA extend kernel), plus the
// merge of partial results.  The vector-ALU kernel below serves fp32 pools
// (fp32 arithmetic end to end); bf16 and fp8 pools use the matrix-core
// version of the same work items, k_decode_mfma.
//
// What is computed ("vLLM 源码完全拆解（十六）", third walk-through path): for a
// query row q of kv head kvh, the keys are walked through the block table
// (paging only changes where K/V come from); s_j = scale * q.k_j, and the
// softmax is stabilised by the running maximum.  The key range of a row may
// be cut into partitions; each yields (m_r, l_r, o_r) and k_merge rescales
// every partial by exp(m_r - m) before summing (the V2 partitioned form the
// same section describes).  Scores are kept in log2 units (the scale is
// pre-multiplied by log2 e) so exp becomes v_exp_f32.
//
// Work decomposition (gfx950, wave64): one wave owns one (item, kv head):
// all g query heads of that kv head over keys [kv_begin, kv_end), so every
// K/V byte is loaded once for the whole GQA group.
//  QK:  lane l scores key (it + l) of the 64-key step; it loads that key's
//       row as 16-byte chunks (the K tile is chunk-major, so the 16 lanes of
//       a block read 256 contiguous bytes per chunk) and dots it with the q
//       chunks, which are uniform across the wave and come from the scalar
//       cache.  No cross-lane reduction is needed for the dot products.
//  softmax: one wave-max per head per 64 keys; p goes to LDS.
//  PV:  lane l loads 16-byte vectors of the dimension-major V tile (one dim,
//       KPV consecutive keys) and accumulates o[dim] += p * v for its dims;
//       the p values of those keys are read back from LDS.  Lanes that share
//       a dim (bf16: 2, fp32: 4) are summed once at the end.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

template <int KV, int D, int G>
__global__ __launch_bounds__(256) void k_decode(const DecodeArgs a) {
  const StagingRelease staging_release{a.release};
  constexpr int PB = KvTraits<KV>::bytes;     // pool element bytes
  constexpr int E = 16 / PB;                  // elements per 16-byte vector
  constexpr int NCH = D / E;                  // K chunks per key row
  constexpr int TILE = D * kBlock * PB;       // bytes per (block, head) tile
  constexpr int KPV = E;                      // keys per V vector (one dim)
  constexpr int VPR = kBlock / KPV;           // V vectors per dim row
  constexpr int NVL = TILE / 1024;            // V loads per lane per tile
  constexpr int DSTEP = 64 / VPR;             // dims covered by one V load across the wave
  static_assert(NVL >= 1 && NCH >= 1, "tile shape");

  __shared__ float lds_p[kWavesPerGroup][G][kKeysPerIter];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int unit = blockIdx.x * kWavesPerGroup + wave;
  if (unit >= a.n_items * a.num_kv_heads) return;
  const int item_idx = unit / a.num_kv_heads;
  const int kvh = unit - item_idx * a.num_kv_heads;
  const DecodeItem item = a.items[item_idx];
  const int token = uniform(item.token), req = uniform(item.req);
  const int kv_begin = uniform(item.kv_begin), kv_end = uniform(item.kv_end);
  const int part = uniform(item.part);
  const int g = a.g;
  const int qh0 = kvh * a.g_total + a.h0;     // first q head of this wave

  const int32_t *__restrict__ btrow = a.block_table + (int64_t)req * a.bt_stride;
  const char *__restrict__ kbase = (const char *)a.k_cache;
  const char *__restrict__ vbase = (const char *)a.v_cache;

  // q rows of this wave's heads (uniform addresses -> scalar loads)
  const char *__restrict__ qbase = (const char *)a.q + ((int64_t)token * a.num_q_heads + qh0) * D *
                                                           (KV == KV_F32 ? 4 : 2);

  // KV update (items with wpos >= 0): the row is its request's only new
  // token, at position wpos = kv_end - 1.  The key loop below stops before
  // it; the new key then enters the softmax as one more step, with the value
  // the pool will hold (the scatter's own encoding), and its K/V rows are
  // stored into the pool at the end.  No wave reads that slot in this launch.
  // The new key's inputs are loaded here, before the loop, so that their
  // latency overlaps the loop's first loads; they are used after the loop.
  // Lane l handles K/V dims l + 64 j of the new rows, and the V dims of its
  // own accumulators.
  const int wpos = uniform(item.wpos);
  const bool wnew = wpos >= 0 && a.knew != nullptr;
  const int kv_last = wnew ? kv_end - 1 : kv_end;   // end of the keys read from the pool
  constexpr int IN = KV == KV_F32 ? KV_F32 : KV_BF16;  // new rows come in the query dtype
  constexpr int IB = KvTraits<IN>::bytes;
  constexpr int KD = D / 64;
  constexpr bool VSAME = VPR == 1 && DSTEP == 64 && NVL == KD;  // accumulator dims = l + 64 j
  constexpr int NO = VSAME ? 1 : NVL;
  constexpr bool QPRE = KV != KV_F32 && G <= 8;      // q of the new key also loaded early
  auto load_in = [](const char *row, int e) -> uint32_t {
    if constexpr (IB == 2) return ((const uint16_t *)row)[e];
    else return ((const uint32_t *)row)[e];
  };
  // (seeded with a run-time zero, not a constant, so that the compiler does
  // not fold the later conversions into this branch and wait for the loads)
  uint32_t kraw[KD], vraw[KD], oraw[NO], qraw[QPRE ? G : 1][KD];
  const uint32_t rz = (uint32_t)a.zero;
#pragma unroll
  for (int j2 = 0; j2 < KD; ++j2) kraw[j2] = vraw[j2] = rz;
#pragma unroll
  for (int i = 0; i < NO; ++i) oraw[i] = rz;
#pragma unroll
  for (int h = 0; h < (QPRE ? G : 1); ++h)
#pragma unroll
    for (int j2 = 0; j2 < KD; ++j2) qraw[h][j2] = rz;
  const char *krow = (const char *)a.knew, *vrow = (const char *)a.vnew;
  // block of the new slot (a block id outside the pool: no write and no key,
  // as for a key the loop reads; the separate scatter skips such slots too)
  const int wblk = wnew ? btrow[wpos / kBlock] : -1;
  if (wnew) {
    const int64_t th = (int64_t)token * a.num_kv_heads + kvh;
    krow += th * D * IB;
    vrow += th * D * IB;
#pragma unroll
    for (int j2 = 0; j2 < KD; ++j2) {
      kraw[j2] = load_in(krow, lane + 64 * j2);
      vraw[j2] = load_in(vrow, lane + 64 * j2);
    }
    if constexpr (!VSAME) {
#pragma unroll
      for (int i = 0; i < NVL; ++i) oraw[i] = load_in(vrow, i * DSTEP + lane / VPR);
    }
    if constexpr (QPRE) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int j2 = 0; j2 < KD; ++j2)
          qraw[h][j2] = load_in(qbase + ((int64_t)(h < g ? h : 0) * D + lane + 64 * j2) * IB, 0);
    }
  }

  float m_run[G], l_run[G], o[G][NVL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.0f;
#pragma unroll
    for (int i = 0; i < NVL; ++i) o[h][i] = 0.0f;
  }

  // block ids of the step's four blocks (lane l: block l / 16), read one
  // step ahead so that the K/V loads never wait for the block table
  const int tl = lane >> 4;                         // which of the 4 blocks
  int phys_next = (kv_begin + tl * kBlock) < kv_last ? btrow[(kv_begin >> 4) + tl] : -1;
  for (int it = kv_begin; it < kv_last; it += kKeysPerIter) {
    const int j = it + lane;                        // this lane's key position
    int phys = phys_next;
    if (phys >= a.num_blocks) phys = -1;            // out-of-range id: never dereferenced
    {
      const int itn = it + kKeysPerIter;
      phys_next = (itn + tl * kBlock) < kv_last ? btrow[(itn >> 4) + tl] : -1;
    }
    const bool key_ok = phys >= 0 && j < kv_last;

    // ---- K row of this lane's key ----
    uint4 kr[NCH];
    if (phys >= 0) {
      const char *kp = kbase + ((int64_t)phys * a.num_kv_heads + kvh) * TILE + (lane & 15) * 16;
#pragma unroll
      for (int c = 0; c < NCH; ++c) kr[c] = *(const uint4 *)(kp + c * (kBlock * 16));
    } else {
#pragma unroll
      for (int c = 0; c < NCH; ++c) kr[c] = make_uint4(0, 0, 0, 0);
    }

    // ---- V vectors of the 4 blocks (issued before the QK math) ----
    int vphys[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) vphys[t] = readlane(phys, t * 16);
    uint4 vr[4][NVL];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (vphys[t] >= 0) {
        const char *vp = vbase + ((int64_t)vphys[t] * a.num_kv_heads + kvh) * TILE + lane * 16;
#pragma unroll
        for (int i = 0; i < NVL; ++i) vr[t][i] = *(const uint4 *)(vp + i * 1024);
      } else {
#pragma unroll
        for (int i = 0; i < NVL; ++i) vr[t][i] = make_uint4(0, 0, 0, 0);
      }
    }

    // ---- scores ----
    float s[G];
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const uint4 kc = kr[c];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const int hh = h < g ? h : 0;
        if constexpr (KV == KV_BF16) {
          const uint4 qv = *(const uint4 *)(qbase + ((int64_t)hh * D + c * E) * 2);
          s[h] = dot2_bf16(qv.x, kc.x, s[h]);
          s[h] = dot2_bf16(qv.y, kc.y, s[h]);
          s[h] = dot2_bf16(qv.z, kc.z, s[h]);
          s[h] = dot2_bf16(qv.w, kc.w, s[h]);
        } else if constexpr (KV == KV_F32) {
          const float4 qv = *(const float4 *)(qbase + ((int64_t)hh * D + c * E) * 4);
          s[h] = fmaf(qv.x, __uint_as_float(kc.x), s[h]);
          s[h] = fmaf(qv.y, __uint_as_float(kc.y), s[h]);
          s[h] = fmaf(qv.z, __uint_as_float(kc.z), s[h]);
          s[h] = fmaf(qv.w, __uint_as_float(kc.w), s[h]);
        } else {
          // 16 E4M3 codes -> 8 exact bf16 pairs (every E4M3 value is a bf16 value)
          const uint4 q0 = *(const uint4 *)(qbase + ((int64_t)hh * D + c * E) * 2);
          const uint4 q1 = *(const uint4 *)(qbase + ((int64_t)hh * D + c * E + 8) * 2);
          const uint32_t kw[4] = {kc.x, kc.y, kc.z, kc.w};
          const uint32_t qw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const f32x2_t lo = fp8x2_to_f32(kw[w], false), hi = fp8x2_to_f32(kw[w], true);
            s[h] = dot2_bf16(qw[2 * w], pack_bf16x2(lo.x, lo.y), s[h]);
            s[h] = dot2_bf16(qw[2 * w + 1], pack_bf16x2(hi.x, hi.y), s[h]);
          }
        }
      }
    }

    // ---- online softmax (log2 domain) ----
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float sv = key_ok ? s[h] * a.scale_log2 : -INFINITY;
      const float mt = wave_max_dpp(sv);
      const float mn = fmaxf(m_run[h], mt);
      const bool any = mn != -INFINITY;
      const float alpha = any ? __builtin_amdgcn_exp2f(m_run[h] - mn) : 1.0f;
      const float p = any ? __builtin_amdgcn_exp2f(sv - mn) : 0.0f;
      l_run[h] = l_run[h] * alpha + p;
#pragma unroll
      for (int i = 0; i < NVL; ++i) o[h][i] *= alpha;
      m_run[h] = mn;
      lds_p[wave][h][lane] = p;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- PV ----
    const bool tail = it + kKeysPerIter > kv_last;
    const int key0 = (lane % VPR) * KPV;            // first key (in block) of this lane's vectors
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (vphys[t] < 0) continue;
      const int kpos0 = it + t * 16 + key0;        // position of the vectors' first key
      float v[NVL][KPV];
#pragma unroll
      for (int i = 0; i < NVL; ++i) {
        const uint4 w4 = vr[t][i];
        const uint32_t ww[4] = {w4.x, w4.y, w4.z, w4.w};
        if constexpr (KV == KV_BF16) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            v[i][2 * q] = bf16_lo(ww[q]);
            v[i][2 * q + 1] = bf16_hi(ww[q]);
          }
        } else if constexpr (KV == KV_F32) {
#pragma unroll
          for (int q = 0; q < 4; ++q) v[i][q] = __uint_as_float(ww[q]);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x2_t lo = fp8x2_to_f32(ww[q], false), hi = fp8x2_to_f32(ww[q], true);
            v[i][4 * q] = lo.x;
            v[i][4 * q + 1] = lo.y;
            v[i][4 * q + 2] = hi.x;
            v[i][4 * q + 3] = hi.y;
          }
        }
        if (tail) {
#pragma unroll
          for (int k = 0; k < KPV; ++k)
            if (kpos0 + k >= kv_last) v[i][k] = 0.0f;  // unwritten slots may hold anything
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float pk[KPV];
#pragma unroll
        for (int k4 = 0; k4 < KPV; k4 += 4) {
          const float4 pv = *(const float4 *)&lds_p[wave][h][t * 16 + key0 + k4];
          pk[k4] = pv.x;
          pk[k4 + 1] = pv.y;
          pk[k4 + 2] = pv.z;
          pk[k4 + 3] = pv.w;
        }
#pragma unroll
        for (int i = 0; i < NVL; ++i) {
          float acc = o[h][i];
#pragma unroll
          for (int k = 0; k < KPV; ++k) acc = fmaf(pk[k], v[i][k], acc);
          o[h][i] = acc;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- the new key (KV update), then its rows into the pool ----
  if (wnew && kvh == 0 && lane == 0 && a.slots_out)
    a.slots_out[token] = (int64_t)wblk * kBlock + wpos % kBlock;
  if (wnew && wblk >= 0 && wblk < a.num_blocks) {
    uint32_t kbits[KD], vbits[KD];
    float kval[KD], vval[NVL];
#pragma unroll
    for (int j2 = 0; j2 < KD; ++j2) {
      kbits[j2] = pool_bits<IN, KV>(kraw[j2], a.enc_k_scale);
      vbits[j2] = pool_bits<IN, KV>(vraw[j2], a.enc_v_scale);
      kval[j2] = pool_value<KV>(kbits[j2]);
    }
#pragma unroll
    for (int i = 0; i < NVL; ++i) {
      if constexpr (VSAME) vval[i] = pool_value<KV>(vbits[i]);
      else vval[i] = pool_value<KV>(pool_bits<IN, KV>(oraw[i], a.enc_v_scale));
    }
    const bool vlane = lane % VPR == 0;             // one lane per dim adds the new key's p * v
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float sp = 0.0f;
#pragma unroll
      for (int j2 = 0; j2 < KD; ++j2) {
        uint32_t qb;
        if constexpr (QPRE) qb = qraw[h][j2];
        else qb = load_in(qbase + ((int64_t)(h < g ? h : 0) * D + lane + 64 * j2) * IB, 0);
        sp = fmaf(in_to_f32<IN>(qb), kval[j2], sp);
      }
      const float sv = wave_sum_dpp(sp) * a.scale_log2;
      const float mn = fmaxf(m_run[h], sv);
      const bool any = mn != -INFINITY;
      const float alpha = any ? __builtin_amdgcn_exp2f(m_run[h] - mn) : 1.0f;
      const float p = any ? __builtin_amdgcn_exp2f(sv - mn) : 0.0f;
      l_run[h] = l_run[h] * alpha + (lane == 0 ? p : 0.0f);
#pragma unroll
      for (int i = 0; i < NVL; ++i) o[h][i] = o[h][i] * alpha + (vlane ? p * vval[i] : 0.0f);
      m_run[h] = mn;
    }
    // the rows into the pool: element e of the K tile sits in chunk e / E at
    // position e % E of slot off's 16 bytes; of the V tile, in row e
    const int off = wpos % kBlock;
    char *kt = (char *)a.k_store + ((int64_t)wblk * a.num_kv_heads + kvh) * TILE;
    char *vt = (char *)a.v_store + ((int64_t)wblk * a.num_kv_heads + kvh) * TILE;
#pragma unroll
    for (int j2 = 0; j2 < KD; ++j2) {
      const int e = lane + 64 * j2;
      char *kd = kt + (e / E) * (kBlock * 16) + off * 16 + (e % E) * PB;
      char *vd = vt + (e * kBlock + off) * PB;
      if constexpr (PB == 4) {
        *(uint32_t *)kd = kbits[j2];
        *(uint32_t *)vd = vbits[j2];
      } else if constexpr (PB == 2) {
        *(uint16_t *)kd = (uint16_t)kbits[j2];
        *(uint16_t *)vd = (uint16_t)vbits[j2];
      } else {
        *(uint8_t *)kd = (uint8_t)kbits[j2];
        *(uint8_t *)vd = (uint8_t)vbits[j2];
      }
    }
  }

  // ---- combine lanes that share dims; totals ----
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int i = 0; i < NVL; ++i) {
#pragma unroll
      for (int x = 1; x < VPR; x <<= 1) o[h][i] += __shfl_xor(o[h][i], x, 64);
    }
    l_run[h] = wave_sum_dpp(l_run[h]);
  }

  if (lane % VPR != 0) return;
  const int drow = lane / VPR;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (h >= g) break;
    const int qh = qh0 + h;
    if (part < 0) {
      const float inv = 1.0f / l_run[h];
#pragma unroll
      for (int i = 0; i < NVL; ++i) {
        const int e = i * DSTEP + drow;
        const float val = o[h][i] * inv * a.v_scale;
        const int64_t idx = ((int64_t)token * a.num_q_heads + qh) * D + e;
        if constexpr (KV == KV_F32) ((float *)a.out)[idx] = val;
        else ((uint16_t *)a.out)[idx] = f32_to_bf16(val);
      }
    } else {
      float *po = a.part_o + ((int64_t)part * a.num_q_heads + qh) * D;
#pragma unroll
      for (int i = 0; i < NVL; ++i) po[i * DSTEP + drow] = o[h][i] * a.v_scale;
      if (lane == 0) {
        float *pml = a.part_ml + ((int64_t)part * a.num_q_heads + qh) * 2;
        pml[0] = m_run[h];
        pml[1] = l_run[h];
      }
    }
  }
}

// The merge as a launch of its own: one wave per (merge item, q head).
template <int D, bool F32OUT>
__global__ __launch_bounds__(256) void k_merge(const MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int unit = blockIdx.x * 4 + wave;
  if (unit >= a.n_items * a.num_q_heads) return;
  const int item_idx = unit / a.num_q_heads;
  const int qh = unit - item_idx * a.num_q_heads;
  const MergeItem it = a.inline_items ? a.inl[item_idx] : a.items[item_idx];
  merge_unit<D, F32OUT>(uniform(it.first), uniform(it.count), uniform(it.token), qh, a.num_q_heads, a.part_ml,
                        a.part_o, a.out, lane);
}

template <int KV, int D>
static hipError_t decode_g(const DecodeArgs &a, int g_tmpl, hipStream_t s) {
  const int units = a.n_items * a.num_kv_heads;
  const dim3 grid((units + kWavesPerGroup - 1) / kWavesPerGroup);
  switch (g_tmpl) {
    case 1: hipLaunchKernelGGL((k_decode<KV, D, 1>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_decode<KV, D, 2>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_decode<KV, D, 4>), grid, dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL((k_decode<KV, D, 8>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((k_decode<KV, D, 16>), grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const pa_kv_pool &p, pa_dtype q_dtype, const DecodeArgs &a, int g_tmpl,
                         hipStream_t s) {
  (void)q_dtype;
  if (a.n_items == 0) return hipSuccess;
  prof_begin("k_decode", s);
  hipError_t e;
  if (p.kv_dtype == PA_BF16 || p.kv_dtype == PA_FP8_E4M3)
    e = launch_decode_mfma(p, a, s);
  else
    e = p.head_dim == 128 ? decode_g<KV_F32, 128>(a, g_tmpl, s) : decode_g<KV_F32, 64>(a, g_tmpl, s);
  prof_end(s);
  return e;
}

hipError_t launch_merge(pa_dtype q_dtype, int head_dim, const MergeArgs &a, hipStream_t s) {
  if (a.n_items == 0) return hipSuccess;
  const int units = a.n_items * a.num_q_heads;
  const dim3 grid((units + 3) / 4);
  prof_begin("k_merge", s);
  if (q_dtype == PA_F32) {
    if (head_dim == 128) hipLaunchKernelGGL((k_merge<128, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_merge<64, true>), grid, dim3(256), 0, s, a);
  } else {
    if (head_dim == 128) hipLaunchKernelGGL((k_merge<128, false>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_merge<64, false>), grid, dim3(256), 0, s, a);
  }
  prof_end(s);
  return hipGetLastError();
}

}  // namespace pa
