// MFMA attention for prefill / chunked-prefill rows (requests with many new
// tokens), bf16 pool, head_dim 128.
//
// What is computed ("vLLM 推理流程分析" §6.2 and §10.1; "vLLM 源码完全拆解（十六）"
// third walk-through path): every new token t of a request with seq_len L and
// c new tokens attends causally over keys 0 .. L - c + t, read from the paged
// pool through the block table (earlier chunks' history included), with a
// softmax stabilised by the running maximum.
//
// Work decomposition (gfx950): a workgroup (4 waves) owns 128 "columns" of one
// (request, kv head); column k is query row (token k / g, head k % g), so the
// GQA heads that share a kv head share every K/V tile.  The workgroup walks
// 64-key tiles; each tile is gathered from 4 pool blocks into LDS (K as
// [key][dim], V as [dim][key] -- the V tile is already dimension-major in the
// pool, so no transpose is needed), double-buffered so the next tile's loads
// overlap this tile's math.  Each wave owns 32 columns and computes
//   S^T (64 keys x 32 cols) = K (64 x 128) . Q^T (128 x 32)
//   O^T (128 dims x 32 cols) += V^T (128 x 64) . P^T (64 x 32)
// with v_mfma_f32_32x32x16_bf16.  Keeping the column index on the lane makes
// the online softmax a per-lane affair (one exchange with lane^32 for the
// max).  P is rounded to bf16 for the second product.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kExtD = 128;
constexpr int kTileKeys = 64;
constexpr int kKPitch = kExtD * 2 + 16;        // bytes per key row of the K tile in LDS
// bytes per dim row of the V tile in LDS: 136 = 34 banks, so the 16 rows read
// together by an 8-byte LDS read land on 16 distinct bank pairs
constexpr int kVPitch = kTileKeys * 2 + 8;
constexpr int kKBytes = kTileKeys * kKPitch;   // 17408
constexpr int kVBytes = kExtD * kVPitch;       // 18432
constexpr int kBufBytes = kKBytes + kVBytes;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__global__ __launch_bounds__(256, 2) void k_extend(const ExtendArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const ExtendItem item = a.items[blockIdx.x];
  const int req = uniform(item.req), kvh = uniform(item.kvh), tok0 = uniform(item.tok0);
  const int c = uniform(item.c), L = uniform(item.L), col0 = uniform(item.col0);
  const int g = a.g;
  const int ncols = c * g;
  const int hist = L - c;                       // tokens before this step's first new token

  // key range of the workgroup and of this wave
  const int last_col_wg = min(ncols, col0 + kExtCols) - 1;
  const int kend_wg = a.causal ? hist + last_col_wg / g + 1 : L;
  const int last_col_w = min(ncols, col0 + wave * 32 + 32) - 1;
  const bool wave_active = col0 + wave * 32 < ncols;
  const int kend_w = a.causal ? hist + last_col_w / g + 1 : L;
  const int n_tiles = (kend_wg + kTileKeys - 1) / kTileKeys;

  // this lane's column (clamped to a valid one; invalid columns are not stored)
  const int col_raw = col0 + wave * 32 + (lane & 31);
  const bool col_ok = col_raw < ncols;
  const int col = col_ok ? col_raw : ncols - 1;
  const int t = col / g, hg = col - t * g;
  const int nvis = a.causal ? hist + t + 1 : L;  // visible keys of this column
  const int hsel = lane >> 5;                    // which 8-element k group the lane feeds
  // visible keys of the wave's first column (columns are token-major, so the
  // smallest); tiles below it need no causal mask
  const int wave_first_col = min(col0 + wave * 32, ncols - 1);
  const int wave_min_nvis = a.causal ? hist + wave_first_col / g + 1 : L;

  // Q^T operand: 8 k-steps of 16 dims; lane holds dims 16ks + 8 hsel .. +8
  const uint16_t *qrow = (const uint16_t *)a.q + ((int64_t)(tok0 + t) * a.num_q_heads + kvh * g + hg) * kExtD;
  bf16x8_t qop[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) qop[ks] = as_bf16x8(*(const uint4 *)(qrow + ks * 16 + hsel * 8));

  const int32_t *btrow = a.block_table + (int64_t)req * a.bt_stride;
  const char *kpool = (const char *)a.k_cache;
  const char *vpool = (const char *)a.v_cache;
  constexpr int TILE = kExtD * kBlock * 2;       // bytes per (block, head) tile

  // ---- staging: thread owns 4 K pieces and 4 V pieces (16 B each) per tile ----
  uint4 kst[4], vst[4];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int p = tid + 256 * r;               // piece index 0..1023
      const int b = p >> 8;                      // block within the tile
      const int kpos_blk = kt * kTileKeys + b * kBlock;
      int phys = -1;
      if (kpos_blk < kend_wg) phys = btrow[kpos_blk / kBlock];
      if (phys >= a.num_blocks) phys = -1;
      const int w = p & 255;
      if (phys >= 0) {
        const int64_t tile_off = ((int64_t)phys * a.num_kv_heads + kvh) * TILE;
        kst[r] = *(const uint4 *)(kpool + tile_off + w * 16);     // chunk w/16, key w%16
        uint4 v = *(const uint4 *)(vpool + tile_off + w * 16);    // dim w/2, keys 8(w%2)..+8
        const int key0 = kpos_blk + (w & 1) * 8;
        if (key0 + 8 > kend_wg) {                  // unwritten slots may hold anything
          uint32_t vw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t lo = (key0 + 2 * q < kend_wg) ? (vw[q] & 0xffffu) : 0u;
            const uint32_t hi = (key0 + 2 * q + 1 < kend_wg) ? (vw[q] & 0xffff0000u) : 0u;
            vw[q] = lo | hi;
          }
          v = make_uint4(vw[0], vw[1], vw[2], vw[3]);
        }
        vst[r] = v;
      } else {
        kst[r] = make_uint4(0, 0, 0, 0);
        vst[r] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&](int buf) {
    char *kb = smem + buf * kBufBytes;
    char *vb = kb + kKBytes;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int p = tid + 256 * r;
      const int b = p >> 8, w = p & 255;
      const int kc = w >> 4, kk = w & 15;        // K: chunk, key in block
      *(uint4 *)(kb + (b * kBlock + kk) * kKPitch + kc * 16) = kst[r];
      const int vd = w >> 1, vh = w & 1;         // V: dim, key half
      uint2 *vdst = (uint2 *)(vb + vd * kVPitch + (b * kBlock + vh * 8) * 2);  // 8-byte aligned rows
      vdst[0] = make_uint2(vst[r].x, vst[r].y);
      vdst[1] = make_uint2(vst[r].z, vst[r].w);
    }
  };

  f32x16_t oacc[4];
#pragma unroll
  for (int md = 0; md < 4; ++md)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[md][r] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < n_tiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_tiles) load_tile(kt + 1);     // global loads in flight during the math

    const int kbase = kt * kTileKeys;
    if (wave_active && kbase < kend_w) {
      const char *kb = smem + buf * kBufBytes;
      const char *vb = kb + kKBytes;
      // ---- S^T = K . Q^T ----
      f32x16_t sacc[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[mt][r] = 0.0f;
        const char *krow = kb + (mt * 32 + (lane & 31)) * kKPitch + hsel * 16;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const bf16x8_t aop = as_bf16x8(*(const uint4 *)(krow + ks * 32));
          sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, qop[ks], sacc[mt], 0, 0, 0);
        }
      }
      // ---- online softmax over this tile (column = lane & 31) ----
      // Scores stay unscaled until the exponent (scale > 0 commutes with max);
      // keys past a column's causal limit are masked only on tiles that cross
      // some column's limit.  The reference max m_ref is raised only when a
      // column's maximum exceeds it by more than 2^8 (decided for the whole
      // wave), so O and l are rescaled rarely; exp2(s*c - m_ref) <= 2^8 stays
      // well inside bf16 and fp32, and O / l is unchanged by the choice of
      // reference.
      const bool crosses = kbase + kTileKeys > wave_min_nvis;
      float mt_max = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float sv = sacc[mt][r];
          if (crosses) {
            const int key = kbase + mt * 32 + 8 * (r >> 2) + 4 * hsel + (r & 3);
            sv = key < nvis ? sv : -INFINITY;
            sacc[mt][r] = sv;
          }
          mt_max = fmaxf(mt_max, sv);
        }
      mt_max = fmaxf(mt_max, __shfl_xor(mt_max, 32, 64));
      const float cand = mt_max * a.scale_log2;      // this tile's max, log2 units
      const bool raise = cand > m_run + 8.0f;
      if (__builtin_amdgcn_ballot_w64(raise) != 0) {  // wave-uniform: rescale
        const float m_new = raise ? cand : m_run;
        const float alpha = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int md = 0; md < 4; ++md)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[md][r] *= alpha;
        m_run = m_new;
      }
      const float neg_m = m_run == -INFINITY ? 0.0f : -m_run;  // fully masked column: p = 0
      float psum = 0.0f;
      uint32_t pp[2][8];                          // P^T as bf16 pairs, [mt][r/2]
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[mt][r], a.scale_log2, neg_m));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[mt][r + 1], a.scale_log2, neg_m));
          psum += p0 + p1;
          pp[mt][r >> 1] = pack_bf16x2(p0, p1);
        }
      l_run += psum;
      // ---- O^T += V^T . P^T ----
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int mt = ks >> 1, half = ks & 1;
        const uint4 pb = make_uint4(pp[mt][half * 4 + 0], pp[mt][half * 4 + 1], pp[mt][half * 4 + 2],
                                    pp[mt][half * 4 + 3]);
        const bf16x8_t bop = as_bf16x8(pb);
#pragma unroll
        for (int md = 0; md < 4; ++md) {
          const char *vrow = vb + (md * 32 + (lane & 31)) * kVPitch + (ks * 16 + 4 * hsel) * 2;
          const uint2 lo = *(const uint2 *)vrow;          // keys 16ks + 4h + 0..3
          const uint2 hi = *(const uint2 *)(vrow + 16);   // keys 16ks + 8 + 4h + 0..3
          const bf16x8_t aop = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
          oacc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, bop, oacc[md], 0, 0, 0);
        }
      }
    }
    if (kt + 1 < n_tiles) {
      // buf ^ 1 was last read in the previous iteration, which every wave
      // finished before that iteration's closing barrier
      store_tile(buf ^ 1);
      __syncthreads();
    }
  }

  if (!wave_active) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (!col_ok) return;
  const float inv = 1.0f / l_tot;
  uint16_t *orow = (uint16_t *)a.out + ((int64_t)(tok0 + t) * a.num_q_heads + kvh * g + hg) * kExtD;
#pragma unroll
  for (int md = 0; md < 4; ++md)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int dim = md * 32 + 8 * q + 4 * hsel;  // rows r = 4q .. 4q+3
      const uint32_t w0 = pack_bf16x2(oacc[md][4 * q] * inv, oacc[md][4 * q + 1] * inv);
      const uint32_t w1 = pack_bf16x2(oacc[md][4 * q + 2] * inv, oacc[md][4 * q + 3] * inv);
      *(uint2 *)(orow + dim) = make_uint2(w0, w1);
    }
}

hipError_t launch_extend(const pa_kv_pool &p, const ExtendArgs &a, hipStream_t s) {
  if (a.n_items == 0) return hipSuccess;
  if (p.kv_dtype != PA_BF16 || p.head_dim != kExtD) return hipErrorNotSupported;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void *)k_extend, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       2 * kBufBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  prof_begin("k_extend", s);
  hipLaunchKernelGGL(k_extend, dim3(a.n_items), dim3(256), 2 * kBufBytes, s, a);
  prof_end(s);
  return hipGetLastError();
}

}  // namespace pa
