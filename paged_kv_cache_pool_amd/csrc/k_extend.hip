// MFMA attention for prefill / chunked-prefill rows (requests with many new
// tokens), bf16 pool, head_dim 128.
//
// What is computed ("vLLM 推理流程分析" §6.2 and §10.1; "vLLM 源码完全拆解（十六）"
// third walk-through path): every new token t of a request with seq_len L and
// c new tokens attends causally over keys 0 .. L - c + t, read from the paged
// pool through the block table (earlier chunks' history included), with a
// softmax stabilised by a running maximum.
//
// Work decomposition (gfx950).  A workgroup of 8 waves owns 128 "columns" of
// one (request, kv head); column k is query row (token k / g, head k % g), so
// the GQA heads that share a kv head share every K/V tile.  The keys are cut
// into 64-key tiles (four pool blocks) taken in pairs: waves 0-3 compute the
// even tile of each pair and waves 4-7 the odd one, for the same 4 x 32
// columns, and the two partial (m, l, O) of a column are merged in LDS at the
// end, so that the longest items of a causal chunk are half as long.  Each
// wave computes, for its 32 columns,
//   S^T (64 keys x 32 cols)   = K (64 x 128) . Q^T (128 x 32)
//   O^T (128 dims x 32 cols) += V^T (128 x 64) . P^T (64 x 32)
// on v_mfma_f32_32x32x16_bf16.  The column index stays on the lane, so the
// online softmax needs one exchange with lane^32.  P is rounded to bf16 for
// the second product.
//
// Data movement.  Tiles are copied from the pool straight into LDS with the
// direct global->LDS load (no staging registers) into a ring of two pairs
// (128 KB): one pair is computed while the next is in flight.  Q of the 128
// columns rides the first pair's copies.
//
// LDS layouts (per stage: K 16 KB + V^T 16 KB):
//  K:   row r holds key swap_bits23(r) of the tile; its 16-byte chunk c sits
//       in slot c ^ (r & 15).  The row permutation makes the MFMA output rows
//       of one lane the keys 8*hsel .. 8*hsel+7 of each 16-key group, so the
//       V operand below is one 16-byte read.
//  V^T: [tile block b][dim d][16 keys], 32 bytes per (b, d); the 16-byte
//       half h (keys 8h .. 8h+7) sits at position h ^ ((d >> 2) ^ (d >> 3)) & 1.
//       Each block's part is a permutation of the pool's (block, head) V
//       tile, so one 1 KB copy instruction reads 1 KB of one pool tile.
// A 16-byte LDS read is served 16 lanes at a time over 64 four-byte banks;
// both swizzles put the 16 rows that one pass reads on distinct banks (on
// gfx950 a conflict-free read of 1 KB takes about 5 clocks, a two-way
// conflicted one 8).
// The copy writes lane i's 16 bytes at base + 16 i, so each lane's source
// address is chosen to produce these layouts.
//
// The wide launch (k_extend_wide) also runs the wide layout (256 columns
// per workgroup, below) and, after its extend items, workgroups that merge
// the split-K partials of the same call (merge_unit), so that the merge needs
// no launch of its own.
#include <mutex>
#include <vector>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kXD = 128;                        // head dim
constexpr int kXT = 64;                         // keys per tile
constexpr int kXStages = 4;
constexpr int kXLds = 128 * 1024;               // ring (<= 128 KB), Q, epilogue staging

// Per pool dtype (bf16, fp8): bytes of a K row and of the K / V^T halves of a
// stage in LDS, and pool bytes of one (block, head) tile.
template <int KV>
struct XLayout {
  static constexpr int PB = KvTraits<KV>::bytes;
  static constexpr int kRow = kXD * PB;         // 256 / 128
  static constexpr int kKBytes = kXT * kRow;    // 16 KB / 8 KB
  static constexpr int kStage = 2 * kKBytes;    // K + V^T
  static constexpr int kTileB = kXD * kBlock * PB;
  static constexpr int kCopies = kKBytes / 8 / 1024;  // 1 KB copies per wave per half of a tile
};
static_assert(kXStages * XLayout<KV_BF16>::kStage <= kXLds, "ring fits");
static_assert(kExtCols == 128, "4 column blocks of 32, each split over two waves");

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }
// half-row swizzle of dim d in the LDS V^T tile, and byte offset of (dim d, tile key k)
__device__ __forceinline__ int vt_swz(int d) { return ((d >> 2) ^ (d >> 3)) & 1; }
__device__ __forceinline__ int vt_offset(int d, int k) {
  return (k >> 4) * 4096 + d * 32 + ((((k >> 3) & 1) ^ vt_swz(d)) * 16) + (k & 7) * 2;
}
// fp8 V^T tile: [tile block b][dim d][16 keys], one byte per key (the pool's
// own block tile layout).
__device__ __forceinline__ int vt8_offset(int d, int k) { return (k >> 4) * 2048 + d * 16 + (k & 15); }

// 8 E4M3 codes -> 8 bf16 values (exact: every E4M3 value is a bf16 value).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16x8(uint2 u) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u.x, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u.x, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u.y, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u.y, 1.0f, true);
  return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// 16 bytes per lane from base + off (global) to LDS at lds_base + 16 * lane;
// base and lds_base are wave-uniform.  Written as inline asm so that the
// compiler does not see an LDS write and does not drain every copy in flight
// before the next LDS read: completion is handled explicitly (s_waitcnt
// vmcnt + barrier) by the caller.  m0 (the LDS base of the copy) is saved and
// restored; one wait state separates the m0 write from the copy (gfx9 hazard).
__device__ __forceinline__ void copy16_to_lds(const char *base, uint32_t off, char *lds_base) {
  const uint32_t lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)lds_base;
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(off), "s"(base)
      : "memory");
}

// Uniform load through the scalar data path (read-only data).
__device__ __forceinline__ int32_t load_uniform(const int32_t *p) {
  return *(const __attribute__((address_space(4))) int32_t *)p;
}

// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding; expcnt left free).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | (((N >> 4) & 3) << 14));
}

// s_waitcnt lgkmcnt(0) only (vmcnt and expcnt left free).
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }

// Which 8-element k group of a 32x32x16 MFMA operand a lane feeds.
__device__ __forceinline__ int hsel_of(int lane) { return lane >> 5; }

// Workgroup barrier that leaves outstanding vector loads in flight (the
// compiler's __syncthreads waits for every copy first).
__device__ __forceinline__ void barrier_keep_loads() { asm volatile("s_barrier" ::: "memory"); }

// x combined with its value in lane l ^ 32.  v_permlane32_swap of x with
// itself returns, per lane, x and the partner's x (in an order that depends
// on the half), so only symmetric combinations are formed.
__device__ __forceinline__ float max_x32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_x32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Per-lane byte offsets of a wave's MFMA operands inside a stage, computed
// once per kernel.  K (S^T = K . Q^T), k-step ks: row rho = 32 mt +
// (lane & 31) of the permuted tile, 16-byte chunk 2 ks + hsel at its
// swizzled slot; the row block mt adds a constant (kKRowBlk).  The XOR of ks
// with lane bits is not affine in ks, so one offset per ks is kept.  V^T
// (O^T += V^T . P^T): dim d = 32 md + (lane & 31), keys 16 ks + 8 hsel; the
// swizzle bit depends on d's low bits only, so md and ks add constants
// (kVmd, kVks) and one offset serves every read.
template <int KV>
struct XOperands {
  static constexpr int kKRowBlk = 32 * XLayout<KV>::kRow;       // 8192 / 4096
  static constexpr int kVks = KV == KV_BF16 ? 4096 : 2048;
  static constexpr int kVmd = KV == KV_BF16 ? 32 * 32 : 32 * 16;
  int k[8];
  int v;
  __device__ __forceinline__ explicit XOperands(int lane) {
    const int hsel = lane >> 5, r = lane & 31;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if constexpr (KV == KV_BF16) k[ks] = r * 256 + (((2 * ks + hsel) ^ (r & 15)) * 16);
      else k[ks] = r * 128 + ((ks ^ ((r >> 1) & 7)) * 16) + hsel * 8;
    }
    if constexpr (KV == KV_BF16) v = XLayout<KV>::kKBytes + vt_offset(r, 8 * hsel);
    else v = XLayout<KV>::kKBytes + vt8_offset(r, 8 * hsel);
  }
};

// One 64-key tile for this wave's 32 columns: S^T = K . Q^T, online
// softmax, O^T += V^T . P^T.  `mask` (wave-uniform) applies the causal
// limit of each column; it is set only on tiles that cross some column's
// limit (the last one or two of a wave).
template <int KV>
__device__ __forceinline__ void xtile(const char *stg, const XOperands<KV> &op, int kbase, bool mask, int nvis,
                                      int lane, float scale_log2, const bf16x8_t (&qop)[8], f32x16_t (&oacc)[4],
                                      float &m_run, float &l_run) {
  using OP = XOperands<KV>;
  const int hsel = lane >> 5;
  f32x16_t sacc[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[mt][r] = 0.0f;
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {             // the two chains alternate
      const char *ka = stg + op.k[ks] + mt * OP::kKRowBlk;
      bf16x8_t aop;
      if constexpr (KV == KV_BF16) aop = as_bf16x8(*(const uint4 *)ka);
      else aop = fp8x8_to_bf16x8(*(const uint2 *)ka);
      sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, qop[ks], sacc[mt], 0, 0, 0);
    }
  // Schedule: four LDS operand reads ahead, then alternate one MFMA and
  // one read, so each read has about four MFMAs (~128 clocks) to land.
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int i = 0; i < 12; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  __builtin_amdgcn_s_setprio(0);

  // Online softmax (column = lane % 32).  Scores stay unscaled until the
  // exponent (scale > 0 commutes with max).  The reference max is raised
  // only when a column's maximum exceeds it by more than 2^8 (decided for
  // the whole wave), so O and l are rescaled rarely; exp2(s * c - m_ref) <=
  // 2^8 stays well inside bf16 and fp32, and O / l does not depend on the
  // reference.
  if (mask) {
    const int lim = nvis - kbase;              // keys of this tile the column sees
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = swap23(mt * 32 + 8 * (r >> 2) + 4 * hsel + (r & 3));
        sacc[mt][r] = key < lim ? sacc[mt][r] : -INFINITY;
      }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[mt][r]);
  mx = max_x32(mx);
  const float cand = mx * scale_log2;
  const bool raise = cand > m_run + 8.0f;
  if (__builtin_amdgcn_ballot_w64(raise) != 0) {
    const float m_new = raise ? cand : m_run;
    const float alpha = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int md = 0; md < 4; ++md)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[md][r] *= alpha;
    m_run = m_new;
  }
  // P is rounded to bf16 for the PV product, and l sums those rounded
  // values (one v_dot2 with (1, 1) per pair, two chains), so the weights the
  // output is normalised by are exactly the ones it is made of.
  const float neg_m = m_run == -INFINITY ? 0.0f : -m_run;  // fully masked column: p = 0
  constexpr uint32_t kOnes = 0x3F803F80u;      // (1.0, 1.0) in bf16
  float psum0 = 0.0f, psum1 = 0.0f;
  uint32_t pp[2][8];                           // P^T as bf16 pairs [mt][r / 2]
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[mt][r], scale_log2, neg_m));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[mt][r + 1], scale_log2, neg_m));
      pp[mt][r >> 1] = pack_bf16x2(p0, p1);
      if (mt == 0) psum0 = dot2_bf16(pp[mt][r >> 1], kOnes, psum0);
      else psum1 = dot2_bf16(pp[mt][r >> 1], kOnes, psum1);
    }
  l_run += psum0 + psum1;

  // O^T += V^T . P^T (k-step ks covers keys 16 ks .. 16 ks + 15)
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int mt = ks >> 1, half = ks & 1;
    const bf16x8_t bop = as_bf16x8(make_uint4(pp[mt][half * 4 + 0], pp[mt][half * 4 + 1],
                                              pp[mt][half * 4 + 2], pp[mt][half * 4 + 3]));
#pragma unroll
    for (int md = 0; md < 4; ++md) {                // keys 16 ks + 8 hsel .. +8 of dim 32 md + lane % 32
      const char *va = stg + op.v + ks * OP::kVks + md * OP::kVmd;
      bf16x8_t aop;
      if constexpr (KV == KV_BF16) aop = as_bf16x8(*(const uint4 *)va);
      else aop = fp8x8_to_bf16x8(*(const uint2 *)va);
      oacc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, bop, oacc[md], 0, 0, 0);
    }
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
  for (int i = 0; i < 12; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);
  __builtin_amdgcn_s_setprio(0);
}

// PREFIX = false: a prefill chunk of one request (columns = its new tokens x
// GQA heads, causal or not), written to the output.  PREFIX = true: the
// shared-prefix (cascade) pass: columns = the prefix rows (rows of every
// request that shares the common prefix) x GQA heads, keys = one chunk of the
// common prefix, all visible; written as partial (m, l, o) for the merge.
template <int KV, bool PREFIX>
__device__ __forceinline__ void extend_split_body(const ExtendArgs &a, char *smem) {
  using X = XLayout<KV>;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int g = a.g;
  const int hsel = lane >> 5;                    // which 8-element k group the lane feeds
  int kvh, col0, ncols, kspan, kc = 0, hist = 0, tok0 = 0, cnew = 0;
  bool wself = false;                            // the item writes its request's new K/V rows
  const int32_t *btrow;
  if constexpr (PREFIX) {
    const PrefixItem it = a.pitems[blockIdx.x];
    kvh = uniform(it.kvh);
    col0 = uniform(it.col0);
    kc = uniform(it.kc);
    const int key0 = uniform(it.key0), key1 = uniform(it.key1);
    ncols = a.prefix_cols;
    kspan = key1 - key0;                         // keys are counted from key0 (a multiple of 64)
    btrow = a.prefix_bt + key0 / kBlock;
  } else {
    const ExtendItem item = a.items[blockIdx.x];
    const int req = uniform(item.req), c = uniform(item.c), L = uniform(item.L);
    wself = uniform(item.wnew) != 0 && a.knew != nullptr;
    cnew = c;
    kvh = uniform(item.kvh);
    tok0 = uniform(item.tok0);
    col0 = uniform(item.col0);
    ncols = c * g;
    hist = L - c;                                // tokens before this step's first new token
    kspan = L;
    btrow = a.block_table + (int64_t)req * a.bt_stride;
  }
  const bool causal = !PREFIX && a.causal;

  // key range of the workgroup and of this wave (columns are token-major)
  const int last_col_wg = min(ncols, col0 + kExtCols) - 1;
  const int kend_wg = causal ? hist + last_col_wg / g + 1 : kspan;
  const int n_tiles = (kend_wg + kXT - 1) / kXT;
  const int blk_last = (kend_wg - 1) / kBlock;   // last logical block read
  const int grp = wave >> 2;                     // key-split group: even (0) or odd (1) tiles
  const int cw = wave & 3;                       // column block within the workgroup
  const int wcol0 = col0 + cw * 32;
  const bool wave_active = wcol0 < ncols;
  const int kend_w = causal ? hist + (min(ncols, wcol0 + 32) - 1) / g + 1 : kspan;
  const int wave_min_nvis = causal ? hist + min(wcol0, ncols - 1) / g + 1 : kspan;

  // this lane's column (clamped to a valid one; invalid columns are not stored)
  const int col_raw = wcol0 + (lane & 31);
  const int col = min(col_raw, ncols - 1);
  const int nvis = causal ? hist + col / g + 1 : kspan;

  // q / output row (in units of head_dim elements) of workgroup column cc,
  // clamped to a valid column; increasing in cc.
  auto out_row = [&](int cc) -> int64_t {
    const int cg = min(col0 + cc, ncols - 1);
    const int tt = cg / g;
    if constexpr (PREFIX) return (int64_t)a.row_token[tt] * a.num_q_heads + kvh * g + (cg - tt * g);
    else return (int64_t)(tok0 + tt) * a.num_q_heads + kvh * g + (cg - tt * g);
  };
  bf16x8_t qop[8];                               // Q^T operand: dims 16 ks + 8 hsel .. +8 of the lane's column

  const char *kpool = (const char *)a.k_cache + (int64_t)kvh * X::kTileB;
  const char *vpool = (const char *)a.v_cache + (int64_t)kvh * X::kTileB;
  const int64_t bstride = (int64_t)a.num_kv_heads * X::kTileB;

  // Block id of logical block b (uniform).  Blocks past the range repeat the
  // last one and ids outside the pool read block 0: both in bounds, and every
  // key taken from them is masked (K) or zeroed (V) below.
  auto blk_id = [&](int b) -> int {
    const int v = load_uniform(btrow + min(b, blk_last));
    return (v >= 0 && v < a.num_blocks) ? v : 0;
  };
  // This wave's copy share of a tile, all from tile block w / 2, each
  // instruction moving 1 KB of LDS.  bf16: K rows 8 w + 4 u .. +3 and V^T
  // dims 32 (2 w + u) % 128 .. +31 for u = 0, 1.  fp8 (K rows of 128 bytes,
  // chunk c of row r in slot c ^ ((r >> 1) & 7); the V^T block tile is the
  // pool's own): K rows 8 w .. 8 w + 7 and V^T dims 64 (w % 2) .. +63.
  // Per-lane source offsets within the pool tile of a (block, head):
  uint32_t koff[X::kCopies], voff[X::kCopies];
#pragma unroll
  for (int u = 0; u < X::kCopies; ++u) {
    if constexpr (KV == KV_BF16) {
      const int I = wave * 2 + u;
      const int rho = 4 * I + (lane >> 4);
      const int chunk = (lane & 15) ^ (rho & 15);
      koff[u] = chunk * 256 + (swap23(rho) & 15) * 16;
      const int d = 32 * (I & 3) + (lane >> 1);
      const int half = (lane & 1) ^ vt_swz(d);
      voff[u] = d * 32 + half * 16;
    } else {
      const int rho = 8 * wave + (lane >> 3);
      const int chunk = (lane & 7) ^ ((rho >> 1) & 7);
      koff[u] = chunk * 256 + (swap23(rho) & 15) * 16;
      voff[u] = (wave & 1) * 1024 + lane * 16;
    }
  }
  const int my_blk = wave >> 1;
  int next_id = blk_id(my_blk);                  // block id for the next tile to issue
  auto issue = [&](int kt) {
    char *kst = smem + (kt % kXStages) * X::kStage + wave * (X::kCopies * 1024);
    char *vst = kst + X::kKBytes;
    const char *ksrc = kpool + (int64_t)next_id * bstride;
    const char *vsrc = vpool + (int64_t)next_id * bstride;
#pragma unroll
    for (int u = 0; u < X::kCopies; ++u) {
      copy16_to_lds(ksrc, koff[u], kst + u * 1024);
      copy16_to_lds(vsrc, voff[u], vst + u * 1024);
    }
    next_id = blk_id((kt + 1) * 4 + my_blk);
  };

  f32x16_t oacc[4];
#pragma unroll
  for (int md = 0; md < 4; ++md)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[md][r] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;
  const XOperands<KV> xop(lane);

  // Tiles go in pairs (2p, 2p + 1): group 0 computes the even tile, group 1
  // the odd one, for the same columns.  The ring holds two pairs: while pair
  // p is computed, pair p + 1 is in flight.
  const int n_pairs = (n_tiles + 1) / 2;
  auto issue_pair = [&](int p) {
    issue(2 * p);
    if (2 * p + 1 < n_tiles) issue(2 * p + 1);
  };
  // KV update of an item that is the only reader of its request's new rows
  // (one key-split item per kv head): it writes them into the pool itself,
  // with the scatter's encoder, before any tile that holds them is copied.
  if constexpr (!PREFIX) {
    if (wself) {
      constexpr int PB = KvTraits<KV>::bytes, E = 16 / PB, NCH = kXD / E;
      for (int w = tid; w < cnew * NCH; w += 512) {
        const int t = w / NCH, ch = w - t * NCH;
        const int pos = hist + t;
        const int blk = btrow[pos / kBlock];
        const int off = pos % kBlock;
        if (ch == 0 && kvh == 0 && a.slots_out) a.slots_out[tok0 + t] = (int64_t)blk * kBlock + off;
        if (blk < 0 || blk >= a.num_blocks) continue;   // slot outside the pool: not written
        const int64_t th = (int64_t)(tok0 + t) * a.num_kv_heads + kvh;
        const KvChunkIn<KV_BF16, KV> in =
            load_kv_chunk<KV_BF16, KV>((const char *)a.knew + th * kXD * 2, (const char *)a.vnew + th * kXD * 2, ch);
        const int64_t tile = ((int64_t)blk * a.num_kv_heads + kvh) * X::kTileB;
        *(uint4 *)((char *)a.k_store + tile + ch * (kBlock * 16) + off * 16) =
            k_chunk_bits<KV_BF16, KV>(in, a.enc_k_scale);
        char *vt = (char *)a.v_store + tile;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const uint32_t b = v_elem_bits<KV_BF16, KV>(in, e, a.enc_v_scale);
          char *pv = vt + ((ch * E + e) * kBlock + off) * PB;
          if constexpr (PB == 2) *(uint16_t *)pv = (uint16_t)b;
          else *(uint8_t *)pv = (uint8_t)b;
        }
      }
      __builtin_amdgcn_s_waitcnt(0);             // every store of this wave has completed
      __syncthreads();
    }
  }
  // Q of the workgroup's 128 columns is copied into the last 32 KB of LDS
  // (for bf16 pools stage 3, not refilled before pair 1 is issued) together
  // with pair 0: row cc (256 bytes) holds column cc's
  // 16-byte chunk c in slot c ^ (cc & 15), so the operand reads below are
  // conflict-free.  Instruction u of wave w moves columns 4 (4 w + u) .. +3.
  char *qst = smem + kXLds - 32 * 1024;
  {
    const char *qsrc = (const char *)a.q + (int64_t)out_row(0) * (kXD * 2);
    const int64_t row0 = out_row(0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int J = wave * 4 + u;
      const int cc = 4 * J + (lane >> 4);
      const int chunk = (lane & 15) ^ (cc & 15);
      copy16_to_lds(qsrc, (uint32_t)((out_row(cc) - row0) * (kXD * 2) + chunk * 16), qst + J * 1024);
    }
  }
  issue_pair(0);
  for (int p = 0; p < n_pairs; ++p) {
    // Only pair p's copies (and, for p = 0, Q's) are outstanding: wait for
    // them, then the barrier makes every wave's copies visible and
    // guarantees that the stages of pair p - 1, refilled below, are no
    // longer read.
    wait_vm_lgkm0<0>();
    barrier_keep_loads();
    if (p == 0) {
      const int cc = cw * 32 + (lane & 31);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        qop[ks] = as_bf16x8(*(const uint4 *)(qst + cc * 256 + (((2 * ks + hsel) ^ (cc & 15)) * 16)));
      __syncthreads();                           // every wave has Q before stage 3 is refilled
    }
    if (p + 1 < n_pairs) issue_pair(p + 1);
    if (2 * p + 2 >= n_tiles) {
      // Last pair: keys past the range may hold anything (unwritten slots,
      // stand-in blocks); zero their V so that 0 * v stays 0.
      const int tl = n_tiles - 1;
      char *vb = smem + (tl % kXStages) * X::kStage + X::kKBytes;
      const int kv = kend_wg - tl * kXT;
      for (int e = tid; e < kXD * kXT; e += 512) {
        const int d = e >> 6, k = e & 63;
        if (k >= kv) {
          if constexpr (KV == KV_BF16) *(uint16_t *)(vb + vt_offset(d, k)) = 0;
          else *(uint8_t *)(vb + vt8_offset(d, k)) = 0;
        }
      }
      __syncthreads();
    }
    const int kt = 2 * p + grp;
    const int kbase = kt * kXT;
    if (kt >= n_tiles || !wave_active || kbase >= kend_w) continue;
    const char *kb = smem + (kt % kXStages) * X::kStage;
    xtile<KV>(kb, xop, kbase, kbase + kXT > wave_min_nvis, nvis, lane, a.scale_log2, qop, oacc, m_run, l_run);
  }

  // Merge the odd-tile partial (m, l, O) of each column into the even-tile
  // one through LDS (the ring is free once every wave has passed the
  // barrier).  Both are relative to their own reference maxima m_g:
  //   O = O_0 2^(m_0 - m) + O_1 2^(m_1 - m),  l likewise,  m = max(m_0, m_1);
  // m_0 is finite (tile 0, key 0 is visible to every column), m_1 may be
  // -inf when the odd tiles hold no visible key.
  const float l_half = sum_x32(l_run);
  __syncthreads();
  float *xo = (float *)smem;                     // [cw][md * 16 + r][lane]
  float *xm = xo + 4 * 64 * 64;                  // [cw][lane]
  float *xl = xm + 4 * 64;
  if (grp == 1 && wave_active) {
#pragma unroll
    for (int md = 0; md < 4; ++md)
#pragma unroll
      for (int r = 0; r < 16; ++r) xo[(cw * 64 + md * 16 + r) * 64 + lane] = oacc[md][r];
    xm[cw * 64 + lane] = m_run;
    xl[cw * 64 + lane] = l_half;
  }
  __syncthreads();
  // The merged bf16 outputs are staged as [column][dims] rows (pitch 272
  // bytes, so the 8-byte writes of 32 columns spread over the banks) and
  // then written out as whole 256-byte rows.
  constexpr int kOutPitch = kXD * 2 + 16;
  char *ost = smem + 80 * 1024;
  if constexpr (PREFIX) {
    // partial (m, l, o) of this key chunk: o unnormalised, relative to m (log2
    // units), v_scale applied -- the split-K kernel's format
    if (grp == 0 && wave_active && col_raw < ncols) {
      const float m1 = xm[cw * 64 + lane];
      const float m = fmaxf(m_run, m1);
      const float a0 = __builtin_amdgcn_exp2f(m_run - m);
      const float a1 = m1 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m1 - m);
      const int r = col / g;
      const int head = kvh * g + (col - r * g);
      const int64_t slot = (int64_t)a.row_slot0[r] + kc;
      float *po = a.part_o + (slot * a.num_q_heads + head) * kXD;
      const float s0 = a0 * a.v_scale, s1 = a1 * a.v_scale;
#pragma unroll
      for (int md = 0; md < 4; ++md)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int dim = md * 32 + 8 * q + 4 * hsel;  // rows r = 4q .. 4q+3
          float o[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            o[i] = oacc[md][4 * q + i] * s0 + xo[(cw * 64 + md * 16 + 4 * q + i) * 64 + lane] * s1;
          *(float4 *)(po + dim) = make_float4(o[0], o[1], o[2], o[3]);
        }
      if (hsel == 0) {
        float *pml = a.part_ml + (slot * a.num_q_heads + head) * 2;
        pml[0] = m;
        pml[1] = l_half * a0 + xl[cw * 64 + lane] * a1;
      }
    }
    return;
  }
  if (grp == 0 && wave_active) {
    const float m1 = xm[cw * 64 + lane];
    const float m = fmaxf(m_run, m1);
    const float a0 = __builtin_amdgcn_exp2f(m_run - m);
    const float a1 = m1 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m1 - m);
    const float inv = a.v_scale / (l_half * a0 + xl[cw * 64 + lane] * a1);
    const float s0 = a0 * inv, s1 = a1 * inv;
    char *orow = ost + (cw * 32 + (lane & 31)) * kOutPitch;
#pragma unroll
    for (int md = 0; md < 4; ++md)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int dim = md * 32 + 8 * q + 4 * hsel;  // rows r = 4q .. 4q+3
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o[i] = oacc[md][4 * q + i] * s0 + xo[(cw * 64 + md * 16 + 4 * q + i) * 64 + lane] * s1;
        *(uint2 *)(orow + dim * 2) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
      }
  }
  __syncthreads();
  const int ncols_wg = min(kExtCols, ncols - col0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int piece = tid + 512 * i;             // column piece / 16, 16-byte chunk piece % 16
    const int cc = piece >> 4, chunk = piece & 15;
    if (cc < ncols_wg)
      *(uint4 *)((char *)a.out + out_row(cc) * (kXD * 2) + chunk * 16) =
          *(const uint4 *)(ost + cc * kOutPitch + chunk * 16);
  }
}

template <int KV, bool PREFIX>
__global__ __launch_bounds__(512, 1) void k_extend(const ExtendArgs a) {
  const StagingRelease staging_release{a.release};
  extern __shared__ __attribute__((aligned(16))) char smem[];
  extend_split_body<KV, PREFIX>(a, smem);
}

// Wide workgroups for long prefill chunks.  A workgroup of 8 waves owns
// kWideCols = 256 columns of one (request, kv head), one wave per 32
// columns, and every wave takes every 64-key tile of the item's key range
// [key0, min(key1, visible end)).  Each K/V tile copied into LDS then feeds
// twice the columns of the key-split layout above.  Tiles go in steps of two
// through a 4-stage ring with one barrier per step: the barrier at the top
// of a step frees the previous step's two stages, and the next step's tiles
// are copied into them while this step computes.  Q of the 256 columns
// (64 KB) is copied into stage 3 and the 32 KB above the ring together with
// the first step's tiles and moved to registers before stage 3 is refilled.
//
// A request whose items are too long to balance over the compute units is
// cut into key pieces (item.slot0 >= 0): each piece writes partial
// (m, l, o) at partial slot slot0 + token * slot_stride, and the merge
// kernel combines the pieces ("vLLM 源码完全拆解（十六）", third walk-through
// path: partitions of the key range merged by their maxima).
template <int KV>
__global__ __launch_bounds__(512, 1) void k_extend_wide(const ExtendArgs a) {
  const StagingRelease staging_release{a.release};
  using X = XLayout<KV>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  if (blockIdx.x >= (unsigned)a.n_items) {
    // a merge workgroup (the extend items come first, so these run in the
    // launch's tail as compute units free up): one (merge item, q head) per wave
    const int unit = (int)(blockIdx.x - a.n_items) * 8 + wave;
    if (unit < a.n_merge_units) {
      const int mi = unit / a.num_q_heads;
      const int qh = unit - mi * a.num_q_heads;
      const MergeItem it = a.mitems[mi];
      merge_unit<kXD, false>(uniform(it.first), uniform(it.count), uniform(it.token), qh, a.num_q_heads,
                             a.part_ml, a.part_o, a.out, lane);
    }
    return;
  }
  const int g = a.g;
  const ExtendItem item = a.items[blockIdx.x];
  if (uniform(item.mode) != 0) {                 // a key-split item (kExtCols columns)
    extend_split_body<KV, false>(a, smem);
    return;
  }
  const int req = uniform(item.req), c = uniform(item.c), L = uniform(item.L);
  const int kvh = uniform(item.kvh), tok0 = uniform(item.tok0), col0 = uniform(item.col0);
  const int key0 = uniform(item.key0), key1 = uniform(item.key1);
  const int slot0 = uniform(item.slot0), sstride = uniform(item.slot_stride);
  const int ncols = c * g;
  const int hist = L - c;                        // tokens before this step's first new token
  const int32_t *btrow = a.block_table + (int64_t)req * a.bt_stride;
  const bool causal = a.causal;
  // keys [0, vis(cc)) are visible to column cc within this item (key1 caps a piece)
  auto vis = [&](int cc) { return min(key1, causal ? hist + cc / g + 1 : L); };

  const int last_col_wg = min(ncols, col0 + kWideCols) - 1;
  const int kend_wg = vis(last_col_wg);          // key range of the workgroup: [key0, kend_wg)
  const int t_first = key0 / kXT;                // key0 is a multiple of 64
  const int t_end = (kend_wg + kXT - 1) / kXT;
  const int blk_last = (kend_wg - 1) / kBlock;   // last logical block read
  const int wcol0 = col0 + wave * 32;
  const bool wave_active = wcol0 < ncols;
  const int kend_w = wave_active ? vis(min(ncols, wcol0 + 32) - 1) : 0;
  const int wave_min_nvis = vis(min(wcol0, ncols - 1));
  const int col_raw = wcol0 + (lane & 31);
  const int col = min(col_raw, ncols - 1);       // clamped; columns past ncols are not stored
  const int nvis = vis(col);

  // q / output row of workgroup column cc (clamped to a valid column)
  auto out_row = [&](int cc) -> int64_t {
    const int cg = min(col0 + cc, ncols - 1);
    const int tt = cg / g;
    return (int64_t)(tok0 + tt) * a.num_q_heads + kvh * g + (cg - tt * g);
  };

  const char *kpool = (const char *)a.k_cache + (int64_t)kvh * X::kTileB;
  const char *vpool = (const char *)a.v_cache + (int64_t)kvh * X::kTileB;
  const int64_t bstride = (int64_t)a.num_kv_heads * X::kTileB;
  auto blk_id = [&](int b) -> int {
    const int v = load_uniform(btrow + min(b, blk_last));
    return (v >= 0 && v < a.num_blocks) ? v : 0;
  };
  // copy share of a tile: as in the key-split kernel (wave w copies 1 KB
  // pieces of tile block w / 2)
  uint32_t koff[X::kCopies], voff[X::kCopies];
#pragma unroll
  for (int u = 0; u < X::kCopies; ++u) {
    if constexpr (KV == KV_BF16) {
      const int I = wave * 2 + u;
      const int rho = 4 * I + (lane >> 4);
      const int chunk = (lane & 15) ^ (rho & 15);
      koff[u] = chunk * 256 + (swap23(rho) & 15) * 16;
      const int d = 32 * (I & 3) + (lane >> 1);
      const int half = (lane & 1) ^ vt_swz(d);
      voff[u] = d * 32 + half * 16;
    } else {
      const int rho = 8 * wave + (lane >> 3);
      const int chunk = (lane & 7) ^ ((rho >> 1) & 7);
      koff[u] = chunk * 256 + (swap23(rho) & 15) * 16;
      voff[u] = (wave & 1) * 1024 + lane * 16;
    }
  }
  const int my_blk = wave >> 1;
  int next_id = blk_id(t_first * 4 + my_blk);   // block id of the next tile to issue
  // ring stage of tile t: counted from the item's first tile, so that the
  // first step's two tiles never land on stage 3 (Q)
  auto stage = [&](int t) { return (t - t_first) & (kXStages - 1); };
  auto issue = [&](int kt) {
    char *kst = smem + stage(kt) * X::kStage + wave * (X::kCopies * 1024);
    char *vst = kst + X::kKBytes;
    const char *ksrc = kpool + (int64_t)next_id * bstride;
    const char *vsrc = vpool + (int64_t)next_id * bstride;
#pragma unroll
    for (int u = 0; u < X::kCopies; ++u) {
      copy16_to_lds(ksrc, koff[u], kst + u * 1024);
      copy16_to_lds(vsrc, voff[u], vst + u * 1024);
    }
    next_id = blk_id((kt + 1) * 4 + my_blk);
  };

  f32x16_t oacc[4];
#pragma unroll
  for (int md = 0; md < 4; ++md)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[md][r] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;
  const XOperands<KV> xop(lane);
  bf16x8_t qop[8];

  // Q: row cc (256 bytes) holds column cc's 16-byte chunk c in slot
  // c ^ (cc & 15); instruction u of wave w moves columns 4 (8 w + u) .. +3.
  char *qst = smem + 3 * X::kStage;
  {
    const char *qsrc = (const char *)a.q + out_row(0) * (kXD * 2);
    const int64_t row0 = out_row(0);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int J = wave * 8 + u;
      const int cc = 4 * J + (lane >> 4);
      const int chunk = (lane & 15) ^ (cc & 15);
      copy16_to_lds(qsrc, (uint32_t)((out_row(cc) - row0) * (kXD * 2) + chunk * 16), qst + J * 1024);
    }
  }
  issue(t_first);
  if (t_first + 1 < t_end) issue(t_first + 1);
  for (int t = t_first; t < t_end; t += 2) {
    // Tiles go in steps of two with one barrier per step: only this step's
    // copies (and, at the first step, Q's) are outstanding; the barrier makes
    // every wave's copies visible and frees the stages of the previous step,
    // into which the next step's tiles are copied while this step computes.
    wait_vm_lgkm0<0>();
    barrier_keep_loads();
    if (t == t_first) {
      const int cc = wave * 32 + (lane & 31);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        qop[ks] = as_bf16x8(*(const uint4 *)(qst + cc * 256 + (((2 * ks + hsel_of(lane)) ^ (cc & 15)) * 16)));
      wait_lgkm0();
      barrier_keep_loads();                      // every wave holds Q before stage 3 is refilled
    }
    if (t + 2 < t_end) issue(t + 2);
    if (t + 3 < t_end) issue(t + 3);
    if (t + 2 >= t_end && kend_wg < t_end * kXT) {
      // keys past the range may hold anything (unwritten slots, stand-in
      // blocks); zero their V so that 0 * v stays 0
      const int tl = t_end - 1;
      char *vb = smem + stage(tl) * X::kStage + X::kKBytes;
      const int kv = kend_wg - tl * kXT;
      for (int e = tid; e < kXD * kXT; e += 512) {
        const int d = e >> 6, k = e & 63;
        if (k >= kv) {
          if constexpr (KV == KV_BF16) *(uint16_t *)(vb + vt_offset(d, k)) = 0;
          else *(uint8_t *)(vb + vt8_offset(d, k)) = 0;
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int tt = t + u;
      const int kbase = tt * kXT;
      if (tt >= t_end || !wave_active || kbase >= kend_w) continue;
      const char *kb = smem + stage(tt) * X::kStage;
      xtile<KV>(kb, xop, kbase, kbase + kXT > wave_min_nvis, nvis, lane, a.scale_log2, qop, oacc, m_run, l_run);
    }
  }

  const float l_tot = sum_x32(l_run);
  const int hsel = hsel_of(lane);
  if (slot0 >= 0) {
    // a key piece: partial (m, l, o), o unnormalised relative to m (log2
    // units) with v_scale applied -- the split-K kernel's format
    if (!wave_active || col_raw >= ncols) return;
    const int r = col / g;
    const int head = kvh * g + (col - r * g);
    const int64_t slot = (int64_t)slot0 + (int64_t)r * sstride;
    float *po = a.part_o + (slot * a.num_q_heads + head) * kXD;
#pragma unroll
    for (int md = 0; md < 4; ++md)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int dim = md * 32 + 8 * q + 4 * hsel;  // rows r = 4q .. 4q+3
        *(float4 *)(po + dim) = make_float4(oacc[md][4 * q] * a.v_scale, oacc[md][4 * q + 1] * a.v_scale,
                                            oacc[md][4 * q + 2] * a.v_scale, oacc[md][4 * q + 3] * a.v_scale);
      }
    if (hsel == 0) {
      float *pml = a.part_ml + (slot * a.num_q_heads + head) * 2;
      pml[0] = m_run;
      pml[1] = l_tot;
    }
    return;
  }
  // whole range: normalise, stage the bf16 rows in LDS (pitch 272 bytes) and
  // write them out as whole 256-byte rows
  constexpr int kOutPitch = kXD * 2 + 16;
  __syncthreads();                               // every wave is done with the ring
  if (wave_active) {
    const float inv = a.v_scale / l_tot;
    char *orow = smem + (wave * 32 + (lane & 31)) * kOutPitch;
#pragma unroll
    for (int md = 0; md < 4; ++md)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int dim = md * 32 + 8 * q + 4 * hsel;
        *(uint2 *)(orow + dim * 2) = make_uint2(pack_bf16x2(oacc[md][4 * q] * inv, oacc[md][4 * q + 1] * inv),
                                                pack_bf16x2(oacc[md][4 * q + 2] * inv, oacc[md][4 * q + 3] * inv));
      }
  }
  __syncthreads();
  const int ncols_wg = min(kWideCols, ncols - col0);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int piece = tid + 512 * i;             // column piece / 16, 16-byte chunk piece % 16
    const int cc = piece >> 4, chunk = piece & 15;
    if (cc < ncols_wg)
      *(uint4 *)((char *)a.out + out_row(cc) * (kXD * 2) + chunk * 16) =
          *(const uint4 *)(smem + cc * kOutPitch + chunk * 16);
  }
}

// The LDS size above the default limit is a per-device attribute of each
// kernel: set it once for each (kernel, device) the library launches on.
template <int KV, bool PREFIX>
static hipError_t set_lds_attr() {
  static std::mutex mu;
  static std::vector<char> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(mu);
  if ((int)done.size() <= dev) done.resize(dev + 1, 0);
  if (!done[dev]) {
    e = hipFuncSetAttribute((const void *)k_extend<KV, PREFIX>, hipFuncAttributeMaxDynamicSharedMemorySize, kXLds);
    if (e != hipSuccess) return e;
    done[dev] = 1;
  }
  return hipSuccess;
}

template <int KV, bool PREFIX>
static hipError_t launch_t(int n, const ExtendArgs &a, hipStream_t s) {
  hipError_t e = set_lds_attr<KV, PREFIX>();
  if (e != hipSuccess) return e;
  prof_begin(PREFIX ? "k_prefix" : "k_extend", s);
  hipLaunchKernelGGL((k_extend<KV, PREFIX>), dim3(n), dim3(512), kXLds, s, a);
  prof_end(s);
  return hipGetLastError();
}

constexpr int kWLds = 160 * 1024;              // wide kernel: stages 0-2, then Q over stage 3 and above
static_assert(3 * XLayout<KV_BF16>::kStage + 64 * 1024 <= kWLds, "Q fits after three stages");
static_assert(kWideCols * (kXD * 2 + 16) <= kWLds, "output staging fits");

template <int KV>
static hipError_t launch_wide_t(int n, const ExtendArgs &a, hipStream_t s) {
  static std::mutex mu;
  static std::vector<char> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  {
    std::lock_guard<std::mutex> lk(mu);
    if ((int)done.size() <= dev) done.resize(dev + 1, 0);
    if (!done[dev]) {
      e = hipFuncSetAttribute((const void *)k_extend_wide<KV>, hipFuncAttributeMaxDynamicSharedMemorySize, kWLds);
      if (e != hipSuccess) return e;
      done[dev] = 1;
    }
  }
  prof_begin("k_extend", s);
  hipLaunchKernelGGL((k_extend_wide<KV>), dim3(n + (a.n_merge_units + 7) / 8), dim3(512), kWLds, s, a);
  prof_end(s);
  return hipGetLastError();
}

// Wide items (a.items, kWideCols columns each, possibly key pieces).
hipError_t launch_extend_wide(const pa_kv_pool &p, const ExtendArgs &a, hipStream_t s) {
  if (a.n_items == 0) return hipSuccess;
  if (p.head_dim != kXD) return hipErrorNotSupported;
  if (p.kv_dtype == PA_BF16) return launch_wide_t<KV_BF16>(a.n_items, a, s);
  if (p.kv_dtype == PA_FP8_E4M3) return launch_wide_t<KV_FP8>(a.n_items, a, s);
  return hipErrorNotSupported;
}

// The shared-prefix pass: a.n_items prefix items (a.pitems).
hipError_t launch_prefix(const pa_kv_pool &p, const ExtendArgs &a, hipStream_t s) {
  if (a.n_items == 0) return hipSuccess;
  if (p.head_dim != kXD) return hipErrorNotSupported;
  if (p.kv_dtype == PA_BF16) return launch_t<KV_BF16, true>(a.n_items, a, s);
  if (p.kv_dtype == PA_FP8_E4M3) return launch_t<KV_FP8, true>(a.n_items, a, s);
  return hipErrorNotSupported;
}

}  // namespace pa
