// Token-parallel split-K attention on the matrix cores, for bf16 and fp8
// pools: the same computation and the same work items as k_decode (a wave
// per (item, kv head), or per pair of items below; all g <= 16 query heads
// of the kv head over keys
// [kv_begin, kv_end) walked through the block table, online softmax in log2
// units, partial (m, l, o) for split rows; "vLLM 源码完全拆解（十六）", third
// walk-through path), with the dot products moved from the vector ALUs to
// v_mfma_f32_16x16x32_bf16.  The wave's q heads are the 16 MFMA columns
// (columns g .. 15 are zero), so per 64-key step
//   S   (16 keys x 16 heads)   = K   (16 keys x 32 dims) . Q^T (32 dims x 16 heads), D/32 slices, 4 times
//   O^T (16 dims x 16 heads)  += V^T (16 dims x 32 keys) . P^T (32 keys x 16 heads), D/16 dim groups, twice
// Lane l = n + 16 j holds column (head) n = l & 15 of every result, so one
// head's softmax lives in the four lanes n, n + 16, n + 32, n + 48 and is
// combined with two lane swaps (v_permlane16_swap / v_permlane32_swap).
//
// Key order.  Row r of S-product u = 2c + h of a step is the key at offset
// 8 ((r >> 2) & 1) + 4 h + (r & 3) of block 2c + (r >> 3).  Lane group j then
// receives, over the two products of pair c, the scores of keys 32c + 8j ..
// 32c + 8j + 7 of the step: exactly the k-slots of lane group j in the P^T
// operand of PV chunk c.  So P needs no exchange between lanes, and the V^T
// operand of (chunk c, dim d) is one read of the 8 consecutive keys of dim
// row d of one block tile (16 bytes for bf16, 8 for fp8).  A K read is 64
// contiguous bytes per (block, chunk, 4 keys).
//
// fp8 pools: K and V codes become bf16 in registers (exact: every E4M3 value
// is a bf16 value); the K scale is folded into the score scale, the V scale is
// applied to the output, as in k_decode.  The probabilities are rounded to
// bf16 for the PV product, and l sums the rounded values, so the output is
// normalised by exactly the weights it is made of.
//
// Loads: bf16 K/V tiles are read non-temporally (each byte is read once per
// row); measured faster on the bf16 decode workloads (up to 6 % when prefill
// data fills the caches), and slower on the fp8 pool, which keeps plain loads.
//
// Pipelining: the next step's K is read as soon as this step's S products have
// consumed the K registers, and the next step's V as soon as the PV products
// have consumed V, so a wave always has one step's K or V in flight while it
// computes.  Block ids are read two steps ahead.
//
// Pairs (PAIR): one wave per SIMD runs two items (token pieces) in turn; the
// second item's first K/V are read into spare registers at the start, so it
// begins without a wait.  The kernel then holds up to 512 registers (one
// wave per SIMD); the single-item form keeps two waves per SIMD.
//
// KV update (items with wpos >= 0, the row's own new token at position
// kv_end - 1): the new key enters the softmax with the value the pool will
// hold (the scatter's own encoding; before the key loop, or after it in the
// paired form), and its K/V rows are stored into the pool; the key loop
// stops before it.  No wave reads that slot in this launch.  One-wave
// workgroups appended after the decode units may also scatter other
// requests' new rows (prefill chunks read only by the extend kernel, which
// runs after this launch).
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// 16 bytes from global memory, non-temporal (streamed: each K/V byte of a
// decode row is read once, so it is not kept in the caches at the expense of
// data that is reused).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const void *p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4_t *)p));
}

// 8 E4M3 codes -> 8 bf16 values (exact)
__device__ __forceinline__ bf16x8_t fp8x8_bf16(uint32_t lo, uint32_t hi) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// x combined with the value of lane l ^ 16 (rows of 16 lanes swapped in
// pairs), and with lane l ^ 32 (halves swapped)
__device__ __forceinline__ float max_x16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_x32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_x16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_x32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace

constexpr int kDecodeWaves = 1;                // waves (work units) per workgroup

// NH: column halves.  A launch whose items have at most 16 (row, head)
// columns runs NH = 1; items of up to 32 columns (kind 1) run NH = 2, where
// every K and V operand feeds two products (columns 0-15 and 16-31) and each
// half keeps its own softmax state.  (With NH = 2 the paired form does not
// pre-read the second item's first step: the registers go to the second
// half.)
template <int KV, int D, bool PAIR, int NH>
__global__ __launch_bounds__(64 * kDecodeWaves) __attribute__((amdgpu_waves_per_eu(PAIR || NH == 2 ? 1 : 2))) void k_decode_mfma(const DecodeArgs a) {
  const StagingRelease staging_release{a.release};
  static_assert(KV == KV_BF16 || KV == KV_FP8, "bf16 and fp8 pools");
  static_assert(NH == 1 || NH == 2, "one or two column halves");
  constexpr bool F8 = KV == KV_FP8;
  constexpr bool PREFETCH = PAIR && NH == 1;     // the second item's first step read at the start
  // the new key after the key loop in the paired form (one wave per SIMD):
  // measured 4 % faster on the decode layer; the single-item forms keep it
  // first (two waves per SIMD: registers for its inputs are short, and the
  // fp8 shared-prefix step was 2 % slower with it last)
  constexpr bool LATE_KEY = PAIR;
  constexpr int PB = KvTraits<KV>::bytes;
  constexpr int E = 16 / PB;                     // elements per 16-byte K chunk row
  constexpr int TILE = D * kBlock * PB;          // bytes per (block, head) tile
  constexpr int NS = D / 32;                     // k-slices of the S product
  constexpr int NDG = D / 16;                    // dim groups of the PV product
  constexpr int NKX = F8 ? NS / 2 : NS;          // 16-byte K reads per S product
  constexpr int VROW = kBlock * PB;              // bytes of one dim row of a V tile
  using VReg = std::conditional_t<F8, uint2, uint4>;
  static_assert(NS >= 2 && NKX >= 1, "head_dim 64 or 128");

  const int lane = threadIdx.x & 63;
  const int r = lane & 15;                       // MFMA column within a half / A-operand row
  const int j = lane >> 4;                       // lane group
  const int wave = uniform(threadIdx.x >> 6);
  const int unit = blockIdx.x * kDecodeWaves + wave;
  // PAIR: wave (bin, kv head) runs item bin, then item pair_stride + bin when
  // there is one.  Otherwise one item per wave.
  const int n_first = PAIR ? a.pair_stride : a.n_items;
  if (unit >= n_first * a.num_kv_heads) {
    // Workgroups after the decode units run in the launch's tail, as compute
    // units free up.  Scatter workgroups write new rows that no decode unit
    // reads (instead of a launch of their own before this one); copy
    // workgroups move the later launches' work lists into device memory.
    const int u = unit - n_first * a.num_kv_heads;
    if (u >= a.n_wseg_units) {
      // four loads per lane in flight (indices clamped to the last vector,
      // so every read is in bounds), then the stores of the valid ones
      static_assert(kCopyVecsPerUnit == 256, "four vectors per lane");
      const int v0 = (u - a.n_wseg_units) * kCopyVecsPerUnit;
      const int n = min(kCopyVecsPerUnit, a.copy_vecs - v0);
      const uint4 *src = a.copy_src + v0;
      uint4 *dst = a.copy_dst + v0;
      const uint4 x0 = src[min(lane, n - 1)], x1 = src[min(64 + lane, n - 1)];
      const uint4 x2 = src[min(128 + lane, n - 1)], x3 = src[min(192 + lane, n - 1)];
      if (lane < n) dst[lane] = x0;
      if (64 + lane < n) dst[64 + lane] = x1;
      if (128 + lane < n) dst[128 + lane] = x2;
      if (192 + lane < n) dst[192 + lane] = x3;
    } else {
      __shared__ __attribute__((aligned(16))) uint8_t vt[TILE];
      const int h = u % a.num_kv_heads;
      const WriteSeg sg = a.wseg[u / a.num_kv_heads];
      scatter_segment<KV_BF16, KV, D, 64>(sg.req, sg.tok0, sg.pos0, sg.count, h, a.num_kv_heads, a.knew, a.vnew,
                                          a.block_table, a.bt_stride, a.num_blocks, a.k_store, a.v_store,
                                          a.enc_k_scale, a.enc_v_scale, a.slots_out, vt, threadIdx.x);
    }
    return;
  }
  const int bin = unit / a.num_kv_heads;
  const int kvh = unit - bin * a.num_kv_heads;
  const int g = a.g;
  const int qh0 = kvh * a.g_total + a.h0;        // q head of a column with head index 0
  const char *__restrict__ kbase = (const char *)a.k_cache + (int64_t)kvh * TILE;
  const char *__restrict__ vbase = (const char *)a.v_cache + (int64_t)kvh * TILE;
  const int64_t bstride = (int64_t)a.num_kv_heads * TILE;   // bytes between blocks

  // first of the 8 dims that lane group j holds in k-slice c (the K read
  // layout decides it: bf16 reads one 8-dim chunk row per slice, fp8 one
  // 16-dim chunk row per two slices)
  auto qdim = [&](int c) { return F8 ? 64 * (c >> 1) + 16 * j + 8 * (c & 1) : 32 * c + 8 * j; };

  // lane-constant parts of the addresses
  const int kofs = j * (kBlock * 16) + (8 * ((r >> 2) & 1) + (r & 3)) * 16;   // + 64 h + 1024 x
  const int vofs = r * VROW + (j & 1) * 8 * PB;                              // + 16 VROW dg
  const int ksel = r >> 3, vsel = j >> 1;        // which block of a pair

  uint4 kr[4][NKX];                              // [S product u][read x]
  VReg vr[2][NDG];                               // [chunk c][dim group]
  // the second item's first step (PREFETCH), read during the first item's
  // start, from the block ids pb0 .. pb3
  uint4 kr2[PREFETCH ? 4 : 1][NKX];
  VReg vr2[PREFETCH ? 2 : 1][NDG];
  int pb0 = -1, pb1 = -1, pb2 = -1, pb3 = -1;
  // block of pair c that a lane reads (b0 .. b3: the step's four block ids)
  auto pick = [](int sel, int lo, int hi) { return sel ? hi : lo; };
  auto issue_k = [&](uint4 (&kd)[4][NKX], int b0, int b1, int b2, int b3) {
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const int p = c2 == 0 ? pick(ksel, b0, b1) : pick(ksel, b2, b3);
      const char *kp = kbase + (int64_t)(p < 0 ? 0 : p) * bstride + kofs;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int x = 0; x < NKX; ++x)
          kd[2 * c2 + h][x] = F8 ? *(const uint4 *)(kp + 64 * h + 1024 * x) : load_stream(kp + 64 * h + 1024 * x);
    }
  };
  auto issue_v = [&](VReg (&vd)[2][NDG], int b0, int b1, int b2, int b3) {
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const int p = c2 == 0 ? pick(vsel, b0, b1) : pick(vsel, b2, b3);
      const char *vp = vbase + (int64_t)(p < 0 ? 0 : p) * bstride + vofs;
#pragma unroll
      for (int dg = 0; dg < NDG; ++dg) {
        if constexpr (F8) vd[c2][dg] = *(const VReg *)(vp + 16 * VROW * dg);
        else vd[c2][dg] = load_stream(vp + 16 * VROW * dg);
      }
    }
  };

  auto blk = [&](int idv, int t) {
    const int p = __builtin_amdgcn_readlane(idv, 16 * t);
    return p < a.num_blocks ? p : -1;            // ids outside the pool: never dereferenced
  };


  // One item: keys [kv_begin, kv_last) of its rows.  pre: its first step's
  // K/V are already in kr / vr, from the block ids b0 .. b3 (next: idv_next).
  // fetch_next (PREFETCH): once this item's Q loads are issued, the next
  // item's first step is read into kr2 / vr2 from the ids next_idv, so that
  // those loads queue behind the Q rows rather than ahead of them.
  auto run = [&](const DecodeItem item, const bool pre, int b0, int b1, int b2, int b3, int idv_next,
                 const bool fetch_next, const int next_idv) {
    const int token = uniform(item.token), req = uniform(item.req);
    const int kv_begin = uniform(item.kv_begin), kv_end = uniform(item.kv_end);
    const int part = uniform(item.part);
    const int aux = uniform(item.wpos);
    const int kind = uniform((int)item.kind);
    const int ntok = kind == 0 ? 1 : uniform((int)item.ntok);
    const int stride = uniform(item.stride);
    const int wpos = kind == 0 ? aux : -1;
    const bool wnew = wpos >= 0 && a.knew != nullptr;
    const int kv_last = wnew ? kv_end - 1 : kv_end;   // end of the keys read from the pool
    const int32_t *__restrict__ btrow = kind == 2 ? a.prefix_bt : a.block_table + (int64_t)req * a.bt_stride;
    // ---- columns: lane column 16 hf + r of half hf is (row ct, head ch) ----
    const bool rows_causal = kind == 1 && a.causal != 0;
    int ct[NH], ch[NH], clim[NH];
    bool cval[NH];
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
      const int n = 16 * hf + r;
      const int t = n / g;
      cval[hf] = t < ntok;
      ct[hf] = cval[hf] ? t : 0;
      ch[hf] = cval[hf] ? n - t * g : 0;
      // key limit of the column's row (exclusive)
      clim[hf] = rows_causal ? aux - (ntok - 1 - ct[hf]) : kv_last;
    }
    // keys from which some column can be cut off (the masked steps start there)
    const int cut = rows_causal ? min(kv_last, aux - (ntok - 1)) : kv_last;
    // flat row (q / output row) of each half's column
    int crow[NH];
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) crow[hf] = kind == 2 ? a.row_token[token + ct[hf]] : token + ct[hf];
    // ---- block ids: lane group j reads block j of a step ----
    // (the read itself is unconditional, at an index clamped to the row's last
    // block, so that no branch sits between the step's loads)
    const int last_bi = kv_last > 0 ? (kv_last - 1) >> 4 : 0;
    auto ids_of = [&](int itx) {
      const int bi = (itx >> 4) + j;
      const int id = btrow[bi < last_bi ? bi : last_bi];
      return bi <= last_bi ? id : -1;
    };
    // ---- the first step's K/V: read before the Q operands and the new key's
    // work below, so that their latency overlaps (the first step never reads
    // the new key's slot).  A kind-1 piece that stores its rows' K/V reads
    // after the stores. ----
    auto issue_first = [&]() {
      const int idv = ids_of(kv_begin);
      b0 = blk(idv, 0), b1 = blk(idv, 1), b2 = blk(idv, 2), b3 = blk(idv, 3);
      idv_next = ids_of(kv_begin + kKeysPerIter);
      issue_k(kr, b0, b1, b2, b3);
      asm volatile("" ::: "memory");              // K before V, as in the loop
      issue_v(vr, b0, b1, b2, b3);
      asm volatile("" ::: "memory");
    };
    const bool rows_first = kind == 1 && a.knew != nullptr && kv_end == aux;
    if (!pre && !rows_first && kv_begin < kv_last) issue_first();

    // ---- Q^T operand of each half: column r = (row ct, head ch) (zero when invalid) ----
    // (invalid columns are cleared with a mask, not a branch: a branch around
    // a loaded register makes the compiler wait for each load in turn)
    bf16x8_t qop[NH][NS];
    uint4 qv[NH][NS];
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
      const uint16_t *qrow =
          (const uint16_t *)a.q + ((int64_t)crow[hf] * a.num_q_heads + qh0 + ch[hf]) * D;
#pragma unroll
      for (int c = 0; c < NS; ++c) qv[hf][c] = *(const uint4 *)(qrow + qdim(c));
    }
    if constexpr (PREFETCH) {
      if (fetch_next) {
        asm volatile("" ::: "memory");          // after the Q loads
        pb0 = blk(next_idv, 0), pb1 = blk(next_idv, 1), pb2 = blk(next_idv, 2), pb3 = blk(next_idv, 3);
        issue_k(kr2, pb0, pb1, pb2, pb3);
        asm volatile("" ::: "memory");
        issue_v(vr2, pb0, pb1, pb2, pb3);
        asm volatile("" ::: "memory");
      }
    }
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
      const uint32_t qm = cval[hf] ? ~0u : 0u;
#pragma unroll
      for (int c = 0; c < NS; ++c)
        qop[hf][c] = as_bf16x8(make_uint4(qv[hf][c].x & qm, qv[hf][c].y & qm, qv[hf][c].z & qm, qv[hf][c].w & qm));
    }

    // ---- the new key's inputs (kind 0) ----
    uint4 kin[NS];
    uint2 vin[NDG];
    int wblk_v = -1;                               // (made uniform after the key loop)
    if (wnew) {
      const int64_t th = (int64_t)token * a.num_kv_heads + kvh;
      const uint16_t *krow = (const uint16_t *)a.knew + th * D;
      const uint16_t *vrow = (const uint16_t *)a.vnew + th * D;
#pragma unroll
      for (int c = 0; c < NS; ++c) kin[c] = *(const uint4 *)(krow + qdim(c));
#pragma unroll
      for (int dg = 0; dg < NDG; ++dg) vin[dg] = *(const uint2 *)(vrow + dg * 16 + 4 * j);
      wblk_v = btrow[wpos / kBlock];
    }

    float m_run[NH], l_run[NH];                    // per half, column r; l_run: this lane's keys only
    f32x4_t o[NH][NDG];
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
      m_run[hf] = -INFINITY;
      l_run[hf] = 0.0f;
#pragma unroll
      for (int dg = 0; dg < NDG; ++dg) o[hf][dg] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }

    // ---- the new key (kind 0, half 0): one online-softmax update with the
    // value the pool will hold, then its rows go into the pool.  With the
    // state still empty (m = -inf, l = 0, o = 0) the update is exactly the
    // first step (m = s, l = 1, o = v).  Where the registers allow it
    // (LATE_KEY), it runs after the key loop (the online softmax does not
    // depend on the order), which keeps the wait for its inputs and its
    // encoding off the path to the first K/V. ----
    auto new_key = [&]() {
    const int wblk = wnew ? uniform(wblk_v) : -1;
    if (wnew && kvh == 0 && lane == 0 && a.slots_out)
      a.slots_out[token] = (int64_t)wblk * kBlock + wpos % kBlock;
    if (wnew && wblk >= 0 && wblk < a.num_blocks) {
      uint32_t kb[NS][8], vb[NDG][4];
      if constexpr (F8) {
        // The 16 lanes of a lane group hold the same D / 4 input elements of
        // K and of V; each encodes D / 64 of them, and the codes go round
        // through LDS (the encoder's division and rounding would otherwise
        // run 16 times over).
        constexpr int EPL = D / 64;              // elements per lane
        __shared__ __attribute__((aligned(16))) uint8_t codes[2][4][D / 4];   // [K, V][lane group][element]
#pragma unroll
        for (int u = 0; u < EPL; ++u) {
          const int x = r * EPL + u;             // K element x: dims qdim(x / 8) + x % 8; V element x: 16 (x / 4) + 4 j + x % 4
          // (the element is picked with masks, not an index into kin / vin,
          // which the compiler would turn into a private-memory array)
          uint32_t kw = 0, vw = 0;
#pragma unroll
          for (int c = 0; c < NS; ++c) {
            const uint32_t w[4] = {kin[c].x, kin[c].y, kin[c].z, kin[c].w};
#pragma unroll
            for (int h = 0; h < 4; ++h)
              kw |= w[h] & (0u - (uint32_t)(c == (x >> 3) && h == ((x & 7) >> 1)));
          }
          const uint32_t hi_half = 0u - (uint32_t)((x >> 1) & 1);   // .y when set, else .x
#pragma unroll
          for (int dg = 0; dg < NDG; ++dg)
            vw |= ((vin[dg].x & ~hi_half) | (vin[dg].y & hi_half)) & (0u - (uint32_t)(dg == (x >> 2)));
          codes[0][j][x] = (uint8_t)pool_bits<KV_BF16, KV>((kw >> (16 * (x & 1))) & 0xffffu, a.enc_k_scale);
          codes[1][j][x] = (uint8_t)pool_bits<KV_BF16, KV>((vw >> (16 * (x & 1))) & 0xffffu, a.enc_v_scale);
        }
        // one wave per workgroup: its LDS writes are done once lgkmcnt is 0
        // (no barrier, which would also wait for the first K/V in flight)
        static_assert(kDecodeWaves == 1, "the codes' exchange is within one wave");
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        uint32_t kw[D / 16], vw[D / 16];
#pragma unroll
        for (int i = 0; i < D / 16; ++i) {
          kw[i] = ((const uint32_t *)codes[0][j])[i];
          vw[i] = ((const uint32_t *)codes[1][j])[i];
        }
#pragma unroll
        for (int c = 0; c < NS; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) kb[c][e] = (kw[(8 * c + e) >> 2] >> (8 * (e & 3))) & 0xffu;
#pragma unroll
        for (int dg = 0; dg < NDG; ++dg)
#pragma unroll
          for (int i = 0; i < 4; ++i) vb[dg][i] = (vw[(4 * dg + i) >> 2] >> (8 * i)) & 0xffu;
      } else {
#pragma unroll
        for (int c = 0; c < NS; ++c) {
          const uint32_t w[4] = {kin[c].x, kin[c].y, kin[c].z, kin[c].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) kb[c][e] = pool_bits<KV_BF16, KV>((w[e >> 1] >> (16 * (e & 1))) & 0xffffu, a.enc_k_scale);
        }
#pragma unroll
        for (int dg = 0; dg < NDG; ++dg) {
          const uint32_t w[2] = {vin[dg].x, vin[dg].y};
#pragma unroll
          for (int i = 0; i < 4; ++i)
            vb[dg][i] = pool_bits<KV_BF16, KV>((w[i >> 1] >> (16 * (i & 1))) & 0xffffu, a.enc_v_scale);
        }
      }
      float sp = 0.0f;
#pragma unroll
      for (int c = 0; c < NS; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) sp = fmaf((float)qop[0][c][e], pool_value<KV>(kb[c][e]), sp);
      sp = sum_x32(sum_x16(sp));
      const float s_new = sp * a.scale_log2;
      const float mn = fmaxf(m_run[0], s_new);
      const float alpha = __builtin_amdgcn_exp2f(m_run[0] - mn);   // 0 when the loop saw no key
      const float p_new = __builtin_amdgcn_exp2f(s_new - mn);
      l_run[0] = l_run[0] * alpha + (j == 0 ? p_new : 0.0f);
      m_run[0] = mn;
#pragma unroll
      for (int dg = 0; dg < NDG; ++dg)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[0][dg][i] = fmaf(p_new, pool_value<KV>(vb[dg][i]), o[0][dg][i] * alpha);
      // K element d of slot off sits at (d / E) * 256 + off * 16 + (d % E) * PB
      // of the tile; V element d at (d * 16 + off) * PB
      const int off = wpos % kBlock;
      char *kt = (char *)a.k_store + ((int64_t)wblk * a.num_kv_heads + kvh) * TILE;
      char *vt = (char *)a.v_store + ((int64_t)wblk * a.num_kv_heads + kvh) * TILE;
#pragma unroll
      for (int c = 0; c < NS; ++c) {
        if (r == c) {
          const int d0 = qdim(c);
          char *kd = kt + (d0 / E) * (kBlock * 16) + off * 16 + (d0 % E) * PB;
          if constexpr (F8) {
            uint2 w;
            w.x = kb[c][0] | kb[c][1] << 8 | kb[c][2] << 16 | kb[c][3] << 24;
            w.y = kb[c][4] | kb[c][5] << 8 | kb[c][6] << 16 | kb[c][7] << 24;
            *(uint2 *)kd = w;
          } else {
            uint4 w;
            w.x = kb[c][0] | kb[c][1] << 16;
            w.y = kb[c][2] | kb[c][3] << 16;
            w.z = kb[c][4] | kb[c][5] << 16;
            w.w = kb[c][6] | kb[c][7] << 16;
            *(uint4 *)kd = w;
          }
        }
      }
#pragma unroll
      for (int dg = 0; dg < NDG; ++dg) {
        if (r == dg) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            char *vd = vt + ((dg * 16 + 4 * j + i) * kBlock + off) * PB;
            if constexpr (F8) *(uint8_t *)vd = (uint8_t)vb[dg][i];
            else *(uint16_t *)vd = (uint16_t)vb[dg][i];
          }
        }
      }
    }
    };
    if constexpr (!LATE_KEY) new_key();

    // ---- kind 1, attention with the KV update: the piece holding the rows'
    // own keys (positions aux - ntok .. aux - 1; the plan puts all of them in
    // the last piece, which ends at aux) stores the rows' K/V into the pool
    // first, and its key loop then reads them like any other key.  No other
    // wave reads those slots in this launch.
    if (rows_first) {
      constexpr int NCH = D / E;                 // 16-byte pool chunks per row
      for (int w = lane; w < ntok * NCH; w += 64) {
        const int t = w / NCH, chn = w - t * NCH;
        const int pos = aux - ntok + t;
        const int wb = btrow[pos / kBlock];
        const int off = pos % kBlock;
        if (chn == 0 && kvh == 0 && a.slots_out) a.slots_out[token + t] = (int64_t)wb * kBlock + off;
        if (wb < 0 || wb >= a.num_blocks) continue;   // slot outside the pool: not written
        const int64_t th = (int64_t)(token + t) * a.num_kv_heads + kvh;
        const KvChunkIn<KV_BF16, KV> in =
            load_kv_chunk<KV_BF16, KV>((const char *)a.knew + th * D * 2, (const char *)a.vnew + th * D * 2, chn);
        store_kv_chunk<KV_BF16, KV, D>(in, a.k_store, a.v_store, ((int64_t)wb * a.num_kv_heads + kvh) * TILE, off, chn,
                                       a.enc_k_scale, a.enc_v_scale);
      }
      __builtin_amdgcn_s_waitcnt(0);             // every store of this wave has completed
      asm volatile("" ::: "memory");             // and no read below moves above them
    }

    // ---- the first step's K/V, when the rows' own keys came first ----
    if (!pre && rows_first && kv_begin < kv_last) issue_first();

    // ---- key loop ----
    for (int it = kv_begin; it < kv_last; it += kKeysPerIter) {
      const int idv_next2 = ids_of(it + 2 * kKeysPerIter);
      const bool slow = it + kKeysPerIter > cut || (b0 | b1 | b2 | b3) < 0;

      // S products (each K operand feeds every half)
      f32x4_t s[NH][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int hf = 0; hf < NH; ++hf) s[hf][u] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < NS; ++c) {
          bf16x8_t kop;
          if constexpr (F8) {
            const uint4 w = kr[u][c >> 1];
            kop = (c & 1) ? fp8x8_bf16(w.z, w.w) : fp8x8_bf16(w.x, w.y);
          } else {
            kop = as_bf16x8(kr[u][c]);
          }
#pragma unroll
          for (int hf = 0; hf < NH; ++hf)
            s[hf][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[hf][c], s[hf][u], 0, 0, 0);
        }
      }

      // the next step's K, into the registers just consumed (after the last
      // step too, where every id is -1 and block 0 is read: a valid address
      // already in the caches, and no branch between the loads)
      const int n0 = blk(idv_next, 0), n1 = blk(idv_next, 1), n2 = blk(idv_next, 2), n3 = blk(idv_next, 3);
      issue_k(kr, n0, n1, n2, n3);

      // valid keys of this lane: positions it + 32 c + 8 j + e, e < nv[c]
      // (and, per column, e < cl[hf][c]: the row's causal limit)
      int nv[2] = {8, 8};
      int cl[NH][2];
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) cl[hf][0] = cl[hf][1] = 8;
      if (slow) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const int p = c2 == 0 ? pick(vsel, b0, b1) : pick(vsel, b2, b3);
          const int lim = kv_last - (it + 32 * c2 + 8 * j);
          nv[c2] = p < 0 ? 0 : lim < 0 ? 0 : lim > 8 ? 8 : lim;
#pragma unroll
          for (int hf = 0; hf < NH; ++hf) cl[hf][c2] = clim[hf] - (it + 32 * c2 + 8 * j);
        }
      }

      // online softmax (log2 units), per half; S element i of product 2c + h is key 4h + i of chunk c.
      // P is rounded to bf16 for the PV product, and l sums those rounded
      // values (v_dot2 with (1, 1) per pair), so the output is normalised by
      // exactly the weights it is made of
      constexpr uint32_t kOnes = 0x3F803F80u;    // (1.0, 1.0) in bf16
      bf16x8_t pop[NH][2];
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) {
        float sc[4][4];
        float mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v = s[hf][u][i] * a.scale_log2;
            const int e = 4 * (u & 1) + i;
            if (slow && (e >= nv[u >> 1] || e >= cl[hf][u >> 1])) v = -INFINITY;
            sc[u][i] = v;
            mx = fmaxf(mx, v);
          }
        mx = max_x32(max_x16(mx));
        const float mn = fmaxf(m_run[hf], mx);
        const float mu = mn == -INFINITY ? 0.0f : mn;   // no key yet: every p and alpha is 0
        const float alpha = __builtin_amdgcn_exp2f(m_run[hf] - mu);
        float psum = 0.0f;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            const float p0 = __builtin_amdgcn_exp2f(sc[u][i] - mu);
            const float p1 = __builtin_amdgcn_exp2f(sc[u][i + 1] - mu);
            const uint32_t pw = pack_bf16x2(p0, p1);
            psum = dot2_bf16(pw, kOnes, psum);
            const bf16x2_t pb = __builtin_bit_cast(bf16x2_t, pw);
            pop[hf][u >> 1][4 * (u & 1) + i] = pb[0];
            pop[hf][u >> 1][4 * (u & 1) + i + 1] = pb[1];
          }
        l_run[hf] = l_run[hf] * alpha + psum;
        m_run[hf] = mn;
#pragma unroll
        for (int dg = 0; dg < NDG; ++dg) o[hf][dg] *= alpha;
      }

      // PV products (keys past the end or in invalid blocks: V zeroed, since
      // unwritten slots may hold anything; keys cut by a row's causal limit
      // are valid rows with p = 0)
      if (slow) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          if constexpr (F8) {
            const uint64_t m8 = nv[c2] >= 8 ? ~0ull : ((1ull << (8 * nv[c2])) - 1);
#pragma unroll
            for (int dg = 0; dg < NDG; ++dg) {
              vr[c2][dg].x &= (uint32_t)m8;
              vr[c2][dg].y &= (uint32_t)(m8 >> 32);
            }
          } else {
            uint32_t mw[4];
#pragma unroll
            for (int w = 0; w < 4; ++w)
              mw[w] = (2 * w < nv[c2] ? 0xffffu : 0u) | (2 * w + 1 < nv[c2] ? 0xffff0000u : 0u);
#pragma unroll
            for (int dg = 0; dg < NDG; ++dg) {
              vr[c2][dg].x &= mw[0];
              vr[c2][dg].y &= mw[1];
              vr[c2][dg].z &= mw[2];
              vr[c2][dg].w &= mw[3];
            }
          }
        }
      }
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int dg = 0; dg < NDG; ++dg) {
          bf16x8_t vop;
          if constexpr (F8) vop = fp8x8_bf16(vr[c2][dg].x, vr[c2][dg].y);
          else vop = as_bf16x8(vr[c2][dg]);
#pragma unroll
          for (int hf = 0; hf < NH; ++hf)
            o[hf][dg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[hf][c2], o[hf][dg], 0, 0, 0);
        }

      // the next step's V.  (The empty asm with a memory clobber keeps the
      // compiler from merging these reads with the first step's into one read
      // at the top of the loop, which would issue V only when it is needed.)
      issue_v(vr, n0, n1, n2, n3);
      asm volatile("" ::: "memory");
      b0 = n0, b1 = n1, b2 = n2, b3 = n3;
      idv_next = idv_next2;
    }

    if constexpr (LATE_KEY) new_key();

    // ---- totals and output: lane (r, j) holds dims 16 dg + 4 j + i of its column ----
    float l_tot[NH];
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) l_tot[hf] = sum_x32(sum_x16(l_run[hf]));   // every lane takes part
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
      if (!cval[hf]) continue;
      const int row = crow[hf];
      const int qh = qh0 + ch[hf];
      if (part < 0) {
        const float f = a.v_scale / l_tot[hf];
        uint16_t *orow = (uint16_t *)a.out + ((int64_t)row * a.num_q_heads + qh) * D + 4 * j;
#pragma unroll
        for (int dg = 0; dg < NDG; ++dg) {
          uint2 w;
          w.x = pack_bf16x2(o[hf][dg][0] * f, o[hf][dg][1] * f);
          w.y = pack_bf16x2(o[hf][dg][2] * f, o[hf][dg][3] * f);
          *(uint2 *)(orow + 16 * dg) = w;
        }
      } else {
        const int slot = kind == 2 ? a.row_slot0[token + ct[hf]] + part : part + ct[hf] * stride;
        float *po = a.part_o + ((int64_t)slot * a.num_q_heads + qh) * D + 4 * j;
#pragma unroll
        for (int dg = 0; dg < NDG; ++dg) {
          const f32x4_t v = o[hf][dg] * a.v_scale;
          *(float4 *)(po + 16 * dg) = make_float4(v[0], v[1], v[2], v[3]);
        }
        if (j == 0) {
          float *pml = a.part_ml + ((int64_t)slot * a.num_q_heads + qh) * 2;
          pml[0] = m_run[hf];
          pml[1] = l_tot[hf];
        }
      }
    }
  };

  // The start of a wave: its items, then their first steps' block ids (each
  // round issued for both items before waiting), then the first item's first
  // K/V into kr / vr.  The second item's first K/V (PREFETCH) follow the
  // first item's Q loads, inside its body.  So the first item's loads start
  // after one read of host memory and one of HBM, and its Q rows do not wait
  // behind the second item's K/V.
  const int item_b = PAIR && a.pair_stride + bin < a.n_items ? a.pair_stride + bin : -1;
  const DecodeItem ia = a.items[bin];
  DecodeItem ib{};
  if (PAIR && item_b >= 0) ib = a.items[item_b];
  // whether an item's first step can be read now (a kind-1 piece that stores
  // its rows' K/V first reads after the stores), and its block ids: lane
  // group j reads block j of the step, at an index clamped to the row's last
  // block (always in the row)
  struct First {
    bool ok;
    int idv, idv_next;
  };
  auto first_of = [&](const DecodeItem &it) -> First {
    const int req = uniform(it.req), kv_begin = uniform(it.kv_begin), kv_end = uniform(it.kv_end);
    const int ikind = uniform((int)it.kind), iaux = uniform(it.wpos);
    const bool own = ikind == 0 && iaux >= 0 && a.knew != nullptr;
    const int kv_last = own ? kv_end - 1 : kv_end;
    const bool stores_rows = ikind == 1 && a.knew != nullptr && kv_end == iaux;
    const int32_t *__restrict__ btrow = ikind == 2 ? a.prefix_bt : a.block_table + (int64_t)req * a.bt_stride;
    const int last_bi = kv_last > 0 ? (kv_last - 1) >> 4 : 0;
    auto ids_of = [&](int itx) {
      const int bi = (itx >> 4) + j;
      const int id = btrow[bi < last_bi ? bi : last_bi];
      return bi <= last_bi ? id : -1;
    };
    return First{kv_begin < kv_last && !stores_rows, ids_of(kv_begin), ids_of(kv_begin + kKeysPerIter)};
  };
  const First fa = first_of(ia);
  First fb{false, -1, -1};
  if (PREFETCH && item_b >= 0) fb = first_of(ib);
  int a0 = -1, a1 = -1, a2 = -1, a3 = -1;
  if (fa.ok) {
    a0 = blk(fa.idv, 0), a1 = blk(fa.idv, 1), a2 = blk(fa.idv, 2), a3 = blk(fa.idv, 3);
    issue_k(kr, a0, a1, a2, a3);
    asm volatile("" ::: "memory");              // K before V, as in the loop
    issue_v(vr, a0, a1, a2, a3);
    asm volatile("" ::: "memory");
  }
  run(ia, fa.ok, a0, a1, a2, a3, fa.idv_next, PREFETCH && fb.ok, fb.idv);
  if (PAIR && item_b >= 0) {
    if constexpr (PREFETCH) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int x = 0; x < NKX; ++x) kr[u][x] = kr2[u][x];
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int dg = 0; dg < NDG; ++dg) vr[c2][dg] = vr2[c2][dg];
      run(ib, fb.ok, pb0, pb1, pb2, pb3, fb.idv_next, false, -1);
    } else {
      run(ib, false, -1, -1, -1, -1, -1, false, -1);
    }
  }
}

template <int KV, int D, bool PAIR>
static void launch_nh(const DecodeArgs &a, int nh, dim3 grid, dim3 block, hipStream_t s) {
  if (nh == 2) hipLaunchKernelGGL((k_decode_mfma<KV, D, PAIR, 2>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((k_decode_mfma<KV, D, PAIR, 1>), grid, block, 0, s, a);
}

template <int KV, int D>
static void launch_pair(const DecodeArgs &a, bool pair, int nh, dim3 grid, dim3 block, hipStream_t s) {
  if (pair) launch_nh<KV, D, true>(a, nh, grid, block, s);
  else launch_nh<KV, D, false>(a, nh, grid, block, s);
}

hipError_t launch_decode_mfma(const pa_kv_pool &p, const DecodeArgs &a, hipStream_t s) {
  const bool pair = a.pair_stride > 0;
  static_assert(kDecodeWaves == 1, "scatter workgroups follow the decode units one to one");
  const int units = (pair ? a.pair_stride : a.n_items) * a.num_kv_heads + a.n_wseg_units + a.n_copy_units;
  const dim3 grid((units + kDecodeWaves - 1) / kDecodeWaves), block(64 * kDecodeWaves);
  const int nh = a.max_cols > 16 ? 2 : 1;
  if (p.kv_dtype == PA_BF16 && p.head_dim == 128) launch_pair<KV_BF16, 128>(a, pair, nh, grid, block, s);
  else if (p.kv_dtype == PA_BF16) launch_pair<KV_BF16, 64>(a, pair, nh, grid, block, s);
  else if (p.head_dim == 128) launch_pair<KV_FP8, 128>(a, pair, nh, grid, block, s);
  else launch_pair<KV_FP8, 64>(a, pair, nh, grid, block, s);
  return hipGetLastError();
}

}  // namespace pa
