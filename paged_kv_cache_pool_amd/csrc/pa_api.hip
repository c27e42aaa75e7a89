// C ABI of libpa.so: argument checks, the host-side plan of a step, the
// workspace layout, a pinned staging ring for the plan's upload, and the
// kernel-timing hooks.  Every step of the computation itself runs in the HIP
// kernels of k_write.hip, k_decode.hip and k_extend.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <set>
#include <string>
#include <vector>

#include "pa_internal.h"

namespace pa {

// ------------------------------------------------------------------ errors --

static thread_local std::string g_last_error;

static pa_status fail(pa_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pa_status pa_set_error(pa_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

static pa_status hip_fail(hipError_t e, const char *what) {
  return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// --------------------------------------------------------------- profiling --

struct ProfRec {
  const char *name;
  hipEvent_t start, stop;
};

static std::mutex g_prof_mu;
static bool g_prof_on = false;
static std::vector<ProfRec> g_prof;
static std::vector<hipEvent_t> g_prof_free;
static thread_local int g_prof_open = -1;

static hipEvent_t prof_event() {
  if (!g_prof_free.empty()) {
    hipEvent_t e = g_prof_free.back();
    g_prof_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

static bool capturing(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(s, &st) == hipSuccess && st != hipStreamCaptureStatusNone;
}

// Launches captured into a graph are not timed (their events would become
// graph nodes).
void prof_begin(const char *name, hipStream_t s) {
  if (!g_prof_on || capturing(s)) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  ProfRec r{name, prof_event(), prof_event()};
  if (!r.start || !r.stop) return;
  if (hipEventRecord(r.start, s) != hipSuccess) {   // not timed: the events go back
    g_prof_free.push_back(r.start);
    g_prof_free.push_back(r.stop);
    return;
  }
  g_prof.push_back(r);
  g_prof_open = (int)g_prof.size() - 1;
}

void prof_end(hipStream_t s) {
  if (!g_prof_on || g_prof_open < 0) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (hipEventRecord(g_prof[g_prof_open].stop, s) != hipSuccess) {   // the launch is not timed
    const ProfRec r = g_prof.back();           // (the open record is the last one)
    g_prof.pop_back();
    g_prof_free.push_back(r.start);
    g_prof_free.push_back(r.stop);
  }
  g_prof_open = -1;
}

static void prof_reset_locked() {
  for (auto &r : g_prof) {
    (void)hipEventSynchronize(r.stop);         // an error here only loses a timing record
    g_prof_free.push_back(r.start);
    g_prof_free.push_back(r.stop);
  }
  g_prof.clear();
}

// ------------------------------------------------------ pinned staging ring --
// The plan of a step (work lists) is built on the host.  It is written into
// a pinned, device-mapped host buffer that the kernels read directly (one
// small read per wave or workgroup), so no copy is queued between the
// caller's previous kernel and ours.  A buffer is reused only after every
// kernel that reads it has completed.  No event is recorded per call (an
// event between steps measured 3-5 us per step): the first kernel of the next
// call on the same stream stores a release flag for the previous call's
// buffer when it starts, and by then every earlier kernel of that stream has
// completed.  A buffer whose stream saw no later call before the buffer is
// needed again is waited for with a device synchronisation.  One ring of 16
// buffers per device.  With PA_PLAN_UPLOAD=1 the plan is instead copied into
// the caller's workspace.

constexpr int kDevMax = 64;
constexpr int kStageSlots = 16;

struct StageSlot {
  void *host = nullptr;
  void *dev = nullptr;                           // device address of `host`
  size_t cap = 0;
  hipStream_t stream = nullptr;                  // stream of the call that used it last
  bool pending = false;                          // that call's kernels may still read it
  bool superseded = false;                       // a later call on that stream has been issued
};

struct StageRing {
  StageSlot slot[kStageSlots];
  unsigned next = 0;
  volatile int32_t *flags = nullptr;             // pinned words, one per slot: 1 once released
  int32_t *flags_dev = nullptr;                  // their device addresses
  std::vector<std::pair<hipStream_t, int>> last; // stream -> the slot its last call used
};

static std::mutex g_stage_mu;
static StageRing g_stage[kDevMax];

// A free slot of at least `bytes` for a call on stream s.  *release: the
// device address of the release flag of the previous call's slot on s
// (null if there is none), which the call's first kernel must store 1 to.
static pa_status stage_acquire(size_t bytes, hipStream_t s, StageSlot **out, int32_t **release) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kDevMax) return fail(PA_ERR_UNSUPPORTED, "device %d beyond the %d the library supports", dev, kDevMax);
  std::lock_guard<std::mutex> lk(g_stage_mu);
  StageRing &R = g_stage[dev];
  if (!R.flags) {
    void *h = nullptr, *d = nullptr;
    if ((e = hipHostMalloc(&h, kStageSlots * sizeof(int32_t), hipHostMallocMapped | hipHostMallocCoherent)) != hipSuccess)
      return hip_fail(e, "staging flags");
    if ((e = hipHostGetDevicePointer(&d, h, 0)) != hipSuccess) return hip_fail(e, "staging flags map");
    memset(h, 0, kStageSlots * sizeof(int32_t));
    R.flags = (volatile int32_t *)h;
    R.flags_dev = (int32_t *)d;
  }
  const int k = (int)(R.next++ % kStageSlots);
  StageSlot &slot = R.slot[k];
  if (slot.pending) {
    bool released = R.flags[k] != 0;
    if (!released && slot.superseded) {
      // the next call on its stream has been issued: its first kernel sets
      // the flag when it starts (bounded wait; the device synchronisation
      // below covers a call whose launch failed)
      for (int spin = 0; spin < (1 << 22) && !released; ++spin) released = R.flags[k] != 0;
    }
    if (!released && (e = hipDeviceSynchronize()) != hipSuccess) return hip_fail(e, "staging wait");
    slot.pending = false;
  }
  if (slot.cap < bytes) {
    if (slot.host) (void)hipHostFree(slot.host);   // released above; nothing reads it
    slot.host = slot.dev = nullptr;
    slot.cap = 0;
    const size_t cap = std::max<size_t>(bytes, 64 << 10);
    if ((e = hipHostMalloc(&slot.host, cap, hipHostMallocMapped | hipHostMallocCoherent)) != hipSuccess) {
      slot.host = nullptr;
      return hip_fail(e, "staging buffer");
    }
    if ((e = hipHostGetDevicePointer(&slot.dev, slot.host, 0)) != hipSuccess) return hip_fail(e, "staging map");
    slot.cap = cap;
  }
  // the previous slot of this stream is released by this call's first kernel
  *release = nullptr;
  bool found = false;
  for (auto &entry : R.last) {
    if (entry.first != s) continue;
    StageSlot &prev = R.slot[entry.second];
    if (entry.second != k && prev.pending && !prev.superseded && prev.stream == s) {
      prev.superseded = true;
      *release = R.flags_dev + entry.second;
    }
    entry.second = k;
    found = true;
    break;
  }
  if (!found) {
    if (R.last.size() >= 64) R.last.erase(R.last.begin());
    R.last.push_back({s, k});
  }
  R.flags[k] = 0;
  slot.stream = s;
  slot.pending = true;
  slot.superseded = false;
  *out = &slot;
  return PA_OK;
}

// -------------------------------------------------------- captured plans --
// Work lists of calls captured into a HIP graph: written once, at capture,
// into a pinned, device-mapped host arena that is never reused, so the
// graph's kernels read them at every replay exactly as eager launches read
// the staging ring (no copy nodes in the graph).  One arena per device,
// created by the first call on that device made outside capture (allocation
// is avoided while capturing), kept until the process ends; captured calls
// take space from it until it is full, then fall back to copy kernels that
// carry the lists as arguments into the workspace.

constexpr size_t kArenaBytes = (size_t)8 << 20;

struct PlanArena {
  char *host = nullptr;
  char *dev = nullptr;
  size_t used = 0;
  bool failed = false;                           // allocation failed once: do not retry
};

static std::mutex g_arena_mu;
static PlanArena g_arena[kDevMax];

// Outside capture: create this device's arena if it does not exist yet.
static void arena_ensure() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevMax) return;
  std::lock_guard<std::mutex> lk(g_arena_mu);
  PlanArena &a = g_arena[dev];
  if (a.host || a.failed) return;
  void *h = nullptr, *d = nullptr;
  if (hipHostMalloc(&h, kArenaBytes, hipHostMallocMapped | hipHostMallocCoherent) != hipSuccess) {
    a.failed = true;
    return;
  }
  if (hipHostGetDevicePointer(&d, h, 0) != hipSuccess) {
    (void)hipHostFree(h);
    a.failed = true;
    return;
  }
  a.host = (char *)h;
  a.dev = (char *)d;
}

// Under capture: bytes of the arena for one call's lists (host and device
// addresses), or false when there is no arena or no room.
static bool arena_take(size_t bytes, char **host, const char **dev) {
  int d = 0;
  if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= kDevMax) return false;
  std::lock_guard<std::mutex> lk(g_arena_mu);
  PlanArena &a = g_arena[d];
  const size_t need = (bytes + 255) & ~(size_t)255;
  if (!a.host || a.used + need > kArenaBytes) return false;
  *host = a.host + a.used;
  *dev = a.dev + a.used;
  a.used += need;
  return true;
}

// ------------------------------------------------------------ static scratch --
// Scratch of pa_write_kv_attention_noalloc (for callers that cannot allocate):
// the call's work lists and split-K partials live in this array instead of a
// caller's workspace.  Each device holds its own copy from the time the
// library's code object is loaded on it until the process ends.  In host code
// `scratch` names a host-side stand-in, never the device array: its device
// address is looked up once per device (hipGetSymbolAddress, with that device
// current) and only that address is handed to kernels.

constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
constexpr int kMaxDevices = kDevMax;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

static std::mutex g_scratch_mu;
static void *g_scratch_dev[kMaxDevices];           // device address of `scratch`, per device

static pa_status static_scratch(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(PA_ERR_UNSUPPORTED, "device %d beyond the %d the library supports", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void *ptr = nullptr;
    if ((e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) != hipSuccess) return hip_fail(e, "scratch address");
    if (!ptr) return fail(PA_ERR_HIP, "scratch address is NULL");
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return PA_OK;
}

// ------------------------------------------------------------- side stream --
// Prefill rows (MFMA) and decode rows (HBM-bound) of one step are
// independent; with PA_OVERLAP=1 the extend kernel runs on a second stream,
// forked from and joined back to the caller's stream with events, so the two
// kernels overlap on the GPU while the caller still sees one ordered stream.
// Off by default: measured on the mixed 2048-token step it is slower than
// running the two kernels one after the other (each slows the other more than
// the overlap gains).  One side stream and event pair per device, created on
// first use, default priority.

struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};

static std::mutex g_side_mu;
static std::vector<SideStream> g_side;

static pa_status side_stream(SideStream **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_side_mu);
  if ((int)g_side.size() <= dev) g_side.resize(dev + 1);
  SideStream &ss = g_side[dev];
  if (!ss.stream) {
    if ((e = hipStreamCreateWithFlags(&ss.stream, hipStreamNonBlocking)) != hipSuccess)
      return hip_fail(e, "side stream");
    if ((e = hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&ss.join, hipEventDisableTiming)) != hipSuccess)
      return hip_fail(e, "side stream events");
  }
  *out = &ss;
  return PA_OK;
}

// ---------------------------------------------------------------- checks ---

static int elem_bytes(pa_dtype d) { return d == PA_F32 ? 4 : d == PA_BF16 ? 2 : 1; }

static bool env_flag(const char *name) {
  const char *v = getenv(name);
  return v && *v && strcmp(v, "0") != 0;
}

static pa_status check_pool(const pa_kv_pool *p, bool need_ptrs) {
  if (!p) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
  if (need_ptrs && (!p->k_cache || !p->v_cache)) return fail(PA_ERR_INVALID_ARG, "pool cache pointer is NULL");
  if (p->num_blocks <= 0 || p->num_kv_heads <= 0 || p->block_size <= 0 || p->head_dim <= 0)
    return fail(PA_ERR_INVALID_ARG, "pool sizes must be positive");
  if (p->kv_dtype != PA_F32 && p->kv_dtype != PA_BF16 && p->kv_dtype != PA_FP8_E4M3)
    return fail(PA_ERR_INVALID_ARG, "unknown kv_dtype %d", (int)p->kv_dtype);
  if (p->block_size != kBlock) return fail(PA_ERR_UNSUPPORTED, "block_size %d (only 16)", p->block_size);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d (only 64, 128)", p->head_dim);
  if (p->kv_dtype == PA_FP8_E4M3) {
    if (!(std::isfinite(p->k_scale) && p->k_scale > 0 && std::isfinite(p->v_scale) && p->v_scale > 0))
      return fail(PA_ERR_INVALID_ARG, "fp8 pool needs finite positive k_scale and v_scale");
  }
  return PA_OK;
}

static pa_status check_batch(const pa_batch *b, bool need_dev) {
  if (!b) return fail(PA_ERR_INVALID_ARG, "batch is NULL");
  if (b->num_seqs < 0 || b->num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "negative batch size");
  if (!b->query_start_loc_host || !b->seq_lens_host)
    return fail(PA_ERR_INVALID_ARG, "batch host mirrors are NULL");
  if (need_dev && b->num_seqs > 0 &&
      (!b->query_start_loc || !b->seq_lens || !b->block_table))
    return fail(PA_ERR_INVALID_ARG, "batch device arrays are NULL");
  if (b->bt_stride < 0) return fail(PA_ERR_INVALID_ARG, "negative bt_stride");
  if (b->num_common_prefix_blocks < 0) return fail(PA_ERR_INVALID_ARG, "negative num_common_prefix_blocks");
  const int32_t *q = b->query_start_loc_host, *L = b->seq_lens_host;
  if (q[0] != 0) return fail(PA_ERR_INVALID_ARG, "query_start_loc[0] = %d, expected 0", q[0]);
  for (int32_t i = 0; i < b->num_seqs; ++i) {
    const int32_t c = q[i + 1] - q[i];
    if (c < 0) return fail(PA_ERR_INVALID_ARG, "query_start_loc decreases at request %d", i);
    if (L[i] < c) return fail(PA_ERR_INVALID_ARG, "seq_lens[%d] = %d < %d new tokens", i, L[i], c);
    const int64_t nb = ((int64_t)L[i] + kBlock - 1) / kBlock;
    if (nb > b->bt_stride) return fail(PA_ERR_INVALID_ARG, "request %d needs %lld blocks > bt_stride %d", i, (long long)nb, b->bt_stride);
  }
  if (q[b->num_seqs] != b->num_tokens)
    return fail(PA_ERR_INVALID_ARG, "query_start_loc[N] = %d != num_tokens %d", q[b->num_seqs], b->num_tokens);
  return PA_OK;
}

// Deep checks of device-side metadata (PA_VALIDATE=1): the block table's
// needed entries are valid block ids.  Synchronous (device-to-host copy).
static pa_status validate_block_table(const pa_batch *b, int32_t num_blocks, hipStream_t s) {
  if (b->num_seqs == 0) return PA_OK;
  std::vector<int32_t> bt((size_t)b->num_seqs * b->bt_stride);
  hipError_t e = hipMemcpyAsync(bt.data(), b->block_table, bt.size() * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "validate: block table read");
  for (int32_t i = 0; i < b->num_seqs; ++i) {
    const int64_t nb = ((int64_t)b->seq_lens_host[i] + kBlock - 1) / kBlock;
    for (int64_t j = 0; j < nb; ++j) {
      const int32_t blk = bt[(size_t)i * b->bt_stride + j];
      if (blk < 0 || blk >= num_blocks)
        return fail(PA_ERR_VALIDATION, "block_table[%d][%lld] = %d outside [0, %d)", i, (long long)j, blk, num_blocks);
    }
  }
  // the shared-prefix hint: the same leading blocks in every row with new tokens
  const int32_t np = b->num_common_prefix_blocks;
  int32_t first = -1;
  for (int32_t i = 0; i < b->num_seqs && np > 0; ++i) {
    if (b->query_start_loc_host[i + 1] == b->query_start_loc_host[i]) continue;
    if (np > b->bt_stride) return fail(PA_ERR_VALIDATION, "num_common_prefix_blocks %d > bt_stride", np);
    if (first < 0) {
      first = i;
      continue;
    }
    for (int32_t j = 0; j < np; ++j)
      if (bt[(size_t)i * b->bt_stride + j] != bt[(size_t)first * b->bt_stride + j])
        return fail(PA_ERR_VALIDATION, "block_table[%d][%d] differs from request %d inside the common prefix", i, j, first);
  }
  return PA_OK;
}

// ------------------------------------------------------------------ plan ---
// a3: classify each request's rows (MFMA extend for prefill chunks, split-K
// token-parallel otherwise), pick the partition length, and lay out the
// workspace.  Deterministic in the host mirrors, so the workspace query and
// the call agree.

struct Plan {
  std::vector<DecodeItem> dec;
  std::vector<MergeItem> merge;
  std::vector<ExtendItem> extw;                  // extend items (wide and key-split), one launch
  // shared-prefix (cascade) pass
  std::vector<PrefixItem> pre;
  std::vector<int32_t> row_token, row_slot0;
  int32_t prefix_req = -1;                       // request whose block-table row supplies the prefix
  // attention that includes the KV update: block segments of the tokens the
  // plan-driven scatter writes before the attention kernels (the others are
  // written by their decode unit, DecodeItem::wpos)
  std::vector<WriteSeg> wseg;
  bool wseg_read_by_dec = false;                 // some split-K rows read keys the scatter writes
  bool ext_merge = false;                        // some merge items combine extend key pieces
  int32_t n_slots = 0;
  int32_t part_len = 0;
  int32_t kstart = 0;                            // first key of the split-K items (the cascade's prefix end)
  int32_t pair_stride = 0;                       // paired layout: items b and pair_stride + b share a wave
  int32_t max_cols = 0;                          // largest (row, head) column count of a decode item
  bool pre_dec = false;                          // the prefix rows' prefix attention as kind-2 decode items
  size_t off_dec = 0, off_merge = 0, off_extw = 0, off_pre = 0, off_rtok = 0, off_rslot = 0, off_wseg = 0;
  size_t off_ml = 0, off_o = 0, bytes = 0;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Smallest number of new rows for which a request goes to the MFMA extend
// kernel (bf16 or fp8 pools with bf16 q, head_dim 128); one-row requests use
// the split-K kernel.  Two rows already favour the extend kernel: it reads
// the request's K/V once for all its rows (per kv head), where the split-K
// kernel reads them once per row (the 2..8-row verify chunks of speculative
// decoding run 3x faster on it).
static int extend_min_rows() {
  const char *v = getenv("PA_EXTEND_MIN_ROWS");
  return v ? atoi(v) : 2;
}

static bool extend_supported(const pa_kv_pool &p, pa_dtype q_dtype) {
  return q_dtype == PA_BF16 && (p.kv_dtype == PA_BF16 || p.kv_dtype == PA_FP8_E4M3) && p.head_dim == 128;
}

// Compute units of the current device (256 on MI355X), cached per device;
// 256 when no device can be queried.
static int device_cu_count() {
  static std::mutex mu;
  static std::vector<int> cus;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  std::lock_guard<std::mutex> lk(mu);
  if ((int)cus.size() <= dev) cus.resize(dev + 1, 0);
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

static void build_plan(const pa_kv_pool &p, const pa_batch &b, int32_t Hq, pa_dtype q_dtype,
                       int causal, bool kv_update, Plan &plan) {
  const int32_t *q = b.query_start_loc_host, *L = b.seq_lens_host;
  const int Hkv = p.num_kv_heads, g = Hq / Hkv;
  const bool ext_ok = extend_supported(p, q_dtype) && env_flag("PA_DISABLE_EXTEND") == false;
  const int ext_min = extend_min_rows();
  // PA_MULTIROW=1: short chunks (2 .. 32 / g rows, such as the draft tokens
  // of a verify step) on the matrix-core split-K kernel: one kind-1 item
  // covers all the chunk's rows, each (row, q head) pair an MFMA column, so
  // the request's K/V are read once per kv head at decode bandwidth (the
  // extend kernel leaves most of its 128 columns empty).  Measured on the
  // verify workload (64 chunks of 2..8 rows, g = 4): the split-K kernel
  // takes 118 us against the extend kernel's 131, but its pieces' merge
  // (11 us) and the rows' write (9 us as a scatter launch, 8.5 us inside
  // the last piece) make the step slower (0.136-0.137 ms against 0.131), so
  // the extend kernel stays the default.
  const bool multi_ok = p.kv_dtype != PA_F32 && env_flag("PA_MULTIROW");
  auto multi = [&](int32_t c) { return multi_ok && c >= 2 && (int64_t)c * g <= 32; };
  auto on_ext = [&](int32_t c) { return ext_ok && c >= ext_min && !multi(c); };
  std::vector<int32_t> ext_reqs;                 // requests on the MFMA extend kernel, planned after the loop

  // Shared prefix (cascade): the split-K rows' first P keys are the same
  // blocks for every request; their attention over them is computed once per
  // kv head by the MFMA prefix pass and merged with the rest.  Used when
  // every split-K request holds the prefix wholly in its history.
  // (in int64: a hint of any int32 value is compared with the histories,
  // never wrapped; one longer than INT32_MAX keys or beyond bt_stride cannot
  // lie in any request's history, so it is ignored)
  const int64_t P64 = (int64_t)b.num_common_prefix_blocks * kBlock;
  bool cascade = P64 > 0 && P64 <= INT32_MAX && b.num_common_prefix_blocks <= b.bt_stride &&
                 extend_supported(p, q_dtype) &&
                 !env_flag("PA_DISABLE_CASCADE") &&
                 (int64_t)b.num_tokens * Hq * p.head_dim * 2 < ((int64_t)1 << 32);
  const int32_t P = cascade ? (int32_t)P64 : 0;
  int32_t prefix_rows = 0;
  for (int32_t i = 0; i < b.num_seqs && cascade; ++i) {
    const int32_t c = q[i + 1] - q[i];
    if (c == 0 || on_ext(c)) continue;
    if (L[i] - c < P) cascade = false;
    if (plan.prefix_req < 0) plan.prefix_req = i;
    prefix_rows += c;
  }
  if (prefix_rows == 0) cascade = false;
  if (!cascade) plan.prefix_req = -1;
  const int32_t kstart = cascade ? P : 0;        // first key of the split-K rows' own work
  plan.kstart = kstart;

  // The prefix rows' attention over the shared prefix: by the split-K kernel
  // as kind-2 items (units of 16 / g prefix rows, one MFMA column per (row,
  // q head), packed with the rows' own work into one launch) while the
  // prefix rows have at most kPrefixDecodeCols columns per kv head;
  // otherwise (or with PA_PREFIX_PASS=1) by the MFMA prefix pass.  On the
  // fp8 shared-prefix workload (128 rows, g = 4, a 2048-key prefix) the step
  // takes 0.050 ms against 0.058 with the prefix pass, whose launch, the
  // split-K launch and the merge ran one after the other.  A prefix item
  // reads each K/V byte for 16 columns where the prefix pass's tile feeds
  // 128, so many prefix rows go to the prefix pass.
  constexpr int64_t kPrefixDecodeCols = 1024;
  bool any_multi = false;
  for (int32_t i = 0; i < b.num_seqs && cascade; ++i) any_multi |= multi(q[i + 1] - q[i]);
  const bool pre_dec = cascade && (int64_t)prefix_rows * g <= kPrefixDecodeCols && !any_multi &&
                       !env_flag("PA_PREFIX_PASS");
  const int32_t pre_rows = std::max(1, 16 / g);  // prefix rows per kind-2 unit
  const int32_t n_pre_units = pre_dec ? (prefix_rows + pre_rows - 1) / pre_rows : 0;
  plan.pre_dec = pre_dec;

  // Partition length of the split-K rows (a unit = one token's keys in one
  // partition, for one kv head: one wave).
  //  * One launch round: all units resident at once, at most 8 per compute
  //    unit (two waves per SIMD), so that no compute unit starts a unit while
  //    others idle.  The shortest 64-key multiple whose unit count fits.
  //  * Units that would be longer than 2048 keys even then run at most 4 per
  //    compute unit: measured faster on the long-context decode (four waves
  //    keep a compute unit's memory pipeline full), and half the partials.
  //  * A batch with more rows than fit in one round: about 16 units per
  //    compute unit, handed out longest first.
  // (Measured on the decode workloads against a fixed 16 units per compute
  // unit: 5-11 % less kernel time.)
  std::vector<int32_t> tok_keys;
  int64_t key_work = 0;
  int32_t max_keys = 0;
  for (int32_t u = 0; u < n_pre_units; ++u) {   // kind-2 units first: keys [0, P)
    tok_keys.push_back(P);
    key_work += P;
    max_keys = std::max(max_keys, P);
  }
  for (int32_t i = 0; i < b.num_seqs; ++i) {
    const int32_t c = q[i + 1] - q[i];
    if (c == 0 || on_ext(c)) continue;
    // (a multi-row chunk is one unit over the keys of its last row)
    for (int32_t t = multi(c) ? c - 1 : 0; t < c; ++t) {
      const int32_t k = std::max(0, (causal ? (L[i] - c + t + 1) : L[i]) - kstart);
      tok_keys.push_back(k);
      key_work += k;
      max_keys = std::max(max_keys, k);
    }
  }
  auto round64 = [](int64_t x) { return std::max<int64_t>(64, (x + 63) / 64 * 64); };
  const int64_t cus = device_cu_count();
  int64_t part;
  {
    const int64_t per_cu = key_work * Hkv >= 8 * cus * 2048 ? 4 : 8;
    const int64_t cap = per_cu * cus;
    auto units_of = [&](int64_t pl) {
      int64_t u = 0;
      for (int32_t k : tok_keys) u += (k + pl - 1) / pl;
      return u * Hkv;
    };
    int64_t lo = round64((key_work * Hkv + cap - 1) / cap);
    const int64_t hi = std::max(lo, round64(max_keys));
    if ((int64_t)tok_keys.size() * Hkv <= cap && units_of(hi) <= cap) {
      for (int64_t h = hi; lo < h;) {            // smallest fitting length (the count falls as it grows)
        const int64_t mid = (lo + h) / 128 * 64;
        if (units_of(mid) <= cap) h = mid;
        else lo = mid + 64;
      }
      part = lo;
    } else {
      part = round64((key_work * Hkv + 16 * cus - 1) / (16 * cus));
    }
  }
  if (const char *v = getenv("PA_PARTITION_KEYS")) part = std::max(64, atoi(v) / 64 * 64);
  plan.part_len = (int32_t)part;

  // Paired layout (bf16 and fp8 pools: the matrix-core kernel).  Measured on
  // MI355X: with two waves per SIMD (8 one-wave workgroups per compute unit)
  // workgroups u and u + 4 * CUs share a SIMD, and the older wave takes
  // nearly all of the SIMD's memory issue until it ends, so the two run one
  // after the other and the SIMD ends at a time set by their sum.  So the
  // split-K tokens' 64-key steps, in token order, are packed into at most
  // n_bins = 4 * CUs / Hkv bins of at most T steps and at most two pieces (a
  // bin ends after its second piece), with the smallest T that fits, and one
  // wave per SIMD runs a bin's two pieces in turn (pair_stride: bin b's pieces
  // are items b and pair_stride + b; two-piece bins are numbered first, so
  // the items have no gaps).  The wave reads its second piece's first K/V at
  // the start, so the second piece starts without a wait.  Tokens of several
  // pieces get partials and a merge.  Used when T is at least 8 steps
  // (shorter units are bound by their start-up).  PA_DECODE_PAIRS=2: the same
  // bins as two waves of one SIMD (each piece its own wave; bins split until
  // there are n_bins); 0: the partition form above.
  int64_t n_bins = 0, pair_T = 0;
  std::vector<int32_t> tok_steps;
  // A bin's second piece costs its wave about `pen` steps beyond its keys
  // (the first piece's end, the second's rows and their Q): per-wave
  // timelines of the decode layer and the mixed step show two-piece bins
  // ending 6-10 us after single-piece bins of the same step count.  The
  // cost is charged only where the bins still fit at the step count T found
  // without it (a larger T would lengthen every single-piece bin), and not
  // when the bins' pieces run as waves of their own (below).
  const char *pair_env = getenv("PA_DECODE_PAIRS");
  const bool pair_waves = pair_env ? atoi(pair_env) == 2 : pre_dec;
  int64_t pen = 0;
  int64_t pen_want = 2;
  if (const char *v = getenv("PA_PAIR_PENALTY")) pen_want = std::max(0, atoi(v));
  if (pair_waves) pen_want = 0;
  auto bins_for = [&](int64_t T, std::vector<std::array<int32_t, 4>> *pieces) {
    // greedy packing; pieces: (bin, slot, first step, end step) in token order
    int64_t bins = 0, load = T, np = 2;
    for (size_t x = 0; x < tok_steps.size(); ++x)
      for (int64_t o = 0, st = tok_steps[x]; o < st;) {
        if (np == 1) load += pen;
        if (np == 2 || load >= T) {
          ++bins;
          load = 0;
          np = 0;
        }
        const int64_t take = std::min(st - o, T - load);
        if (pieces) pieces->push_back({(int32_t)(bins - 1), (int32_t)np, (int32_t)o, (int32_t)(o + take)});
        o += take;
        load += take;
        ++np;
      }
    return bins;
  };
  {
    // (not by default when prefix items share the launch: their units are
    // short and bound by their start, and the partition form spreads them
    // over more waves; measured on the fp8 shared-prefix workload: 0.0405
    // against 0.0413 ms per step)
    const char *penv = getenv("PA_DECODE_PAIRS");
    const bool want = p.kv_dtype != PA_F32 && !(penv && atoi(penv) <= 0) && (!pre_dec || (penv && atoi(penv) > 0));
    if (want && (4 * cus) % Hkv == 0 && !tok_keys.empty()) {
      int64_t S = 0, smax = 0;
      for (int32_t k : tok_keys) {
        const int64_t st = (k + kKeysPerIter - 1) / kKeysPerIter;
        tok_steps.push_back((int32_t)st);
        S += st;
        smax = std::max(smax, st);
      }
      n_bins = 4 * cus / Hkv;
      int64_t lo = std::max<int64_t>(1, (S + n_bins - 1) / n_bins), hi = std::max(lo, smax);
      if (S > 0 && bins_for(hi, nullptr) <= n_bins) {
        while (lo < hi) {                        // hi stays feasible
          const int64_t mid = (lo + hi) / 2;
          if (bins_for(mid, nullptr) <= n_bins) hi = mid;
          else lo = mid + 1;
        }
        pen = pen_want;
        if (pen > 0 && bins_for(hi, nullptr) > n_bins) pen = 0;   // the cost does not fit at this T
        if (hi >= 8 || (penv && atoi(penv) > 0)) pair_T = hi;
      } else {
        n_bins = 0;
      }
    }
  }
  const bool paired = pair_T > 0;
  // (When the paired layout is forced on a launch with prefix items, its
  // bins run as two waves per SIMD: the prefix keys come from L2 and a step
  // is bound by latency, which a second wave hides; measured on the fp8
  // shared-prefix workload: split-K launch 36 us against 52 us with one
  // wave per SIMD.)
  std::vector<std::array<int32_t, 4>> pieces;
  if (paired) {
    const int64_t m = bins_for(pair_T, &pieces);
    std::vector<int32_t> cnt(m, 0);
    for (const auto &pc : pieces) ++cnt[pc[0]];
    // split two-piece bins while bins are short of n_bins (the form with two
    // waves per SIMD, PA_DECODE_PAIRS=2: each piece its own wave)
    int64_t extra = pair_waves ? n_bins - m : 0;
    std::vector<char> split(m, 0);
    for (int64_t b0 = 0; b0 < m && extra > 0; ++b0)
      if (cnt[b0] == 2) {
        split[b0] = 1;
        --extra;
      }
    // final numbering: unsplit two-piece bins, then single pieces
    std::vector<int32_t> id0(m, -1);
    int32_t nid = 0;
    for (int64_t b0 = 0; b0 < m; ++b0)
      if (cnt[b0] == 2 && !split[b0]) id0[b0] = nid++;
    std::vector<int32_t> id1(m, -1);          // a split bin's second piece
    for (int64_t b0 = 0; b0 < m; ++b0) {
      if (id0[b0] < 0) id0[b0] = nid++;
      if (split[b0]) id1[b0] = nid++;
    }
    const int32_t nb = nid;                   // bins (n_bins in the two-wave form, unless every bin holds one piece)
    plan.pair_stride = !pair_waves && (int64_t)pieces.size() > nb ? nb : 0;
    for (auto &pc : pieces) {
      const int32_t b0 = pc[0];
      int64_t pos;
      if (pc[1] == 0) pos = id0[b0];
      else if (split[b0]) pos = id1[b0];
      else pos = (int64_t)nb + id0[b0];
      pc[0] = (int32_t)pos;                   // item position
      pc[1] = 0;
    }
  }
  std::vector<int64_t> dec_pos;                  // paired: position of each item
  size_t piece_next = 0;

  // prefix chunks: about one workgroup per compute unit over kv heads x
  // column blocks x chunks (a workgroup costs several microseconds to start
  // and finish, so one round of longer chunks beats two of shorter ones)
  int32_t n_kc = 0, kc_len = 0;
  if (cascade && !pre_dec) {
    const int64_t ncb = ((int64_t)prefix_rows * g + kExtCols - 1) / kExtCols;
    const int64_t max_kc = (P + 63) / 64;
    n_kc = (int32_t)std::min<int64_t>(max_kc, std::max<int64_t>(1, 256 / (Hkv * ncb)));
    kc_len = (int32_t)(((P + n_kc - 1) / n_kc + 63) / 64 * 64);
    n_kc = (P + kc_len - 1) / kc_len;
  }

  // One token's key segments [bnd[r], bnd[r + 1]) -> decode items, their
  // partial slots and the token's merge entry (outside the cascade a token of
  // one segment has none: its item writes the output).  own: the segment
  // that ends at the row's last key also writes the row's new K/V.
  // prefix partials of a prefix row: the pieces of its kind-2 unit, or the
  // prefix pass's chunks
  std::vector<int32_t> pre_np;
  auto npre = [&](size_t row_idx) { return pre_dec ? pre_np[row_idx / pre_rows] : n_kc; };
  auto emit_token = [&](int32_t tok, int32_t i, const int32_t *bnd, int32_t nseg, bool own) {
    auto wpos = [&](int32_t r) { return own && bnd[r + 1] == L[i] ? L[i] - 1 : -1; };
    if (cascade) {
      const int32_t n_pre = npre(plan.row_token.size());
      // slots: the prefix partials, then the segments of keys [P, nvis)
      plan.row_token.push_back(tok);
      plan.row_slot0.push_back(plan.n_slots);
      plan.merge.push_back(MergeItem{tok, plan.n_slots, n_pre + nseg, 0});
      for (int32_t r = 0; r < nseg; ++r)
        plan.dec.push_back(DecodeItem{tok, i, bnd[r], bnd[r + 1], plan.n_slots + n_pre + r, wpos(r), 1, 0, 0});
      plan.n_slots += n_pre + nseg;
    } else if (nseg == 1) {
      plan.dec.push_back(DecodeItem{tok, i, bnd[0], bnd[1], -1, wpos(0), 1, 0, 0});
    } else {
      plan.merge.push_back(MergeItem{tok, plan.n_slots, nseg, 0});
      for (int32_t r = 0; r < nseg; ++r)
        plan.dec.push_back(DecodeItem{tok, i, bnd[r], bnd[r + 1], plan.n_slots + r, wpos(r), 1, 0, 0});
      plan.n_slots += nseg;
    }
  };
  // A multi-row chunk's key segments (those of its last row, whose limit is
  // L[i]) -> kind-1 items; row t's partial of segment r is at slot
  // part + t * stride, so each row's slots are consecutive for its merge.
  auto emit_rows = [&](int32_t i, const int32_t *bnd, int32_t nseg) {
    const int32_t c = q[i + 1] - q[i], tok0 = q[i];
    auto item = [&](int32_t r, int32_t part, int32_t stride) {
      plan.dec.push_back(DecodeItem{tok0, i, bnd[r], bnd[r + 1], part, L[i], (int16_t)c, 1, stride});
    };
    if (cascade) {
      const int32_t per = n_kc + nseg;           // the prefix chunks, then the segments
      for (int32_t t = 0; t < c; ++t) {
        plan.row_token.push_back(tok0 + t);
        plan.row_slot0.push_back(plan.n_slots + t * per);
        plan.merge.push_back(MergeItem{tok0 + t, plan.n_slots + t * per, per, 0});
      }
      for (int32_t r = 0; r < nseg; ++r) item(r, plan.n_slots + n_kc + r, per);
      plan.n_slots += c * per;
    } else if (nseg == 1) {
      item(0, -1, 0);
    } else {
      for (int32_t t = 0; t < c; ++t) plan.merge.push_back(MergeItem{tok0 + t, plan.n_slots + t * nseg, nseg, 0});
      for (int32_t r = 0; r < nseg; ++r) item(r, plan.n_slots + r, nseg);
      plan.n_slots += c * nseg;
    }
  };
  std::vector<int32_t> bnd;
  // key segments of a unit whose keys end at nvis: its pieces of the paired
  // layout (the packing visited the units in this order, with the same step
  // counts), or partitions of `part` keys from kstart
  auto segments = [&](int32_t nvis, int32_t start) {
    bnd.clear();
    if (paired) {
      const int64_t st = std::max<int64_t>(0, (int64_t)nvis - start + kKeysPerIter - 1) / kKeysPerIter;
      bnd.push_back(std::min(nvis, start));
      for (int64_t o = 0; o < st && piece_next < pieces.size();) {
        const auto &pc = pieces[piece_next++];
        o = pc[3];
        bnd.push_back((int32_t)std::min<int64_t>(nvis, start + (int64_t)kKeysPerIter * o));
        dec_pos.push_back(pc[0]);
      }
    } else {
      for (int64_t k = start; k < nvis; k += part) bnd.push_back((int32_t)k);
      bnd.push_back(nvis);
    }
    if (bnd.size() == 1 && !cascade) bnd.insert(bnd.begin(), 0);
  };

  // kind-2 units: prefix rows r0 .. r0 + nr - 1 (indices into the row list
  // that the rows' own emission below builds in the same order), piece r's
  // partial at slot row_slot0[row] + r
  for (int32_t u = 0; u < n_pre_units; ++u) {
    const int32_t r0 = u * pre_rows, nr = std::min(pre_rows, prefix_rows - r0);
    segments(P, 0);
    const int32_t nseg = (int32_t)bnd.size() - 1;
    pre_np.push_back(nseg);
    for (int32_t r = 0; r < nseg; ++r)
      plan.dec.push_back(DecodeItem{r0, plan.prefix_req, bnd[r], bnd[r + 1], r, 0, (int16_t)nr, 2, 0});
    plan.max_cols = std::max(plan.max_cols, nr * g);
  }

  for (int32_t i = 0; i < b.num_seqs; ++i) {
    const int32_t c = q[i + 1] - q[i];
    if (c == 0) continue;
    // KV update: a split-K request with one new token has it written by the
    // decode unit that holds its last key; every other new token is written
    // by the scatter pass that runs before the attention kernels
    const bool own_write = kv_update && c == 1 && !on_ext(c);
    // a request of one key-split extend item per kv head: the item writes
    // the request's new rows itself (no other item reads them); so does the
    // last piece of a multi-row chunk
    const bool ext_self = kv_update && on_ext(c) && (int64_t)c * g <= kExtCols;
    const bool rows_self = kv_update && multi(c);
    if (kv_update && !own_write && !ext_self && !rows_self) {
      plan.wseg_read_by_dec |= !on_ext(c);        // the request's own split-K rows read them
      for (int32_t pos = L[i] - c; pos < L[i];) {
        const int32_t end = std::min(L[i], (pos / kBlock + 1) * kBlock);
        plan.wseg.push_back(WriteSeg{i, q[i] + pos - (L[i] - c), pos, end - pos});
        pos = end;
      }
    }
    if (on_ext(c)) {
      ext_reqs.push_back(i);
      continue;
    }
    if (multi(c)) {
      segments(L[i], kstart);
      // the chunk's own keys [L - c, L) all in the last piece, which writes
      // them (the boundary moves down to the block holding key L - c; the
      // piece before it keeps at least 64 - 47 keys, since pieces other than
      // the last hold multiples of 64 keys and c <= 32)
      if (rows_self && bnd.size() > 2) {
        int32_t &last = bnd[bnd.size() - 2];
        last = std::min(last, (L[i] - c) / kBlock * kBlock);
      }
      emit_rows(i, bnd.data(), (int32_t)bnd.size() - 1);
      plan.max_cols = std::max(plan.max_cols, c * g);
      continue;
    }
    for (int32_t t = 0; t < c; ++t) {
      const int32_t nvis = causal ? (L[i] - c + t + 1) : L[i];
      segments(nvis, kstart);
      emit_token(q[i] + t, i, bnd.data(), (int32_t)bnd.size() - 1, own_write);
    }
    plan.max_cols = std::max(plan.max_cols, g);
  }
  // Extend items, all run by one launch of the wide kernel.
  //  * A request with at most kExtCols (token, head) columns per kv head is
  //    one key-split item (mode 1) per kv head: 4 x 32 columns, the key tiles
  //    shared out between two wave groups of the workgroup.
  //  * Wider requests are cut into blocks of kWideCols columns.  A wide item
  //    (mode 0) gives each of its 8 waves 32 columns and every key tile: each
  //    tile copied into LDS feeds twice the columns, and one wide step costs
  //    about 1 / kSplitCost of a key-split step for the same MFMA work (a
  //    64-key tile x 256 columns).  But a wide item's critical path is twice
  //    as long, so a batch of a few long blocks runs them as key-split pairs.
  //  * PA_WIDE_PIECES = n cuts every wide block into n key pieces whose
  //    partial (m, l, o) the merge kernel combines (n is the same for all
  //    blocks of a request: the merge of a row needs all its heads' pieces).
  //    PA_DISABLE_WIDE runs every request as key-split items.
  if (!ext_reqs.empty()) {
    constexpr double kSplitCost = 1.38;          // key-split pair step / wide step (measured, mixed step)
    constexpr int kXcds = 8;
    const bool wide_ok = !env_flag("PA_DISABLE_WIDE");
    const char *force = getenv("PA_WIDE_PIECES");
    auto tiles = [&](int32_t i, int64_t c0, int64_t width) -> int64_t {
      const int64_t c = q[i + 1] - q[i];
      const int64_t kend = causal ? (int64_t)L[i] - c + std::min<int64_t>(c, (c0 + width + g - 1) / g) : L[i];
      return (kend + 63) / 64;
    };
    struct Blk { int32_t req; int32_t c0; int64_t tw; double cost_w, cost_s; };
    std::vector<Blk> fixed_split, wide;          // key-split-only blocks (128 cols); wide-capable blocks (256)
    for (int32_t i : ext_reqs) {
      const int64_t cols = (int64_t)(q[i + 1] - q[i]) * g;
      if (!wide_ok || cols <= kExtCols) {
        for (int64_t c0 = 0; c0 < cols; c0 += kExtCols)
          fixed_split.push_back(Blk{i, (int32_t)c0, 0, 0.0, kSplitCost * ((tiles(i, c0, kExtCols) + 1) / 2)});
      } else {
        for (int64_t c0 = 0; c0 < cols; c0 += kWideCols) {
          const int64_t tw = tiles(i, c0, kWideCols);
          double cs = kSplitCost * ((tiles(i, c0, kExtCols) + 1) / 2);
          if (c0 + kExtCols < cols) cs = std::max(cs, kSplitCost * ((tiles(i, c0 + kExtCols, kExtCols) + 1) / 2));
          wide.push_back(Blk{i, (int32_t)c0, tw, (double)tw, cs});
        }
      }
    }
    // Wide items only when the batch is large enough that the longest one is
    // at most half of a compute unit's average load: then the longest-first
    // schedule balances them and the cheaper wide step wins.  Otherwise (a
    // few long causal blocks, as in one mixed step with a 1.5k-token chunk)
    // every block runs as key-split pairs, whose critical path is half as
    // long: measured on such a step, both a mix of the two and key pieces
    // were no faster than key-split alone.
    int64_t X = INT64_MAX;                       // wide blocks with tw >= X run as key-split pairs
    if (!wide.empty() && !force) {
      double total = 0.0;
      int64_t tmax = 0;
      for (const Blk &b0 : fixed_split) total += b0.cost_s * Hkv;
      for (const Blk &b0 : wide) {
        total += b0.cost_w * Hkv;
        tmax = std::max(tmax, b0.tw);
      }
      if ((double)tmax > 0.5 * total / device_cu_count()) X = 0;
    }
    int32_t np = force ? std::max(1, atoi(force)) : 1;
    auto push = [&](int32_t i, int32_t c0, int32_t mode, int32_t k0, int32_t k1, int32_t slot0, int32_t stride) {
      const int32_t c = q[i + 1] - q[i];
      const int32_t wnew = kv_update && (int64_t)c * g <= kExtCols ? 1 : 0;
      for (int kvh = 0; kvh < Hkv; ++kvh)
        plan.extw.push_back(ExtendItem{i, kvh, q[i], c, L[i], c0, k0, k1, slot0, stride, mode, wnew});
    };
    for (const Blk &b0 : fixed_split) push(b0.req, b0.c0, 1, 0, L[b0.req], -1, 0);
    // forced key pieces: per request, np pieces (no more than the shortest block's tiles)
    std::vector<int32_t> req_np(b.num_seqs, 1), req_base(b.num_seqs, -1);
    if (np > 1) {
      std::vector<int64_t> tmin(b.num_seqs, INT64_MAX);
      for (const Blk &b0 : wide) tmin[b0.req] = std::min(tmin[b0.req], b0.tw);
      for (int32_t i : ext_reqs) {
        if (tmin[i] == INT64_MAX) continue;
        const int32_t c = q[i + 1] - q[i];
        req_np[i] = (int32_t)std::max<int64_t>(1, std::min<int64_t>(np, tmin[i]));
        if (req_np[i] > 1) {
          plan.ext_merge = true;
          req_base[i] = plan.n_slots;
          for (int32_t t = 0; t < c; ++t) plan.merge.push_back(MergeItem{q[i] + t, plan.n_slots + t * req_np[i], req_np[i], 0});
          plan.n_slots += c * req_np[i];
        }
      }
    }
    for (const Blk &b0 : wide) {
      const int32_t i = b0.req;
      if (b0.tw >= X) {
        push(i, b0.c0, 1, 0, L[i], -1, 0);
        if ((int64_t)b0.c0 + kExtCols < (int64_t)(q[i + 1] - q[i]) * g) push(i, b0.c0 + kExtCols, 1, 0, L[i], -1, 0);
        continue;
      }
      const int64_t n = req_np[i];
      for (int64_t pc = 0; pc < n; ++pc) {
        const int32_t k0 = (int32_t)(b0.tw * pc / n * 64);
        const int32_t k1 = pc + 1 == n ? L[i] : (int32_t)(b0.tw * (pc + 1) / n * 64);
        push(i, b0.c0, 0, k0, k1, n > 1 ? req_base[i] + (int32_t)pc : -1, n > 1 ? (int32_t)n : 0);
      }
    }
    // workgroup b runs on XCD b % 8: each (request, kv head) is pinned to one
    // XCD (its K/V stay in that XCD's L2), longest items first within an XCD
    auto cost_of = [&](const ExtendItem &x) -> double {
      const int64_t width = x.mode ? kExtCols : kWideCols;
      const int64_t vis = causal ? (int64_t)x.L - x.c + std::min<int64_t>(x.c, (x.col0 + width + g - 1) / g) : x.L;
      const int64_t t = (std::min<int64_t>(x.key1, vis) + 63) / 64 - x.key0 / 64;
      return x.mode ? kSplitCost * ((t + 1) / 2) : (double)t;
    };
    std::vector<std::vector<ExtendItem>> qx(kXcds);
    for (const ExtendItem &x : plan.extw) qx[(x.req * Hkv + x.kvh) % kXcds].push_back(x);
    for (auto &v : qx)
      std::stable_sort(v.begin(), v.end(), [&](const ExtendItem &x, const ExtendItem &y) { return cost_of(x) > cost_of(y); });
    plan.extw.clear();
    std::vector<size_t> pos(kXcds, 0);
    for (bool more = true; more;) {
      more = false;
      for (int x = 0; x < kXcds; ++x)
        if (pos[x] < qx[x].size()) {
          plan.extw.push_back(qx[x][pos[x]++]);
          more = true;
        }
    }
  }
  // Split-K units, longest first: workgroups are handed to compute units as
  // earlier ones finish, so starting the long units first leaves short ones
  // for the tail (longest-processing-time-first list scheduling).  A stable
  // counting sort on the number of 64-key steps keeps this O(n).
  if (paired) {
    // items to their bin positions (a permutation: no gaps)
    std::vector<DecodeItem> arr(plan.dec.size());
    for (size_t k = 0; k < plan.dec.size(); ++k) arr[(size_t)dec_pos[k]] = plan.dec[k];
    plan.dec.swap(arr);
  } else if (plan.dec.size() > 1) {
    auto steps = [](const DecodeItem &d) { return (d.kv_end - d.kv_begin + kKeysPerIter - 1) / kKeysPerIter; };
    int32_t max_steps = 0;
    for (const DecodeItem &d : plan.dec) max_steps = std::max(max_steps, steps(d));
    std::vector<int32_t> start(max_steps + 2, 0);
    for (const DecodeItem &d : plan.dec) ++start[max_steps - std::max(0, steps(d)) + 1];
    for (int32_t k = 1; k <= max_steps + 1; ++k) start[k] += start[k - 1];
    std::vector<DecodeItem> sorted(plan.dec.size());
    for (const DecodeItem &d : plan.dec) sorted[start[max_steps - std::max(0, steps(d))]++] = d;
    plan.dec.swap(sorted);
  }

  // Prefix items: all chunks of one kv head read the same blocks, so each kv
  // head is pinned to one XCD (workgroup b runs on XCD b % 8).
  if (cascade && !pre_dec) {
    constexpr int kXcds = 8;
    std::vector<std::vector<PrefixItem>> qx(kXcds);
    const int32_t cols = prefix_rows * g;
    for (int kvh = 0; kvh < Hkv; ++kvh)
      for (int32_t c0 = 0; c0 < cols; c0 += kExtCols)
        for (int32_t kc = 0; kc < n_kc; ++kc)
          qx[kvh % kXcds].push_back(PrefixItem{kvh, c0, kc * kc_len, std::min(P, (kc + 1) * kc_len), kc, {0, 0, 0}});
    std::vector<size_t> pos(kXcds, 0);
    for (bool more = true; more;) {
      more = false;
      for (int x = 0; x < kXcds; ++x)
        if (pos[x] < qx[x].size()) {
          plan.pre.push_back(qx[x][pos[x]++]);
          more = true;
        }
    }
  }

  size_t off = 0;
  plan.off_dec = off;
  off = align256(off + plan.dec.size() * sizeof(DecodeItem));
  plan.off_merge = off;
  off = align256(off + plan.merge.size() * sizeof(MergeItem));
  plan.off_extw = off;
  off = align256(off + plan.extw.size() * sizeof(ExtendItem));
  plan.off_pre = off;
  off = align256(off + plan.pre.size() * sizeof(PrefixItem));
  plan.off_rtok = off;
  off = align256(off + plan.row_token.size() * sizeof(int32_t));
  plan.off_rslot = off;
  off = align256(off + plan.row_slot0.size() * sizeof(int32_t));
  plan.off_wseg = off;
  off = align256(off + plan.wseg.size() * sizeof(WriteSeg));
  plan.off_ml = off;
  off = align256(off + (size_t)plan.n_slots * Hq * 2 * sizeof(float));
  plan.off_o = off;
  off = align256(off + (size_t)plan.n_slots * Hq * p.head_dim * sizeof(float));
  plan.bytes = std::max<size_t>(off, 256);
}

// Host-side consistency of a plan's split-K work (PA_CHECK_PLAN=1, for
// tests): every item lies inside its request, and each split-K row's items
// cover its keys [kstart, visible end) once, in order (a multi-row item's
// range ends at its last row's limit, which covers every row of it), with
// distinct partial slots.  Returns null or what is wrong.
static const char *check_decode_plan(const Plan &plan, const pa_batch &b, int causal, bool kv_update) {
  const int32_t *q = b.query_start_loc_host, *L = b.seq_lens_host;
  struct Use { const DecodeItem *d; int32_t slot; };
  std::vector<std::vector<Use>> by_tok(b.num_tokens);
  const int32_t n_rows = (int32_t)plan.row_token.size();
  for (const DecodeItem &d : plan.dec) {
    if (d.kind < 0 || d.kind > 2) return "unknown item kind";
    if (d.kind == 2) {
      // prefix rows row_token[token ..] over keys of the common prefix
      if (!plan.pre_dec) return "a prefix item without the prefix in the split-K kernel";
      if (d.req != plan.prefix_req || d.token < 0 || d.ntok < 1 || d.token + d.ntok > n_rows) return "prefix item rows out of range";
      if (d.kv_begin < 0 || d.kv_begin >= d.kv_end || d.kv_end > plan.kstart) return "prefix item keys outside the prefix";
      if ((d.kv_begin % kBlock) != 0) return "a prefix piece that starts inside a block";
      for (int32_t t = 0; t < d.ntok; ++t) {
        const int32_t row = plan.row_token[d.token + t];
        const int32_t slot = plan.row_slot0[d.token + t] + d.part;
        if (row < 0 || row >= b.num_tokens) return "prefix row out of range";
        if (d.part < 0 || slot >= plan.n_slots) return "prefix partial slot out of range";
        by_tok[row].push_back(Use{&d, slot});
      }
      continue;
    }
    if (d.req < 0 || d.req >= b.num_seqs || d.token < 0 || d.token >= b.num_tokens) return "item row out of range";
    const int32_t c = q[d.req + 1] - q[d.req];
    const int32_t n = d.kind == 0 ? 1 : d.ntok;
    if (d.kind == 0 && d.ntok != 1) return "a one-row item with ntok != 1";
    if (d.kind == 1 && (d.token != q[d.req] || n != c || d.wpos != L[d.req] || n < 2))
      return "a multi-row item that is not its request's whole chunk";
    if (d.token < q[d.req] || d.token + n > q[d.req + 1]) return "item rows outside their request";
    if (d.kv_begin < 0 || d.kv_begin >= d.kv_end || d.kv_end > L[d.req]) return "item keys outside the row";
    if (d.kind == 0 && d.wpos != -1 && (d.wpos != L[d.req] - 1 || d.kv_end != L[d.req])) return "bad own-write position";
    // (with the KV update the last piece stores the rows' K/V: it holds all their keys)
    if (kv_update && d.kind == 1 && d.kv_end == L[d.req] && d.kv_begin > L[d.req] - n)
      return "a multi-row item's last piece misses some of its rows' keys";
    if (kv_update && d.kind == 1 && d.kv_end < L[d.req] && d.kv_end > L[d.req] - n)
      return "a multi-row item's rows' keys split between pieces";
    if (d.kind == 1 && (d.kv_begin % kBlock) != 0) return "a multi-row piece that starts inside a block";
    for (int32_t t = 0; t < n; ++t) {
      const int32_t slot = d.part < 0 ? -1 : d.part + t * (d.kind == 0 ? 0 : d.stride);
      if (slot >= plan.n_slots) return "partial slot out of range";
      by_tok[d.token + t].push_back(Use{&d, slot});
    }
  }
  // a row's keys start at 0, or after the prefix when the prefix pass covers it
  const int32_t first_key = plan.pre_dec ? 0 : plan.kstart;
  std::vector<char> used(plan.n_slots, 0);
  for (int32_t t = 0; t < b.num_tokens; ++t) {
    auto &v = by_tok[t];
    if (v.empty()) continue;
    std::sort(v.begin(), v.end(), [](const Use &x, const Use &y) { return x.d->kv_begin < y.d->kv_begin; });
    const DecodeItem *own = nullptr;          // an item of the row's own request
    for (const Use &u : v)
      if (u.d->kind != 2) own = u.d;
    if (!own) return "a prefix row without its own keys";
    const int32_t i = own->req, c = q[i + 1] - q[i];
    if (t < q[i] || t >= q[i + 1]) return "a row's items belong to another request";
    const int32_t nvis = causal ? L[i] - c + (t - q[i]) + 1 : L[i];
    const int32_t want_end = own->kind == 1 ? L[i] : nvis;
    if (v.front().d->kv_begin != first_key || v.back().d->kv_end != want_end) return "a row's items do not cover its keys";
    for (size_t k = 0; k < v.size(); ++k) {
      if (k && v[k].d->kv_begin != v[k - 1].d->kv_end) return "a row's items overlap or leave a gap";
      const int32_t pt = v[k].slot;
      if (pt < 0 && (v.size() > 1 || plan.kstart > 0)) return "a split row's item without a partial slot";
      if (pt >= 0) {
        if (used[pt]) return "a partial slot used twice";
        used[pt] = 1;
      }
    }
  }
  // every slot a merge reads is written (the prefix pass's chunks count as
  // written when it runs)
  for (const MergeItem &m : plan.merge) {
    if (m.first < 0 || m.count < 1 || m.first + m.count > plan.n_slots) return "merge slots out of range";
    for (int32_t k = 0; k < m.count; ++k)
      if (!used[m.first + k] && !(plan.kstart > 0 && !plan.pre_dec)) return "a merged slot that no item writes";
  }
  return nullptr;
}

static pa_status check_attention_args(const pa_kv_pool *pool, const pa_batch *batch,
                                      pa_dtype q_dtype, int32_t Hq, bool need_ptrs) {
  pa_status st = check_pool(pool, need_ptrs);
  if (st != PA_OK) return st;
  if ((st = check_batch(batch, need_ptrs)) != PA_OK) return st;
  if (Hq <= 0 || Hq % pool->num_kv_heads)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads %d not a positive multiple of num_kv_heads %d", Hq, pool->num_kv_heads);
  if (Hq / pool->num_kv_heads > 16)
    return fail(PA_ERR_UNSUPPORTED, "more than 16 q heads per kv head");
  if (q_dtype != PA_F32 && q_dtype != PA_BF16) return fail(PA_ERR_INVALID_ARG, "q_dtype must be F32 or BF16");
  if ((q_dtype == PA_F32) != (pool->kv_dtype == PA_F32))
    return fail(PA_ERR_UNSUPPORTED, "q_dtype F32 pairs with an F32 pool, BF16 with BF16/FP8 pools");
  return PA_OK;
}

}  // namespace pa

using namespace pa;

// ================================================================== C ABI ===

extern "C" {

pa_status pa_prepare_metadata(int32_t num_seqs, const int32_t *num_computed,
                              const int32_t *num_scheduled, int32_t *query_start_loc,
                              int32_t *seq_lens) {
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "negative num_seqs");
  if (!query_start_loc || (num_seqs > 0 && (!num_computed || !num_scheduled || !seq_lens)))
    return fail(PA_ERR_INVALID_ARG, "NULL pointer");
  int64_t acc = 0;
  query_start_loc[0] = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    if (num_computed[i] < 0 || num_scheduled[i] < 0)
      return fail(PA_ERR_INVALID_ARG, "negative count at request %d", i);
    acc += num_scheduled[i];
    const int64_t len = (int64_t)num_computed[i] + num_scheduled[i];
    if (acc > INT32_MAX || len > INT32_MAX) return fail(PA_ERR_INVALID_ARG, "counts overflow int32");
    query_start_loc[i + 1] = (int32_t)acc;
    seq_lens[i] = (int32_t)len;
  }
  return PA_OK;
}

pa_status pa_slot_mapping(const pa_batch *batch, int32_t block_size, int64_t *slot_mapping,
                          pa_stream_t stream) {
  pa_status st = check_batch(batch, true);
  if (st != PA_OK) return st;
  if (block_size != kBlock) return fail(PA_ERR_UNSUPPORTED, "block_size %d (only 16)", block_size);
  if (batch->num_tokens > 0 && !slot_mapping) return fail(PA_ERR_INVALID_ARG, "slot_mapping is NULL");
  int max_c = 0;
  for (int32_t i = 0; i < batch->num_seqs; ++i)
    max_c = std::max(max_c, batch->query_start_loc_host[i + 1] - batch->query_start_loc_host[i]);
  hipError_t e = launch_slot_mapping(*batch, slot_mapping, max_c, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : hip_fail(e, "k_slot_mapping launch");
}

pa_status pa_write_kv(const pa_kv_pool *pool, const void *key, const void *value, pa_dtype in_dtype,
                      const int64_t *slot_mapping, int32_t num_tokens, pa_stream_t stream) {
  pa_status st = check_pool(pool, true);
  if (st != PA_OK) return st;
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "negative num_tokens");
  if (num_tokens > 0 && (!key || !value || !slot_mapping)) return fail(PA_ERR_INVALID_ARG, "NULL key/value/slot_mapping");
  if (in_dtype != PA_F32 && in_dtype != PA_BF16) return fail(PA_ERR_INVALID_ARG, "in_dtype must be F32 or BF16");
  if (pool->kv_dtype != PA_FP8_E4M3 && pool->kv_dtype != in_dtype)
    return fail(PA_ERR_UNSUPPORTED, "in_dtype must match an F32/BF16 pool");
  if (env_flag("PA_VALIDATE") && num_tokens > 0) {
    std::vector<int64_t> sl(num_tokens);
    hipError_t e = hipMemcpyAsync(sl.data(), slot_mapping, sl.size() * 8, hipMemcpyDeviceToHost, (hipStream_t)stream);
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "validate: slot read");
    const int64_t cap = (int64_t)pool->num_blocks * pool->block_size;
    for (int32_t n = 0; n < num_tokens; ++n)
      if (sl[n] >= cap) return fail(PA_ERR_VALIDATION, "slot_mapping[%d] = %lld >= capacity %lld", n, (long long)sl[n], (long long)cap);
  }
  hipError_t e = launch_write_kv(*pool, key, value, in_dtype, slot_mapping, num_tokens, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : hip_fail(e, "k_write_kv launch");
}

size_t pa_attention_workspace_bytes(const pa_kv_pool *pool, const pa_batch *batch, int32_t num_q_heads) {
  // the dtype only selects kernels; BF16 gives the largest (extend-capable) plan shape
  const pa_dtype qd = pool && pool->kv_dtype == PA_F32 ? PA_F32 : PA_BF16;
  if (check_attention_args(pool, batch, qd, num_q_heads, false) != PA_OK) return 0;
  // the plan with the KV update holds every section the plan without it has
  Plan plan;
  build_plan(*pool, *batch, num_q_heads, qd, 1, true, plan);
  Plan plan_nc;
  build_plan(*pool, *batch, num_q_heads, qd, 0, true, plan_nc);
  if (env_flag("PA_CHECK_PLAN")) {
    const char *why = check_decode_plan(plan, *batch, 1, true);
    if (!why) why = check_decode_plan(plan_nc, *batch, 0, true);
    if (why) {
      fail(PA_ERR_VALIDATION, "plan check: %s", why);
      return 0;
    }
  }
  return std::max(plan.bytes, plan_nc.bytes);
}

}  // extern "C"

namespace pa {

// The new rows of the attention call that includes the KV update.
struct KvUpdate {
  const void *key;
  const void *value;
  int64_t *slot_mapping;   // may be null
};

// no_alloc: the call's scratch is the library's static device array (the
// workspace arguments are ignored), the work lists are copied into it by
// kernels that carry them as arguments, and nothing is allocated (no
// staging ring, no side stream).
static pa_status attention_impl(const pa_kv_pool *pool, const pa_batch *batch, const void *query,
                                pa_dtype q_dtype, int32_t num_q_heads, float softmax_scale,
                                int32_t causal, void *output, void *workspace,
                                size_t workspace_bytes, hipStream_t s, const KvUpdate *kvu,
                                bool no_alloc = false) {
  pa_status st = check_attention_args(pool, batch, q_dtype, num_q_heads, true);
  if (st != PA_OK) return st;
  if (batch->num_tokens > 0 && (!query || !output)) return fail(PA_ERR_INVALID_ARG, "NULL query/output");
  if (kvu && batch->num_tokens > 0 && (!kvu->key || !kvu->value)) return fail(PA_ERR_INVALID_ARG, "NULL key/value");
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.0f))
    return fail(PA_ERR_INVALID_ARG, "softmax_scale must be finite and positive");
  if (batch->num_tokens == 0) return PA_OK;
  const bool graph = capturing(s);
  if (graph && env_flag("PA_VALIDATE"))
    return fail(PA_ERR_UNSUPPORTED, "PA_VALIDATE reads the block table back synchronously; not under graph capture");
  if (env_flag("PA_VALIDATE") && (st = validate_block_table(batch, pool->num_blocks, s)) != PA_OK) return st;

  Plan plan;
  build_plan(*pool, *batch, num_q_heads, q_dtype, causal ? 1 : 0, kvu != nullptr, plan);
  if (no_alloc) {
    if (plan.bytes > kStaticScratchBytes)
      return fail(PA_ERR_WORKSPACE, "batch needs %zu bytes of scratch, more than the %zu of the static scratch "
                  "(pa_write_kv_attention with a workspace has no such limit)", plan.bytes, kStaticScratchBytes);
    if ((st = static_scratch(&workspace)) != PA_OK) return st;
    workspace_bytes = kStaticScratchBytes;
  }
  if (!workspace) return fail(PA_ERR_WORKSPACE, "workspace is NULL");
  if (((uintptr_t)workspace & 255) != 0) return fail(PA_ERR_WORKSPACE, "workspace not 256-byte aligned");
  if (workspace_bytes < plan.bytes)
    return fail(PA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, plan.bytes);

  // the work lists: written into a staging slot that the kernels read
  // directly, or (PA_PLAN_UPLOAD=1) copied into the workspace.  Under graph
  // capture they are written once into the captured-plan arena, which the
  // graph's kernels read at every replay (PA_GRAPH_PLAN_COPY=1, a full or
  // absent arena, and the call that allocates nothing: copied into the
  // workspace by captured copy kernels that carry them as arguments).
  const size_t plan_bytes = plan.off_ml;
  StageSlot *slot = nullptr;
  int32_t *release = nullptr;                    // set by the call's first kernel (staging ring)
  const char *items = (const char *)workspace;
  auto fill = [&](char *host) {
    memset(host, 0, plan_bytes);
    if (!plan.dec.empty()) memcpy(host + plan.off_dec, plan.dec.data(), plan.dec.size() * sizeof(DecodeItem));
    if (!plan.merge.empty()) memcpy(host + plan.off_merge, plan.merge.data(), plan.merge.size() * sizeof(MergeItem));
    if (!plan.extw.empty()) memcpy(host + plan.off_extw, plan.extw.data(), plan.extw.size() * sizeof(ExtendItem));
    if (!plan.pre.empty()) memcpy(host + plan.off_pre, plan.pre.data(), plan.pre.size() * sizeof(PrefixItem));
    // the prefix row list: read by the prefix pass and by kind-2 decode items
    if (!plan.row_token.empty()) {
      memcpy(host + plan.off_rtok, plan.row_token.data(), plan.row_token.size() * sizeof(int32_t));
      memcpy(host + plan.off_rslot, plan.row_slot0.data(), plan.row_slot0.size() * sizeof(int32_t));
    }
    if (!plan.wseg.empty()) memcpy(host + plan.off_wseg, plan.wseg.data(), plan.wseg.size() * sizeof(WriteSeg));
  };
  if (!graph && !no_alloc) arena_ensure();
  char *arena_host = nullptr;
  const char *arena_dev = nullptr;
  if (plan_bytes && graph && !no_alloc && !env_flag("PA_GRAPH_PLAN_COPY") &&
      arena_take(plan_bytes, &arena_host, &arena_dev)) {
    fill(arena_host);                            // read by every replay of the graph
    items = arena_dev;
  } else if (plan_bytes && (graph || no_alloc)) {
    std::vector<char> host(plan_bytes);
    fill(host.data());
    hipError_t ce = launch_plan_copy(workspace, host.data(), plan_bytes, s);
    if (ce != hipSuccess) return hip_fail(ce, "plan copy launch");
  } else if (plan_bytes) {
    if ((st = stage_acquire(plan_bytes, s, &slot, &release)) != PA_OK) return st;
    char *host = (char *)slot->host;
    fill(host);
    if (env_flag("PA_PLAN_UPLOAD")) {
      hipError_t ce = hipMemcpyAsync(workspace, host, plan_bytes, hipMemcpyHostToDevice, s);
      if (ce != hipSuccess) return hip_fail(ce, "plan upload");
    } else {
      items = (const char *)slot->dev;
    }
  }
  char *ws = (char *)workspace;
  const int g_total = num_q_heads / pool->num_kv_heads;
  const float log2e = 1.4426950408889634f;
  const float kscale = pool->kv_dtype == PA_FP8_E4M3 ? pool->k_scale : 1.0f;
  const float vscale = pool->kv_dtype == PA_FP8_E4M3 ? pool->v_scale : 1.0f;

  // Every check and set-up that can fail without a HIP launch error is done
  // before the first launch, so that such a failure leaves the pool as it was.
  hipStream_t xs = s;
  SideStream *side = nullptr;
  // (not with key pieces: their partials are merged on the caller's stream)
  const bool fork = !no_alloc && !plan.extw.empty() && plan.merge.empty() && !plan.dec.empty() &&
                    env_flag("PA_OVERLAP");
  if (fork && (st = side_stream(&side)) != PA_OK) return st;

  hipError_t e = hipSuccess;
  // KV update, first part: the new rows no decode unit writes itself (slots
  // derived on the fly), before any kernel that may read them.  When only
  // extend items read them and there is split-K work on the matrix-core
  // kernel, extra workgroups of that launch write them, and it runs before
  // the extend and prefix kernels; otherwise (split-K rows of the same
  // requests read them, PA_SCATTER_LAUNCH=1, fp32 pools, no split-K rows) a
  // launch of its own does, first.
  const bool fused_scatter = !plan.wseg.empty() && !plan.dec.empty() && !plan.wseg_read_by_dec &&
                             pool->kv_dtype != PA_F32 && !fork && !env_flag("PA_SCATTER_LAUNCH");
  // The work lists of the launches after the split-K one (merge, extend and
  // prefix-pass items), when they sit in host memory: copy workgroups of the
  // split-K launch move them to the same offsets in the workspace, so those
  // launches' waves read them from device memory instead of over PCIe.
  const char *late = items;                      // where the later launches read their lists
  const size_t late_bytes = plan.off_rtok - plan.off_merge;
  const bool stage_late = items != (const char *)workspace && !plan.dec.empty() && late_bytes > 0 &&
                          (!plan.merge.empty() || !plan.extw.empty() || !plan.pre.empty()) &&
                          pool->kv_dtype != PA_F32 && !fork && !env_flag("PA_LISTS_IN_HOST");
  if (stage_late) late = (const char *)workspace;
  // the split-K launch (with the scatter workgroups when it carries them)
  auto run_decode = [&]() -> pa_status {
    if (plan.dec.empty()) return PA_OK;
    DecodeArgs a{};
    a.q = query;
    a.out = output;
    a.k_cache = pool->k_cache;
    a.v_cache = pool->v_cache;
    a.block_table = batch->block_table;
    a.items = (const DecodeItem *)(items + plan.off_dec);
    a.pair_stride = plan.pair_stride;
    a.causal = causal;
    if (plan.pre_dec) {
      a.row_token = (const int32_t *)(items + plan.off_rtok);
      a.row_slot0 = (const int32_t *)(items + plan.off_rslot);
      a.prefix_bt = batch->block_table + (int64_t)plan.prefix_req * batch->bt_stride;
    }
    a.max_cols = plan.max_cols;
    a.part_ml = (float *)(ws + plan.off_ml);
    a.part_o = (float *)(ws + plan.off_o);
    a.n_items = (int32_t)plan.dec.size();
    a.bt_stride = batch->bt_stride;
    a.num_blocks = pool->num_blocks;
    a.num_kv_heads = pool->num_kv_heads;
    a.num_q_heads = num_q_heads;
    a.g_total = g_total;
    a.scale_log2 = softmax_scale * log2e * kscale;
    a.v_scale = vscale;
    if (kvu) {
      a.knew = kvu->key;
      a.vnew = kvu->value;
      a.slots_out = kvu->slot_mapping;
      a.k_store = pool->k_cache;
      a.v_store = pool->v_cache;
      a.enc_k_scale = kscale;
      a.enc_v_scale = vscale;
    }
    if (fused_scatter) {
      a.wseg = (const WriteSeg *)(items + plan.off_wseg);
      a.n_wseg_units = (int32_t)plan.wseg.size() * pool->num_kv_heads;
    }
    if (stage_late) {
      a.copy_src = (const uint4 *)(items + plan.off_merge);
      a.copy_dst = (uint4 *)((char *)workspace + plan.off_merge);
      a.copy_vecs = (int32_t)(late_bytes / 16);
      a.n_copy_units = (a.copy_vecs + kCopyVecsPerUnit - 1) / kCopyVecsPerUnit;
    }
    // q heads per launch: the whole GQA group where the registers allow it,
    // otherwise the group is covered by several launches (fp32 pools)
    const int g_max = 16;
    for (int h0 = 0; h0 < g_total; h0 += g_max) {
      a.h0 = h0;
      a.g = std::min(g_max, g_total - h0);
      const int g_tmpl = a.g <= 1 ? 1 : a.g <= 2 ? 2 : a.g <= 4 ? 4 : a.g <= 8 ? 8 : 16;
      a.release = release;
      release = nullptr;
      e = launch_decode(*pool, q_dtype, a, g_tmpl, s);
      if (e != hipSuccess) return hip_fail(e, "k_decode launch");
      a.knew = a.vnew = nullptr;                  // rows written by the first launch
      a.slots_out = nullptr;
      a.n_wseg_units = 0;
      a.n_copy_units = 0;
    }
    return PA_OK;
  };
  // the scatter as a launch of its own
  auto run_scatter = [&]() -> pa_status {
    if (plan.wseg.empty() || fused_scatter) return PA_OK;
    WriteArgs w{};
    w.key = kvu->key;
    w.value = kvu->value;
    w.segs = (const WriteSeg *)(items + plan.off_wseg);
    w.block_table = batch->block_table;
    w.slots_out = kvu->slot_mapping;
    w.k_cache = pool->k_cache;
    w.v_cache = pool->v_cache;
    w.num_blocks = pool->num_blocks;
    w.n_segs = (int32_t)plan.wseg.size();
    w.bt_stride = batch->bt_stride;
    w.num_kv_heads = pool->num_kv_heads;
    w.k_scale = kscale;
    w.v_scale = vscale;
    w.release = release;                         // the call's first kernel
    release = nullptr;
    e = launch_write_new(*pool, q_dtype, w, s);
    if (e != hipSuccess) return hip_fail(e, "k_write_new launch");
    return PA_OK;
  };
  // the extend launch, with the merge workgroups when it carries them
  auto run_extend = [&](bool with_merge) -> pa_status {
    if (plan.extw.empty()) return PA_OK;
    ExtendArgs x{};
    x.q = query;
    x.out = output;
    x.k_cache = pool->k_cache;
    x.v_cache = pool->v_cache;
    x.block_table = batch->block_table;
    x.items = (const ExtendItem *)(late + plan.off_extw);
    x.part_ml = (float *)(ws + plan.off_ml);
    x.part_o = (float *)(ws + plan.off_o);
    x.n_items = (int32_t)plan.extw.size();
    x.bt_stride = batch->bt_stride;
    x.num_blocks = pool->num_blocks;
    x.num_kv_heads = pool->num_kv_heads;
    x.num_q_heads = num_q_heads;
    x.g = g_total;
    x.causal = causal ? 1 : 0;
    x.scale_log2 = softmax_scale * log2e * kscale;
    x.k_scale = kscale;
    x.v_scale = vscale;
    if (kvu) {
      x.knew = kvu->key;
      x.vnew = kvu->value;
      x.slots_out = kvu->slot_mapping;
      x.k_store = pool->k_cache;
      x.v_store = pool->v_cache;
      x.enc_k_scale = kscale;
      x.enc_v_scale = vscale;
    }
    if (with_merge) {
      x.mitems = (const MergeItem *)(late + plan.off_merge);
      x.n_merge_units = (int32_t)plan.merge.size() * num_q_heads;
    }
    x.release = release;
    release = nullptr;
    e = launch_extend_wide(*pool, x, xs);
    if (e != hipSuccess) return hip_fail(e, "k_extend_wide launch");
    return PA_OK;
  };
  // the shared-prefix pass
  auto run_prefix = [&]() -> pa_status {
    if (plan.pre.empty()) return PA_OK;
    ExtendArgs x{};
    x.q = query;
    x.k_cache = pool->k_cache;
    x.v_cache = pool->v_cache;
    x.pitems = (const PrefixItem *)(late + plan.off_pre);
    x.row_token = (const int32_t *)(items + plan.off_rtok);
    x.row_slot0 = (const int32_t *)(items + plan.off_rslot);
    x.prefix_bt = batch->block_table + (int64_t)plan.prefix_req * batch->bt_stride;
    x.part_ml = (float *)(ws + plan.off_ml);
    x.part_o = (float *)(ws + plan.off_o);
    x.prefix_cols = (int32_t)plan.row_token.size() * g_total;
    x.n_items = (int32_t)plan.pre.size();
    x.num_blocks = pool->num_blocks;
    x.num_kv_heads = pool->num_kv_heads;
    x.num_q_heads = num_q_heads;
    x.g = g_total;
    x.causal = 0;
    x.scale_log2 = softmax_scale * log2e * kscale;
    x.k_scale = kscale;
    x.v_scale = vscale;
    x.release = release;
    release = nullptr;
    e = launch_prefix(*pool, x, s);
    if (e != hipSuccess) return hip_fail(e, "k_prefix launch");
    return PA_OK;
  };
  // the merge as a launch of its own
  auto run_merge = [&]() -> pa_status {
    if (plan.merge.empty()) return PA_OK;
    MergeArgs m{};
    m.out = output;
    m.part_ml = (const float *)(ws + plan.off_ml);
    m.part_o = (const float *)(ws + plan.off_o);
    m.items = (const MergeItem *)(late + plan.off_merge);
    m.n_items = (int32_t)plan.merge.size();
    m.num_q_heads = num_q_heads;
    if (plan.merge.size() <= (size_t)kMergeInline) {
      m.inline_items = 1;
      memcpy(m.inl, plan.merge.data(), plan.merge.size() * sizeof(MergeItem));
    }
    e = launch_merge(q_dtype, pool->head_dim, m, s);
    if (e != hipSuccess) return hip_fail(e, "k_merge launch");
    return PA_OK;
  };

  // Launch order.  The extend launch carries the merge of the split-K (and
  // prefix-pass) partials when the extend items do not produce partials of
  // their own (PA_MERGE_LAUNCH=1: a launch of its own), so the split-K launch
  // and the prefix pass run before it; without the side stream the order is
  // scatter (when not carried), split-K (with the carried scatter), prefix,
  // extend (with the merge), merge (when not carried).
  if (fork) {
    // the extend kernel on the side stream, beside the split-K work
    if ((st = run_scatter()) != PA_OK) return st;
    if ((e = hipEventRecord(side->fork, s)) != hipSuccess) return hip_fail(e, "fork record");
    if ((e = hipStreamWaitEvent(side->stream, side->fork, 0)) != hipSuccess) return hip_fail(e, "fork wait");
    xs = side->stream;
    if ((st = run_extend(false)) != PA_OK) return st;
    if ((st = run_prefix()) != PA_OK) return st;
    if ((st = run_decode()) != PA_OK) return st;
    if ((st = run_merge()) != PA_OK) return st;
  } else {
    const bool merge_in_extend = !plan.merge.empty() && !plan.extw.empty() && !plan.ext_merge &&
                                 !env_flag("PA_MERGE_LAUNCH");
    if ((st = run_scatter()) != PA_OK) return st;
    if ((st = run_decode()) != PA_OK) return st;
    if ((st = run_prefix()) != PA_OK) return st;
    if ((st = run_extend(merge_in_extend)) != PA_OK) return st;
    if (!merge_in_extend && (st = run_merge()) != PA_OK) return st;
  }
  if (fork) {
    if ((e = hipEventRecord(side->join, xs)) != hipSuccess) return hip_fail(e, "join record");
    if ((e = hipStreamWaitEvent(s, side->join, 0)) != hipSuccess) return hip_fail(e, "join wait");
  }
  return PA_OK;
}

}  // namespace pa

extern "C" {

pa_status pa_attention(const pa_kv_pool *pool, const pa_batch *batch, const void *query,
                       pa_dtype q_dtype, int32_t num_q_heads, float softmax_scale, int32_t causal,
                       void *output, void *workspace, size_t workspace_bytes, pa_stream_t stream) {
  return attention_impl(pool, batch, query, q_dtype, num_q_heads, softmax_scale, causal, output,
                        workspace, workspace_bytes, (hipStream_t)stream, nullptr);
}

pa_status pa_write_kv_attention(const pa_kv_pool *pool, const pa_batch *batch, const void *query,
                                const void *key, const void *value, pa_dtype q_dtype,
                                int32_t num_q_heads, float softmax_scale, int32_t causal,
                                int64_t *slot_mapping, void *output, void *workspace,
                                size_t workspace_bytes, pa_stream_t stream) {
  const KvUpdate kvu{key, value, slot_mapping};
  return attention_impl(pool, batch, query, q_dtype, num_q_heads, softmax_scale, causal, output,
                        workspace, workspace_bytes, (hipStream_t)stream, &kvu);
}

pa_status pa_write_kv_attention_noalloc(const pa_kv_pool *pool, const pa_batch *batch,
                                        const void *query, const void *key, const void *value,
                                        pa_dtype q_dtype, int32_t num_q_heads, float softmax_scale,
                                        int32_t causal, int64_t *slot_mapping, void *output,
                                        pa_stream_t stream) {
  const KvUpdate kvu{key, value, slot_mapping};
  return attention_impl(pool, batch, query, q_dtype, num_q_heads, softmax_scale, causal, output,
                        nullptr, 0, (hipStream_t)stream, &kvu, true);
}

size_t pa_noalloc_scratch_bytes(void) { return kStaticScratchBytes; }

pa_status pa_zero_blocks(const pa_kv_pool *pool, const int32_t *block_ids, int32_t num_ids,
                         pa_stream_t stream) {
  pa_status st = check_pool(pool, true);
  if (st != PA_OK) return st;
  if (num_ids < 0 || (num_ids > 0 && !block_ids)) return fail(PA_ERR_INVALID_ARG, "invalid block id list");
  hipError_t e = launch_zero_blocks(*pool, block_ids, num_ids, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : hip_fail(e, "k_zero_blocks launch");
}

size_t pa_kv_cache_bytes(const pa_kv_pool *pool) {
  if (!pool || pool->num_blocks <= 0 || pool->block_size <= 0 || pool->num_kv_heads <= 0 || pool->head_dim <= 0)
    return 0;
  return (size_t)pool->num_blocks * pool->block_size * pool->num_kv_heads * pool->head_dim *
         elem_bytes(pool->kv_dtype);
}

int64_t pa_kv_elem_offset(const pa_kv_pool *pool, int32_t which, int64_t block, int32_t offset,
                          int32_t head, int32_t dim) {
  if (!pool || block < 0 || block >= pool->num_blocks || offset < 0 || offset >= pool->block_size ||
      head < 0 || head >= pool->num_kv_heads || dim < 0 || dim >= pool->head_dim || (which != 0 && which != 1))
    return -1;
  const int64_t S = pool->block_size, D = pool->head_dim;
  const int64_t tile = (block * pool->num_kv_heads + head) * S * D;
  if (which == 1) return tile + (int64_t)dim * S + offset;  // [dim][slot]
  const int64_t E = 16 / elem_bytes(pool->kv_dtype);
  return tile + ((dim / E) * S + offset) * E + dim % E;     // [chunk][slot][E]
}

const char *pa_status_string(pa_status status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE";
    case PA_ERR_VALIDATION: return "PA_ERR_VALIDATION";
    case PA_ERR_HIP: return "PA_ERR_HIP";
    case PA_ERR_CAPACITY: return "PA_ERR_CAPACITY";
  }
  return "PA_ERR_UNKNOWN";
}

const char *pa_last_error(void) { return g_last_error.c_str(); }

pa_status pa_profile_enable(int32_t enable) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  prof_reset_locked();
  g_prof_on = enable != 0;
  return PA_OK;
}

pa_status pa_profile_read(const char *kernel, int32_t *launches, double *total_ms) {
  if (!kernel || !launches || !total_ms) return fail(PA_ERR_INVALID_ARG, "NULL argument");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  int32_t n = 0;
  double ms = 0;
  for (auto &r : g_prof) {
    if (strcmp(r.name, kernel) != 0) continue;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e != hipSuccess) return hip_fail(e, "profile wait");
    float t = 0;
    if ((e = hipEventElapsedTime(&t, r.start, r.stop)) != hipSuccess) return hip_fail(e, "profile time");
    ms += t;
    ++n;
  }
  *launches = n;
  *total_ms = ms;
  return PA_OK;
}

pa_status pa_placement_check(pa_placement *out) {
  if (!out) return fail(PA_ERR_INVALID_ARG, "NULL argument");
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "placement check: device");
  if (cus <= 0) return fail(PA_ERR_HIP, "placement check: no compute units");
  const size_t n_one = 4 * (size_t)cus, n_two = 8 * (size_t)cus, n_wide = 2 * (size_t)cus;
  const size_t n_all = 2 * (n_one + n_two + n_wide);
  uint32_t *ids = nullptr;
  if ((e = hipMalloc((void **)&ids, n_all * sizeof(uint32_t))) != hipSuccess) return hip_fail(e, "placement check: alloc");
  std::vector<uint32_t> h(n_all);
  uint32_t *one = ids, *two = one + 2 * n_one, *wide = two + 2 * n_two;
  e = launch_placement_probe(cus, one, two, wide, nullptr);
  if (e == hipSuccess) e = hipMemcpy(h.data(), ids, n_all * sizeof(uint32_t), hipMemcpyDeviceToHost);
  const hipError_t ef = hipFree(ids);
  if (e == hipSuccess) e = ef;
  if (e != hipSuccess) return hip_fail(e, "placement check: probe");
  // a SIMD: XCD id, and HW_ID's SIMD (bits 5:4) and CU / array / engine
  // fields (bits 15:8); the wave slot and queue pipe fields are left out
  auto simd = [&](const uint32_t *r, size_t u) -> uint64_t {
    const uint32_t hw = r[2 * u], xcc = r[2 * u + 1] & 0xF;
    return ((uint64_t)xcc << 16) | (((hw >> 8) & 0xFF) << 2) | ((hw >> 4) & 3);
  };
  std::map<uint64_t, int> per_simd;
  for (size_t u = 0; u < n_one; ++u) ++per_simd[simd(h.data() + 0, u)];
  size_t alone = 0;
  for (size_t u = 0; u < n_one; ++u) alone += per_simd[simd(h.data(), u)] == 1;
  const uint32_t *h2 = h.data() + 2 * n_one, *hw3 = h2 + 2 * n_two;
  size_t paired = 0;
  for (size_t u = 0; u < n_one; ++u) paired += simd(h2, u) == simd(h2, u + n_one);
  size_t rr = 0;
  std::set<uint32_t> xcds;
  for (size_t b = 0; b < n_wide; ++b) {
    const uint32_t x = hw3[2 * b + 1] & 0xF;
    xcds.insert(x);
    rr += x == b % 8;
  }
  out->compute_units = cus;
  out->xcds = (int32_t)xcds.size();
  out->one_wave_alone = (float)alone / (float)n_one;
  out->two_wave_paired = (float)paired / (float)n_one;
  out->xcd_round_robin = (float)rr / (float)n_wide;
  return PA_OK;
}

}  // extern "C"
