// C ABI of the host-KV attention layer: argument checks, the kernel adaptor (instance
// lookup and launch planning), the host cache manager, and dispatch onto a HIP stream.
//
// "Paper Notes: DirectKV", System Architecture: the Kernel Generator's pre-built
// instances over <data type, head dim, tile> are the explicit template instances in the
// kernel files; the Kernel Adaptor here picks one by dtype, head dim, group size and
// phase; the KV Cache Manager allocates the pinned host buffers that kernels dereference
// in place. Every argument is checked before any HIP call, so a rejected call enqueues
// nothing and leaves the cache untouched.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/directkv.h"
#include "dkv_internal.h"

using namespace dkv;

namespace {

thread_local std::string g_err;
constexpr int32_t kMagic = 0x444B5631;  // marks descriptors made by kv_alloc_host

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(DKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t elem_size(int dtype) { return dtype == DKV_F32 ? 4 : 2; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// `p` must be the start of (or lie inside) a pinned host allocation from hipHostMalloc that
// holds `bytes` bytes from p on: device memory, pageable memory and allocations too small for
// the descriptor's shape are refused before a kernel could dereference them. The HIP runtime
// keeps the allocation map; a failed query leaves no error behind for a later launch check.
int check_host_buffer(const void* p, size_t bytes, const char* what) {
  hipPointerAttribute_t at;
  memset(&at, 0, sizeof(at));
  hipError_t e = hipPointerGetAttributes(&at, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(DKV_ERR_INVALID_ARG, "%s is not memory the HIP runtime knows (pageable host memory?): %s", what,
                hipGetErrorString(e));
  }
  if (at.type != hipMemoryTypeHost)
    return fail(DKV_ERR_INVALID_ARG, "%s is not pinned host memory (hipMemoryType %d)", what, (int)at.type);
  hipDeviceptr_t start = nullptr;
  size_t size = 0;
  if (hipPointerGetAttribute(&start, HIP_POINTER_ATTRIBUTE_RANGE_START_ADDR, const_cast<void*>(p)) == hipSuccess &&
      hipPointerGetAttribute(&size, HIP_POINTER_ATTRIBUTE_RANGE_SIZE, const_cast<void*>(p)) == hipSuccess &&
      size > 0) {
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(start), q = reinterpret_cast<uintptr_t>(p);
    if (q < s0 || q - s0 > size || size - (q - s0) < bytes)
      return fail(DKV_ERR_INVALID_ARG, "%s: the pinned allocation holds %zu bytes from this pointer, the cache needs %zu",
                  what, size - std::min<size_t>(size, q - s0), bytes);
  } else {
    (void)hipGetLastError();   // no range information: the memory type check above stands alone
  }
  return DKV_OK;
}

int check_cache(const dkv_cache* c) {
  if (!c) return fail(DKV_ERR_INVALID_ARG, "cache descriptor is null");
  if (c->reserved != kMagic || !c->k || !c->v)
    return fail(DKV_ERR_INVALID_ARG, "cache descriptor was not made by kv_alloc_host (or was freed)");
  if (c->dtype < DKV_F32 || c->dtype > DKV_BF16) return fail(DKV_ERR_UNSUPPORTED, "dtype %d", c->dtype);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(DKV_ERR_UNSUPPORTED, "head_dim %d (built: 64, 128)", c->head_dim);
  if (c->batch <= 0 || c->n_kv_heads <= 0 || c->capacity <= 0)
    return fail(DKV_ERR_INVALID_ARG, "cache sizes must be positive");
  return DKV_OK;
}

// The memory behind a cache descriptor, checked after every argument check and before the
// first enqueue: k and v are pinned host allocations of the descriptor's size.
int check_cache_memory(const dkv_cache* c) {
  const size_t bytes = (size_t)c->batch * c->n_kv_heads * c->capacity * c->head_dim * elem_size(c->dtype);
  int st = check_host_buffer(c->k, bytes, "cache k");
  if (st) return st;
  return check_host_buffer(c->v, bytes, "cache v");
}

// common checks of a layer call; T new tokens per sequence
int check_call(const dkv_cache* c, int32_t batch, int32_t T, int32_t D, const int32_t* past_len,
               std::initializer_list<const void*> dev_ptrs) {
  int st = check_cache(c);
  if (st) return st;
  if (batch != c->batch) return fail(DKV_ERR_INVALID_ARG, "batch %d != cache batch %d", batch, c->batch);
  if (batch > kMaxBatch) return fail(DKV_ERR_UNSUPPORTED, "batch %d > %d", batch, kMaxBatch);
  if (T < 0) return fail(DKV_ERR_INVALID_ARG, "T must be >= 0");
  if (D <= 0 || D % 64 != 0) return fail(DKV_ERR_INVALID_ARG, "D=%d must be a positive multiple of 64", D);
  if (!past_len) return fail(DKV_ERR_INVALID_ARG, "past_len is null");
  for (const void* p : dev_ptrs) {
    if (!p) return fail(DKV_ERR_INVALID_ARG, "a device pointer is null");
    if (!aligned16(p)) return fail(DKV_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  }
  for (int b = 0; b < batch; ++b) {
    if (past_len[b] < 0) return fail(DKV_ERR_CAPACITY, "past_len[%d]=%d < 0", b, past_len[b]);
    if ((int64_t)past_len[b] + T > c->capacity)
      return fail(DKV_ERR_CAPACITY, "past_len[%d]=%d + T=%d exceeds capacity %d", b, past_len[b], T, c->capacity);
  }
  // the kernels index the new rows of a call (and their 16-byte pieces) with 32-bit integers
  if ((int64_t)batch * c->n_kv_heads * T * c->head_dim >= ((int64_t)1 << 31))
    return fail(DKV_ERR_UNSUPPORTED, "batch*n_kv_heads*T*head_dim = %lld new K elements per call (limit 2^31)",
                (long long)batch * c->n_kv_heads * T * c->head_dim);
  return DKV_OK;
}

int check_heads(const dkv_cache* c, int32_t n_q_heads) {
  if (n_q_heads <= 0 || n_q_heads % c->n_kv_heads != 0)
    return fail(DKV_ERR_INVALID_ARG, "n_q_heads=%d must be a positive multiple of n_kv_heads=%d", n_q_heads,
                c->n_kv_heads);
  const int G = n_q_heads / c->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(DKV_ERR_UNSUPPORTED, "group size %d (built: 1,2,4,8)", G);
  return DKV_OK;
}

// ---- device facts, queried once per process (the first device a call runs on)
int g_cus = 0, g_xccs = 0;
std::once_flag g_dev_once;
void query_device() {
  std::call_once(g_dev_once, [] {
    int dev = 0;
    hipDeviceProp_t p;
    if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&p, dev) == hipSuccess) g_cus = p.multiProcessorCount;
    if (hipDeviceGetAttribute(&g_xccs, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess) g_xccs = 0;
    (void)hipGetLastError();
    if (g_cus <= 0) g_cus = 256;
  });
}
int cu_count() {
  query_device();
  return g_cus;
}
// The prefill places pairs on XCDs by workgroup index (workgroup i runs on XCD i % 8), which
// holds on the whole MI355X: 256 CUs in 8 XCDs. A partitioned device reports fewer; there the
// placement would only cost L2 reuse, and it is switched off.
bool xcd_placement() {
  query_device();
  return g_cus == 256 && g_xccs == 8;
}

// ---- kernel timing on the caller's stream (dkv_timing): HIP events around each phase's launches
enum TimedPhase { kPhaseProj = 0, kPhaseAttn = 1, kPhaseQproj = 2, kPhaseDecode = 3, kPhaseCombine = 4, kPhases = 5 };
struct TimedSpan {
  int phase, launches;
  hipEvent_t start, stop;
};
std::mutex g_timing_mu;
bool g_timing_on = false;
std::vector<TimedSpan> g_spans;

// Records an event on s if timing is on; the events of a span bracket `launches` launches of one
// phase. Event failures only lose the measurement.
struct PhaseTimer {
  hipStream_t s;
  int phase, launches = 0;
  hipEvent_t start = nullptr;
  PhaseTimer(hipStream_t s_, int phase_) : s(s_), phase(phase_) {
    std::lock_guard<std::mutex> lock(g_timing_mu);
    if (!g_timing_on) return;
    if (hipEventCreate(&start) != hipSuccess || hipEventRecord(start, s) != hipSuccess) {
      (void)hipGetLastError();
      start = nullptr;
    }
  }
  ~PhaseTimer() {
    if (start) (void)hipEventDestroy(start);   // a launch failed before done()
  }
  void done(int n) {
    if (!start) return;
    hipEvent_t stop = nullptr;
    if (hipEventCreate(&stop) != hipSuccess || hipEventRecord(stop, s) != hipSuccess) {
      (void)hipGetLastError();
      return;
    }
    std::lock_guard<std::mutex> lock(g_timing_mu);
    g_spans.push_back(TimedSpan{phase, n, start, stop});
    start = nullptr;
  }
};

// ---- decode plan: equal key chunks for every workgroup, whatever the lengths
struct DecodePlan {
  int chunk;
  int n_splits;
  int split_begin[kMaxBatch + 1];
};

// Splits per kv head so that the whole grid is ~2 workgroups per CU, or ~4 when that would
// leave each split fewer than kShortChunk keys: more, shorter host streams keep the link busier
// there (70B-shaped decode at 16384 past tokens: 2.58 -> 2.51 ms per step), while at long
// lengths they cost the extra partials (the same at 65536: 9.71 -> 9.75 ms; 8B-shaped at 32768:
// 19.24 ms either way).
constexpr int kDecodeWgPerCu = 2;
constexpr int64_t kShortChunk = 1024;

int decode_target_splits(const dkv_cache* c) {
  return std::max(1, kDecodeWgPerCu * cu_count() / c->n_kv_heads);
}

void plan_decode(const dkv_cache* c, const int32_t* past_len, int32_t batch, bool paged, DecodePlan& p) {
  int64_t keys = 0;
  for (int b = 0; b < batch; ++b) keys += past_len[b] + 1;
  int target = decode_target_splits(c);
  const int unit = decode_slots(c->dtype, c->head_dim);  // keys one loop iteration consumes
  if ((keys + target - 1) / target < kShortChunk) target *= 2;
  int64_t chunk = (keys + target - 1) / target;
  chunk = std::max<int64_t>(chunk, 2 * unit);
  chunk = round_up(chunk, unit);
  // a paged split stages its page ids in LDS: at most kPagedDecodeChunk keys (a multiple of unit)
  if (paged) chunk = std::min<int64_t>(chunk, kPagedDecodeChunk);
  p.chunk = (int)chunk;
  p.n_splits = 0;
  for (int b = 0; b < batch; ++b) {
    p.split_begin[b] = p.n_splits;
    p.n_splits += (int)((past_len[b] + 1 + chunk - 1) / chunk);
  }
  p.split_begin[batch] = p.n_splits;
}

// decode workspace: the split partials, then the projected queries [B][Hq*d] fp32
size_t decode_part_bytes(const dkv_cache* c, int32_t batch, int32_t n_q_heads, bool paged) {
  // sum_b ceil((L_b+1)/chunk) <= keys/chunk + batch <= target + batch, target at most twice
  // decode_target_splits; a capped paged chunk adds at most batch * (capacity / kPagedDecodeChunk + 1)
  size_t splits = 2 * (size_t)decode_target_splits(c) + batch + 1;
  if (paged) splits += (size_t)batch * ((size_t)c->capacity / kPagedDecodeChunk + 1);
  return round_up(splits * n_q_heads * (c->head_dim + 2) * sizeof(float), 256);
}

size_t decode_ws_bytes(const dkv_cache* c, int32_t batch, int32_t n_q_heads, bool paged) {
  return decode_part_bytes(c, batch, n_q_heads, paged) +
         round_up((size_t)batch * n_q_heads * c->head_dim * sizeof(float), 256);
}

// Queries are projected once per step by a pre-pass when the decode workgroups projecting their
// own would read Wq again by more than kQpassMinBytes: every split beyond a sequence's first
// re-reads its group's G*d rows of D weights, for each kv head (a 70B-shaped layer re-reads ~8 GiB
// per step, mostly beyond L2). Below that the extra launch costs more than the reads.
// DIRECTKV_DECODE_QPASS=0/1 forces either (both give bitwise the same queries).
constexpr size_t kQpassMinBytes = 256ull << 20;

bool decode_uses_qpass(const dkv_cache* c, const DecodePlan& p, int32_t batch, int32_t n_q_heads, int32_t D) {
  if (const char* env = getenv("DIRECTKV_DECODE_QPASS")) {
    if (env[0] == '0') return false;
    if (env[0] == '1') return true;
  }
  const size_t wq_bytes = (size_t)n_q_heads * c->head_dim * D * elem_size(c->dtype);   // all kv heads' slices
  return (size_t)(p.n_splits - batch) * wq_bytes > kQpassMinBytes;
}

// ---- prefill workspace layout
// Key splits per pair of a one-query-tile prefill at most: enough for two workgroups per CU of a
// 256-CU device, and at most kMaxKeySplits (one split per pair from 512 pairs up: no split).
int key_split_cap(int pairs) { return std::min(kMaxKeySplits, std::max(1, (512 + pairs - 1) / std::max(1, pairs))); }

struct PrefillWs {
  size_t q, k_new, v_new, state, nstate, rope, split, chunk, total;
  int n_chunks;   // past super-chunk states the two-launch prefill has room for (0: not used)
};

int chunked_max(const dkv_cache* c, int32_t batch, int32_t T, int32_t n_q_heads, bool paged);

PrefillWs prefill_layout(const dkv_cache* c, int32_t batch, int32_t T, int32_t n_q_heads, bool paged = false) {
  PrefillWs w;
  const size_t e = elem_size(c->dtype), d = c->head_dim;
  const int G = n_q_heads / std::max(1, c->n_kv_heads);
  w.q = 0;
  w.k_new = w.q + round_up((size_t)batch * T * n_q_heads * d * e, 256);
  w.v_new = w.k_new + round_up((size_t)batch * c->n_kv_heads * T * d * e, 256);
  w.state = w.v_new + round_up((size_t)batch * c->n_kv_heads * T * d * e, 256);
  const size_t sb = round_up(attn_state_bytes(c->head_dim, batch, c->n_kv_heads, T, std::max(1, G)), 256);
  w.nstate = w.state + sb;
  w.rope = w.nstate + sb;   // rotary (cos, sin) table of the call's rows (attn_prefill_rope)
  w.split = w.rope + round_up((size_t)batch * T * (d / 2) * 2 * sizeof(float), 256);
  // one query tile per pair: the running states of the key splits (key_split_cap per pair)
  const bool one_tile = (long long)T * std::max(1, G) <= attn_rows_per_tile();
  const int cap = key_split_cap(batch * std::max(1, c->n_kv_heads));
  w.chunk = w.split + (one_tile && cap > 1 ? (size_t)cap * sb : 0);
  // the two-launch prefill: one running state per past super-chunk
  w.n_chunks = chunked_max(c, batch, T, n_q_heads, paged);
  w.total = w.chunk + (size_t)w.n_chunks * sb;
  return w;
}

// keys per super-chunk: the host KV of every (sequence, kv head) pair an XCD serves
// during one launch must fit about half of that XCD's 4 MB L2 (a quarter for a paged cache:
// its super-chunk is scattered over the pool in 4 KB (page, head) blocks, which at half the
// L2 conflict-miss and are fetched again, 1.28x the host bytes against 1.02x at a quarter).
// With more than kLongLaunchTiles query tiles per pair a launch runs many rounds of query tiles,
// whose running-state streams pass through L2 between the uses of the super-chunk: there it
// takes seven sixteenths of L2 (70B-shaped prefill, 512 tiles per pair, with fetcher and own-key
// items: 3072, 3328 and 3584 keys per super-chunk read 1.014x, 1.021x and 1.028x the algorithmic
// host bytes in 67.0, 66.1 and 66.1 ms; the 8B-shaped prefill, 128 tiles per pair, reads 1.005x
// at a half).
constexpr int kLongLaunchTiles = 256;

int superchunk_keys(const dkv_cache* c, int32_t pairs, bool paged, int32_t q_tiles) {
  // a paged launch stages the page ids of its keys in LDS: at most kPagedSuperchunk keys
  const size_t limit = paged ? kPagedSuperchunk : 1 << 20;
  // tuning override (keys, multiple of 64)
  if (const char* env = getenv("DIRECTKV_PREFILL_CHUNK")) {
    const long v = strtol(env, nullptr, 10);
    if (v >= 64) return (int)std::min<size_t>(v / 64 * 64, limit);
  }
  const int per_xcd = std::max(1, (pairs + 7) / 8);
  const size_t row_bytes = 2 * (size_t)c->head_dim * elem_size(c->dtype);  // K and V
  const size_t budget = paged ? (1u << 20) : q_tiles > kLongLaunchTiles ? (7u << 18) : (2u << 20);
  size_t keys = budget / ((size_t)per_xcd * row_bytes);
  keys = std::max<size_t>(64, keys / 64 * 64);
  return (int)std::min<size_t>(keys, limit);
}

// Past-key items per pair dispatched ahead of a launch's own-key items: they bring the launch's
// super-chunk over the host link into L2 while the own-key items compute, and compute at the
// link's pace themselves (DIRECTKV_PREFILL_FETCHERS overrides it for tuning). 8B-shaped prefill,
// one machine: 0, 1, 2, 4, 8 fetchers per pair (per XCD) 5.19, 5.51, 5.50, 5.13, 5.10 ms; the
// 70B-shaped prefill, link-hidden either way, 66.8-67.2 ms for all.
int prefill_fetchers() {
  if (const char* env = getenv("DIRECTKV_PREFILL_FETCHERS")) {
    const long v = strtol(env, nullptr, 10);
    if (v >= 0 && v <= 64) return (int)v;
  }
  return 8;
}

// The two-launch prefill (attn_kernel, chunked mode): one launch runs the past-key items of every
// super-chunk, each leaving its own state, with the next super-chunk's fetchers dispatched while the
// current one's items compute, so the link works beside the MFMA pipes instead of ahead of them;
// a second launch runs the heavier own-key items, which fold every state in as they finalise.
// Two super-chunks then share an XCD's L2, three eighths of it each (a quarter each for a paged
// cache). It is used where every super-chunk's state fits kChunkStateCap of workspace, else the
// launch-per-super-chunk path runs (DIRECTKV_PREFILL_CHUNKED=0 forces that path, and the workspace
// query then leaves the states out: the mode trades up to kChunkStateCap of workspace, reused by
// every call on a stream, for the overlap).
constexpr size_t kChunkStateCap = (size_t)2 << 30;

int chunk_group(int P) { return P % 8 == 0 ? 8 : P; }

int chunked_keys(const dkv_cache* c, int32_t group, bool paged) {
  // a paged super-chunk keeps the launch-per-super-chunk path's 1 MiB (its pages scatter over the
  // pool, and an item stages at most kPagedSuperchunk keys' page ids)
  const size_t limit = paged ? kPagedSuperchunk : 1 << 20;
  if (const char* env = getenv("DIRECTKV_PREFILL_CHUNK")) {
    const long v = strtol(env, nullptr, 10);
    if (v >= 64) return (int)std::min<size_t>(v / 64 * 64, limit);
  }
  const int per_xcd = std::max(1, (group + 7) / 8);
  const size_t row_bytes = 2 * (size_t)c->head_dim * elem_size(c->dtype);
  const size_t keys = (size_t)(paged ? (1u << 20) : (3u << 19)) / ((size_t)per_xcd * row_bytes);
  return (int)std::min<size_t>(std::max<size_t>(64, keys / 64 * 64), limit);
}

bool chunked_enabled() {
  const char* env = getenv("DIRECTKV_PREFILL_CHUNKED");
  return !(env && env[0] == '0');
}

// super-chunk states the workspace holds for the two-launch prefill: enough for any past length
// up to capacity - T, or 0 where the mode is not used (a paged cache's view has capacity
// max_pages x 16)
int chunked_max(const dkv_cache* c, int32_t batch, int32_t T, int32_t n_q_heads, bool paged) {
  if (c->n_kv_heads <= 0 || !chunked_enabled()) return 0;
  const int G = std::max(1, n_q_heads / c->n_kv_heads);
  if ((long long)T * G <= attn_rows_per_tile()) return 0;   // one query tile per pair: key splits
  const long long max_past = (long long)c->capacity - T;
  const int ck = chunked_keys(c, chunk_group(batch * c->n_kv_heads), paged);
  const long long S = (max_past + ck - 1) / ck;
  const size_t sb = round_up(attn_state_bytes(c->head_dim, batch, c->n_kv_heads, T, G), 256);
  if (S < 2 || (size_t)S * sb > kChunkStateCap) return 0;
  return (int)S;
}

// own-key items of the two-launch prefill's first launch: the lightest query tiles, about a third
// of the own-key work (DIRECTKV_PREFILL_OWN=<percent> overrides it for tuning)
int chunked_own_percent() {
  if (const char* env = getenv("DIRECTKV_PREFILL_OWN")) {
    const long v = strtol(env, nullptr, 10);
    if (v >= 0 && v <= 100) return (int)v;
  }
  return 33;
}

// chunk j's items per pair dispatched ahead of chunk j+1's fetchers: five sixths of them, so the
// next super-chunk crosses the link during the last sixth of this one's items and the fetchers'
// own compute. Earlier, the two super-chunks and the running-state streams overflow L2: 8B-shaped
// prefill (120 such items per pair) with 40, 100 and 120 read 1.10-1.15x, 1.014-1.020x and
// 1.01-1.04x the algorithmic host bytes over two runs, in 4.62-4.76 ms for all from 60 on
// (DIRECTKV_PREFILL_INSERT=<items> overrides it for tuning).
int chunked_insert(int items) {
  if (const char* env = getenv("DIRECTKV_PREFILL_INSERT")) {
    const long v = strtol(env, nullptr, 10);
    if (v >= 0) return (int)std::min<long>(v, items);
  }
  return items * 5 / 6;
}

// block table of a paged cache, already copied into device memory (null: contiguous cache)
struct Paging {
  const int32_t* table = nullptr;
  int32_t max_pages = 0;
};

ProjArgs make_proj(const dkv_cache* c, const void* x, const void* wq, const void* wk, const void* wv,
                   const int32_t* past_len, int32_t batch, int32_t T, int32_t D, int32_t n_q_heads,
                   void* q_out, void* k_dev, void* v_dev) {
  ProjArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x;
  a.w[0] = wq;
  a.w[1] = wk;
  a.w[2] = wv;
  a.n_seg[0] = wq ? n_q_heads * c->head_dim : 0;
  a.n_seg[1] = c->n_kv_heads * c->head_dim;
  a.n_seg[2] = c->n_kv_heads * c->head_dim;
  a.M = batch * T;
  a.D = D;
  a.T = T;
  a.B = batch;
  a.d = c->head_dim;
  a.Hkv = c->n_kv_heads;
  a.cap = c->capacity;
  a.q_out = q_out;
  a.kc = c->k;
  a.vc = c->v;
  a.k_dev = k_dev;
  a.v_dev = v_dev;
  for (int b = 0; b < batch; ++b) a.past_len[b] = past_len[b];
  return a;
}

}  // namespace

namespace {

// ---- the layer calls, on a contiguous cache or (with a device block table) on a page pool
// described by a dkv_cache view; arguments are checked by the caller through check_call

int run_append(const dkv_cache* c, const Paging& pg, const void* x, const void* wk, const void* wv,
               const int32_t* past_len, int32_t batch, int32_t T, int32_t D, hipStream_t s) {
  proj_fn f = find_proj(c->dtype, c->head_dim);
  if (!f) return fail(DKV_ERR_UNSUPPORTED, "no projection instance for dtype %d head_dim %d", c->dtype, c->head_dim);
  ProjArgs a = make_proj(c, x, nullptr, wk, wv, past_len, batch, T, D, 0, nullptr, nullptr, nullptr);
  a.host_out = 1;
  a.table = pg.table;
  a.max_pages = pg.max_pages;
  PhaseTimer tp(s, kPhaseProj);
  hipError_t e = f(a, s);
  if (e != hipSuccess) return hip_fail(e, "projection launch");
  tp.done(1);
  return DKV_OK;
}

int run_decode(const dkv_cache* c, const Paging& pg, const void* x, const void* wq, const void* wk,
               const void* wv, const int32_t* past_len, int32_t batch, int32_t D, int32_t n_q_heads, void* out,
               void* ws, size_t ws_bytes, hipStream_t s, double rope = 0.0) {
  const bool paged = pg.table != nullptr;
  const size_t need = decode_ws_bytes(c, batch, n_q_heads, paged);
  if (!ws || ws_bytes < need || !aligned16(ws))
    return fail(DKV_ERR_WORKSPACE, "workspace %zu bytes, need %zu (16-byte aligned)", ws_bytes, need);
  const int G = n_q_heads / c->n_kv_heads;
  decode_fn fd = find_decode(c->dtype, c->head_dim, G, paged);
  combine_fn fc = find_combine(c->dtype, c->head_dim);
  qproj_fn fq = find_qproj(c->dtype, c->head_dim);
  if (!fd || !fc || !fq)
    return fail(DKV_ERR_UNSUPPORTED, "no decode instance for dtype %d d %d G %d", c->dtype, c->head_dim, G);

  DecodePlan p;
  plan_decode(c, past_len, batch, paged, p);
  DecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x;
  a.wq = wq;
  a.wk = wk;
  a.wv = wv;
  a.kc = c->k;
  a.vc = c->v;
  a.part = reinterpret_cast<float*>(ws);
  a.out = out;
  // one split per sequence: the decode kernel writes the output itself and the combine launch
  // is skipped (DIRECTKV_DECODE_COMBINE=1 keeps the combine, which gives bitwise the same output)
  const char* force_combine = getenv("DIRECTKV_DECODE_COMBINE");
  a.direct = p.n_splits == batch && !(force_combine && force_combine[0] == '1');
  a.qf = decode_uses_qpass(c, p, batch, n_q_heads, D)
             ? reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + decode_part_bytes(c, batch, n_q_heads, paged))
             : nullptr;
  a.B = batch;
  a.D = D;
  a.Hq = n_q_heads;
  a.Hkv = c->n_kv_heads;
  a.cap = c->capacity;
  a.n_splits = p.n_splits;
  a.chunk = p.chunk;
  a.table = pg.table;
  a.max_pages = pg.max_pages;
  for (int b = 0; b < batch; ++b) a.past_len[b] = past_len[b];
  for (int b = 0; b <= batch; ++b) a.split_begin[b] = p.split_begin[b];
  a.rope_theta = rope;

  CombineArgs ca;
  memset(&ca, 0, sizeof(ca));
  ca.part = a.part;
  ca.out = out;
  ca.B = batch;
  ca.Hq = n_q_heads;
  ca.n_splits = p.n_splits;
  for (int b = 0; b <= batch; ++b) ca.split_begin[b] = p.split_begin[b];

  hipError_t e;
  if (a.qf) {
    PhaseTimer tq(s, kPhaseQproj);
    if ((e = fq(a, s)) != hipSuccess) return hip_fail(e, "query projection launch");
    tq.done(1);
  }
  PhaseTimer td(s, kPhaseDecode);
  e = fd(a, s);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  td.done(1);
  if (!a.direct) {
    PhaseTimer tc(s, kPhaseCombine);
    if ((e = fc(ca, s)) != hipSuccess) return hip_fail(e, "combine launch");
    tc.done(1);
  }
  return DKV_OK;
}

int run_prefill(const dkv_cache* c, const Paging& pg, const void* x, const void* wq, const void* wk,
                const void* wv, const int32_t* past_len, int32_t batch, int32_t T, int32_t D, int32_t n_q_heads,
                void* out, void* ws, size_t ws_bytes, hipStream_t s, int32_t variant, double rope = 0.0) {
  const bool paged = pg.table != nullptr;
  const PrefillWs lay = prefill_layout(c, batch, T, n_q_heads, paged);
  if (!ws || ws_bytes < lay.total || !aligned16(ws))
    return fail(DKV_ERR_WORKSPACE, "workspace %zu bytes, need %zu (16-byte aligned)", ws_bytes, lay.total);
  const int G = n_q_heads / c->n_kv_heads;
  proj_fn fp = find_proj(c->dtype, c->head_dim);
  attn_fn fa = find_attn(c->dtype, c->head_dim, G, paged);
  if (!fp || !fa) return fail(DKV_ERR_UNSUPPORTED, "no prefill instance for dtype %d d %d G %d", c->dtype, c->head_dim, G);

  char* w = reinterpret_cast<char*>(ws);
  void* q = w + lay.q;
  void* kn = w + lay.k_new;
  void* vn = w + lay.v_new;
  float* state = reinterpret_cast<float*>(w + lay.state);
  float* nstate = reinterpret_cast<float*>(w + lay.nstate);

  const bool separate = variant == DKV_PREFILL_SEPARATE;
  const bool fused = variant == DKV_PREFILL_FUSED;
  const int rows = attn_rows_per_tile();
  const int Q = (T * G + rows - 1) / rows;
  const int P = batch * c->n_kv_heads;
  // Key splits: with one query tile per pair no key is shared between query tiles, so instead of
  // super-chunk launches each pair's keys are split over enough workgroups to fill the chip (two
  // per CU), and a second launch merges the splits' states.
  int n_splits = 0;
  if (fused && Q == 1) {
    int max_keys = 0;
    for (int b = 0; b < batch; ++b) max_keys = std::max(max_keys, past_len[b] + T);
    const int kt = attn_key_tile(c->dtype, c->head_dim);
    const int tiles = (max_keys + kt - 1) / kt;
    const int cap = key_split_cap(P);   // what the workspace holds
    n_splits = std::min({cap, tiles, std::max(1, (2 * cu_count() + P - 1) / P)});
    // a paged launch stages its keys' page ids in LDS: a split holds at most kPagedSuperchunk keys
    if (paged) n_splits = std::max(n_splits, (tiles + kPagedSuperchunk / kt - 1) / (kPagedSuperchunk / kt));
    if (n_splits <= 1 || n_splits > cap) n_splits = 0;
  }
  ProjArgs pa = make_proj(c, x, wq, wk, wv, past_len, batch, T, D, n_q_heads, q, separate ? nullptr : kn,
                          separate ? nullptr : vn);
  // The projection leaves the new rows in device memory, where attention reads them instead of
  // fetching them back over the link; in the fused path the own-key items write their host copy
  // (the storer role, beside their compute), the baselines write it from the projection epilogue.
  // A step of few rows is the exception: its few own-key items would each push a large share of
  // the rows over the link, so the projection's many small workgroups write them instead.
  // With key splits, storer workgroups of the split launch write them while the splits compute.
  const bool few_rows = (long long)batch * T <= kProjSmallRows;
  pa.host_out = !fused || (few_rows && n_splits == 0);
  pa.table = pg.table;
  pa.max_pages = pg.max_pages;
  if (rope > 0.0) {
    float2* cs = reinterpret_cast<float2*>(w + lay.rope);
    hipError_t re = launch_rope_table(past_len, batch, T, c->head_dim, rope, cs, s);
    if (re != hipSuccess) return hip_fail(re, "rotary table launch");
    pa.rope_cs = cs;
  }
  PhaseTimer tp(s, kPhaseProj);
  hipError_t e = fp(pa, s);
  if (e != hipSuccess) return hip_fail(e, "projection launch");
  tp.done(1);

  AttnArgs aa;
  memset(&aa, 0, sizeof(aa));
  aa.q = q;
  aa.kc = c->k;
  aa.vc = c->v;
  aa.k_new = kn;
  aa.v_new = vn;
  aa.state = state;
  aa.nstate = nstate;
  aa.out = out;
  aa.B = batch;
  aa.T = T;
  aa.Hq = n_q_heads;
  aa.Hkv = c->n_kv_heads;
  aa.cap = c->capacity;
  aa.table = pg.table;
  aa.max_pages = pg.max_pages;
  aa.q_tiles = Q;
  aa.xcd_group = variant != DKV_PREFILL_NAIVE && P >= 8 && xcd_placement();
  aa.new_from_host = separate;
  aa.fetchers = prefill_fetchers();
  aa.store_new = fused && !few_rows && n_splits == 0;
  for (int b = 0; b < batch; ++b) aa.past_len[b] = past_len[b];
  // With a multiple of 8 pairs, the pairs go in groups of 8, one pair per XCD: each XCD's L2
  // then holds one pair's super-chunk, twice as many keys as when two pairs share it, which
  // halves the launches every query tile makes and the running-state traffic they cost.
  const int group = aa.xcd_group && P % 8 == 0 ? 8 : P;
  PhaseTimer ta(s, kPhaseAttn);
  int n_attn = 0;
  auto launch = [&]() -> int {
    const hipError_t le = fa(aa, s);
    ++n_attn;
    return le == hipSuccess ? DKV_OK : hip_fail(le, "attention launch");
  };
  if (n_splits > 0) {
    aa.n_splits = n_splits;
    aa.split_stride = (int64_t)(attn_state_bytes(c->head_dim, batch, c->n_kv_heads, T, G) / sizeof(float));
    aa.state = reinterpret_cast<float*>(w + lay.split);
    aa.pair0 = 0;
    aa.pairs = P;
    aa.xcd_group = 0;
    aa.split_combine = 0;
    // storers: about 16 KB of new rows each (4 KB to 16 KB measure the same), at most one per CU
    const size_t new_bytes = (size_t)2 * P * T * c->head_dim * elem_size(c->dtype);
    aa.split_storers = (int)std::min<size_t>((size_t)cu_count(), std::max<size_t>(1, (new_bytes + 16383) / 16384));
    aa.store_new = 1;
    int st = launch();
    if (st) return st;
    aa.split_combine = 1;
    if ((st = launch())) return st;
    ta.done(n_attn);
    return DKV_OK;
  }
  for (int pair0 = 0; pair0 < P; pair0 += group) {
    aa.pair0 = pair0;
    aa.pairs = group;
    const int b0 = pair0 / c->n_kv_heads, b1 = (pair0 + group - 1) / c->n_kv_heads;   // sequences served
    int max_keys = 0, max_past = 0;
    for (int b = b0; b <= b1; ++b) {
      max_keys = std::max(max_keys, past_len[b] + T);
      max_past = std::max(max_past, past_len[b]);
    }
    // the naive baseline sweeps every key in one launch: no super-chunks, no XCD placement
    const int sk = variant == DKV_PREFILL_NAIVE ? std::max(max_keys, 1) : superchunk_keys(c, group, paged, Q);
    if (!fused) {
      // The baselines: launches over key ranges holding every key, past and new, each carrying the
      // running state to the next (the separate-kernels baseline reads this step's rows back from
      // the host cache, the naive one sweeps every key in one launch).
      std::vector<std::pair<int, int>> ranges;
      for (int k0 = 0; k0 < max_keys; k0 += sk) ranges.emplace_back(k0, std::min(k0 + sk, max_keys));
      aa.past_items = 1;
      aa.clip_past = 0;
      aa.dev_q0 = aa.dev_q1 = 0;
      aa.merge_new = aa.dev_final = 0;
      for (size_t i = 0; i < ranges.size(); ++i) {
        aa.kc0 = ranges[i].first;
        aa.kc1 = ranges[i].second;
        aa.first = i == 0;
        aa.last = i + 1 == ranges.size();
        int st = launch();
        if (st) return st;
      }
      continue;
    }
    // The fused path. Past keys [0, past_len[b]) go in launches over super-chunks of equal size (a
    // multiple of 64 keys, at most sk), the last ending at the longest past length, so no launch
    // sweeps a short remainder. This step's own keys go as own-key items, one per query tile, each
    // over all own keys its rows see, read from their device copies; they are spread over the
    // past-key launches but the last (whose items fold their state in when they finalise), by
    // equal shares of work, and each runs while its launch's fetcher items bring the super-chunk
    // over the link. With one past-key launch they run in a launch of their own before it; with no
    // past keys they are the only items and finalise the output themselves.
    const int n_host = (max_past + sk - 1) / sk;
    const int skp = n_host > 0 ? std::min<int>(sk, (int)round_up((max_past + n_host - 1) / n_host, 64)) : sk;
    std::vector<std::pair<int, int>> ranges;
    for (int k0 = 0; k0 < max_past; k0 += skp) ranges.emplace_back(k0, std::min(k0 + skp, max_past));
    const int S = (int)ranges.size();
    aa.clip_past = 1;
    // own-key work of query tile q: the rows' visible own keys, sum over rows of (row / G + 1)
    std::vector<double> cum(Q + 1, 0.0);
    for (int qt = 0; qt < Q; ++qt) {
      const long long r0 = (long long)qt * rows, r1 = std::min<long long>((long long)T * G, r0 + rows) - 1;
      double wq = 0.0;
      for (long long t = r0 / G; t <= r1 / G; ++t)
        wq += (double)(std::min<long long>(r1, (t + 1) * G - 1) - std::max<long long>(r0, t * G) + 1) * (double)(t + 1);
      cum[qt + 1] = cum[qt] + wq;
    }
    {
      // the two-launch prefill, where its super-chunks' states fit the workspace
      const int ck = chunked_keys(c, group, paged);
      const int nc = max_past > 0 ? (max_past + ck - 1) / ck : 0;
      const int ckp = nc > 0 ? std::min<int>(ck, (int)round_up((max_past + nc - 1) / nc, 64)) : ck;
      const int SC = nc > 0 ? (max_past + ckp - 1) / ckp : 0;
      if (SC >= 2 && SC <= lay.n_chunks && chunked_enabled()) {
        int qa = 0;
        const double goal = cum[Q] * chunked_own_percent() / 100.0;
        while (qa < Q && cum[qa + 1] <= goal + 1e-9) ++qa;
        const int F = std::min(aa.fetchers, Q);
        aa.chunked = 1;
        aa.n_splits = SC;
        aa.split_stride = (int64_t)(round_up(attn_state_bytes(c->head_dim, batch, c->n_kv_heads, T, G), 256) /
                                    sizeof(float));
        aa.chunk_keys = ckp;
        aa.chunk_insert = chunked_insert(Q - F);
        aa.n_own0 = qa;
        aa.state = reinterpret_cast<float*>(w + lay.chunk);
        int st = launch();
        if (st) return st;
        aa.chunked = 2;
        if ((st = launch())) return st;
        aa.chunked = 0;
        aa.n_splits = 0;
        aa.state = state;
        continue;
      }
    }
    if (S <= 1) {
      aa.past_items = 0;
      aa.dev_q0 = 0;
      aa.dev_q1 = Q;
      aa.dev_final = S == 0;
      aa.merge_new = 0;
      aa.first = aa.last = 0;
      int st = launch();
      if (st || S == 0) {
        if (st) return st;
        continue;
      }
      aa.past_items = 1;
      aa.dev_q0 = aa.dev_q1 = 0;
      aa.dev_final = 0;
      aa.kc0 = ranges[0].first;
      aa.kc1 = ranges[0].second;
      aa.first = aa.last = aa.merge_new = 1;
      if ((st = launch())) return st;
      continue;
    }
    int dq = 0;
    for (int i = 0; i < S; ++i) {
      aa.kc0 = ranges[i].first;
      aa.kc1 = ranges[i].second;
      aa.first = i == 0;
      aa.last = aa.merge_new = i == S - 1;
      aa.past_items = 1;
      aa.dev_final = 0;
      int dq1 = dq;
      if (i < S - 1) {
        const double goal = cum[Q] * (double)(i + 1) / (double)(S - 1);
        while (dq1 < Q && (i == S - 2 || cum[dq1 + 1] <= goal + 1e-9)) ++dq1;
      }
      aa.dev_q0 = dq;
      aa.dev_q1 = dq1;
      dq = dq1;
      int st = launch();
      if (st) return st;
    }
  }
  ta.done(n_attn);
  return DKV_OK;
}

// ---- the staging baseline: the past rows are copied into device memory before the kernels
// run (the swap-based offloading the pages compare against), and the new rows copied back

size_t staging_bytes(const dkv_cache* c) {
  return round_up((size_t)c->batch * c->n_kv_heads * c->capacity * c->head_dim * elem_size(c->dtype), 256);
}

// copy token rows [r0[b], r0[b] + n) of every (b, g) between two [B][Hkv][cap][d] caches
hipError_t copy_rows(void* dst, const void* src, const dkv_cache* c, const int32_t* r0, int32_t n_new,
                     bool past, hipMemcpyKind kind, hipStream_t s) {
  const size_t row = (size_t)c->head_dim * elem_size(c->dtype), pitch = (size_t)c->capacity * row;
  for (int b = 0; b < c->batch; ++b) {
    const size_t first = past ? 0 : (size_t)r0[b];
    const size_t n = past ? (size_t)r0[b] : (size_t)n_new;
    if (n == 0) continue;
    const size_t off = (size_t)b * c->n_kv_heads * pitch + first * row;
    hipError_t e = hipMemcpy2DAsync(reinterpret_cast<char*>(dst) + off, pitch,
                                    reinterpret_cast<const char*>(src) + off, pitch, n * row, c->n_kv_heads, kind, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// a device copy of cache c at the front of the workspace: [K staging][V staging]
dkv_cache staged_view(const dkv_cache* c, void* ws) {
  dkv_cache d = *c;
  d.k = ws;
  d.v = reinterpret_cast<char*>(ws) + staging_bytes(c);
  return d;
}

int stage_in(const dkv_cache* c, const dkv_cache& dev, const int32_t* past_len, hipStream_t s) {
  hipError_t e = copy_rows(dev.k, c->k, c, past_len, 0, true, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = copy_rows(dev.v, c->v, c, past_len, 0, true, hipMemcpyHostToDevice, s);
  return e == hipSuccess ? DKV_OK : hip_fail(e, "staging copy to device");
}

int stage_out(const dkv_cache* c, const dkv_cache& dev, const int32_t* past_len, int32_t T, hipStream_t s) {
  hipError_t e = copy_rows(c->k, dev.k, c, past_len, T, false, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = copy_rows(c->v, dev.v, c, past_len, T, false, hipMemcpyDeviceToHost, s);
  return e == hipSuccess ? DKV_OK : hip_fail(e, "new rows back to the host cache");
}

// ---- paged caches
constexpr int32_t kPagedMagic = 0x444B5650;  // marks descriptors made by kv_paged_alloc_host

int check_paged(const dkv_paged_cache* pc) {
  if (!pc) return fail(DKV_ERR_INVALID_ARG, "paged cache descriptor is null");
  if (pc->reserved != kPagedMagic || !pc->k || !pc->v)
    return fail(DKV_ERR_INVALID_ARG, "paged cache descriptor was not made by kv_paged_alloc_host (or was freed)");
  if (pc->dtype < DKV_F32 || pc->dtype > DKV_BF16) return fail(DKV_ERR_UNSUPPORTED, "dtype %d", pc->dtype);
  if (pc->head_dim != 64 && pc->head_dim != 128)
    return fail(DKV_ERR_UNSUPPORTED, "head_dim %d (built: 64, 128)", pc->head_dim);
  if (pc->n_pages <= 0 || pc->n_kv_heads <= 0) return fail(DKV_ERR_INVALID_ARG, "paged cache sizes must be positive");
  return DKV_OK;
}

// the page pools are pinned host allocations of n_pages pages (checked before the first enqueue)
int check_paged_memory(const dkv_paged_cache* pc) {
  const size_t bytes = (size_t)pc->n_pages * pc->n_kv_heads * kPageTokens * pc->head_dim * elem_size(pc->dtype);
  int st = check_host_buffer(pc->k, bytes, "page pool k");
  if (st) return st;
  return check_host_buffer(pc->v, bytes, "page pool v");
}

// a dkv_cache view of a page pool for one call: capacity is what the table can address
dkv_cache paged_view(const dkv_paged_cache* pc, int32_t batch, int32_t max_pages) {
  dkv_cache c;
  memset(&c, 0, sizeof(c));
  c.k = pc->k;
  c.v = pc->v;
  c.batch = batch;
  c.n_kv_heads = pc->n_kv_heads;
  c.head_dim = pc->head_dim;
  c.capacity = (int32_t)std::min<int64_t>((int64_t)max_pages * kPageTokens, INT32_MAX / 2);
  c.dtype = pc->dtype;
  c.reserved = kMagic;
  return c;
}

size_t table_bytes(int32_t batch, int32_t max_pages) { return round_up((size_t)batch * max_pages * 4, 256); }

// Checks the block table on the host before any kernel can follow it: every page that holds
// a row of [0, past_len[b] + T) is in [0, n_pages), and every page this call writes (rows
// [past_len[b], past_len[b] + T)) is mapped exactly once in the used part of the table.
int check_table(const dkv_paged_cache* pc, const int32_t* table, int32_t max_pages, const int32_t* past_len,
                int32_t batch, int32_t T) {
  if (!table) return fail(DKV_ERR_INVALID_ARG, "block_table is null");
  if (max_pages <= 0) return fail(DKV_ERR_INVALID_ARG, "max_pages must be positive");
  if (batch <= 0) return fail(DKV_ERR_INVALID_ARG, "batch must be positive");
  if (batch > kMaxBatch) return fail(DKV_ERR_UNSUPPORTED, "batch %d > %d", batch, kMaxBatch);
  if (!past_len) return fail(DKV_ERR_INVALID_ARG, "past_len is null");
  if (T < 0) return fail(DKV_ERR_INVALID_ARG, "T must be >= 0");
  for (int b = 0; b < batch; ++b) {
    if (past_len[b] < 0) return fail(DKV_ERR_CAPACITY, "past_len[%d]=%d < 0", b, past_len[b]);
    if ((int64_t)past_len[b] + T > (int64_t)max_pages * kPageTokens)
      return fail(DKV_ERR_CAPACITY, "past_len[%d]=%d + T=%d exceeds max_pages*%d", b, past_len[b], T, kPageTokens);
  }
  thread_local std::vector<int32_t> refs;
  refs.assign((size_t)pc->n_pages, 0);
  for (int b = 0; b < batch; ++b) {
    const int used = (past_len[b] + T + kPageTokens - 1) / kPageTokens;
    for (int p = 0; p < used; ++p) {
      const int32_t id = table[(size_t)b * max_pages + p];
      if (id < 0 || id >= pc->n_pages)
        return fail(DKV_ERR_INVALID_ARG, "block_table[%d][%d]=%d is outside [0, %d)", b, p, id, pc->n_pages);
      ++refs[(size_t)id];
    }
  }
  if (T > 0) {
    for (int b = 0; b < batch; ++b) {
      for (int p = past_len[b] / kPageTokens; p <= (past_len[b] + T - 1) / kPageTokens; ++p) {
        const int32_t id = table[(size_t)b * max_pages + p];
        if (refs[(size_t)id] != 1)
          return fail(DKV_ERR_INVALID_ARG, "page %d written by sequence %d (block_table[%d][%d]) is mapped %d times",
                      id, b, b, p, refs[(size_t)id]);
      }
    }
  }
  return DKV_OK;
}

// copies the checked table to the front of the workspace; returns the device table
Paging stage_table(const int32_t* table, int32_t batch, int32_t max_pages, void* ws, hipStream_t s, hipError_t& e) {
  Paging pg;
  pg.table = reinterpret_cast<const int32_t*>(ws);
  pg.max_pages = max_pages;
  e = hipMemcpyAsync(ws, table, (size_t)batch * max_pages * sizeof(int32_t), hipMemcpyHostToDevice, s);
  return pg;
}

// common front of the paged calls: descriptor, table, workspace; on success `view` describes
// the call and the workspace past the table is returned in ws_rest/ws_rest_bytes (the caller
// copies the table into the front of the workspace once its own checks pass)
int paged_front(const dkv_paged_cache* pc, const int32_t* table, int32_t max_pages, const int32_t* past_len,
                int32_t batch, int32_t T, void* ws, size_t ws_bytes, size_t need_rest,
                dkv_cache& view, void*& ws_rest, size_t& ws_rest_bytes) {
  int st = check_paged(pc);
  if (st) return st;
  if ((st = check_table(pc, table, max_pages, past_len, batch, T))) return st;
  const size_t tb = table_bytes(batch, max_pages);
  if (!ws || ws_bytes < tb + need_rest || !aligned16(ws))
    return fail(DKV_ERR_WORKSPACE, "workspace %zu bytes, need %zu (16-byte aligned)", ws_bytes, tb + need_rest);
  view = paged_view(pc, batch, max_pages);
  ws_rest = reinterpret_cast<char*>(ws) + tb;
  ws_rest_bytes = ws_bytes - tb;
  return DKV_OK;
}

// ---- device-resident scratch for attn_decode_noalloc: a file-scope array, one copy per GPU the
// library runs on, held until the process ends. Host code never passes the array's name to a
// kernel (on the host that name is only a stand-in, not a device address): each device's copy
// is looked up once, with that device current, by hipGetSymbolAddress, and the address kept.
constexpr size_t kNoAllocScratchBytes = 8u << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the current device's copy of `scratch` (resolved on the first call on that device)
int scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(DKV_ERR_UNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DKV_OK;
}

}  // namespace

extern "C" {

int32_t dkv_version(void) { return 100; }

const char* dkv_last_error(void) { return g_err.c_str(); }

int dkv_timing(int32_t enable) {
  std::lock_guard<std::mutex> lock(g_timing_mu);
  for (TimedSpan& sp : g_spans) {
    (void)hipEventDestroy(sp.start);
    (void)hipEventDestroy(sp.stop);
  }
  g_spans.clear();
  g_timing_on = enable != 0;
  return DKV_OK;
}

int dkv_timing_read(float* ms, int32_t* launches, int32_t n) {
  if (!ms || !launches || n <= 0) return fail(DKV_ERR_INVALID_ARG, "ms and launches must hold n > 0 values");
  for (int i = 0; i < n; ++i) {
    ms[i] = 0.f;
    launches[i] = 0;
  }
  std::lock_guard<std::mutex> lock(g_timing_mu);
  for (const TimedSpan& sp : g_spans) {
    hipError_t e = hipEventSynchronize(sp.stop);
    float t = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&t, sp.start, sp.stop);
    if (e != hipSuccess) return hip_fail(e, "timing event");
    if (sp.phase < n) {
      ms[sp.phase] += t;
      launches[sp.phase] += sp.launches;
    }
  }
  return DKV_OK;
}

int kv_alloc_host(dkv_cache* out, int32_t batch, int32_t n_kv_heads, int32_t head_dim, int32_t capacity,
                  int32_t dtype) {
  if (!out) return fail(DKV_ERR_INVALID_ARG, "out is null");
  memset(out, 0, sizeof(*out));
  if (batch <= 0 || n_kv_heads <= 0 || capacity <= 0)
    return fail(DKV_ERR_INVALID_ARG, "batch, n_kv_heads and capacity must be positive");
  if (capacity % 64 != 0) return fail(DKV_ERR_INVALID_ARG, "capacity %d must be a multiple of 64", capacity);
  if (dtype < DKV_F32 || dtype > DKV_BF16) return fail(DKV_ERR_UNSUPPORTED, "dtype %d", dtype);
  if (head_dim != 64 && head_dim != 128) return fail(DKV_ERR_UNSUPPORTED, "head_dim %d (built: 64, 128)", head_dim);
  const size_t bytes = (size_t)batch * n_kv_heads * capacity * head_dim * elem_size(dtype);
  if (bytes / elem_size(dtype) / head_dim / capacity != (size_t)batch * n_kv_heads)
    return fail(DKV_ERR_INVALID_ARG, "cache size overflows");
  void *k = nullptr, *v = nullptr;
  const unsigned flags = hipHostMallocMapped | hipHostMallocCoherent;
  hipError_t e = hipHostMalloc(&k, bytes, flags);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(DKV_ERR_HOST_ALLOC, "hipHostMalloc(%zu bytes) for K: %s", bytes, hipGetErrorString(e));
  }
  e = hipHostMalloc(&v, bytes, flags);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    (void)hipHostFree(k);
    return fail(DKV_ERR_HOST_ALLOC, "hipHostMalloc(%zu bytes) for V: %s", bytes, hipGetErrorString(e));
  }
  out->k = k;
  out->v = v;
  out->batch = batch;
  out->n_kv_heads = n_kv_heads;
  out->head_dim = head_dim;
  out->capacity = capacity;
  out->dtype = dtype;
  out->reserved = kMagic;
  return DKV_OK;
}

int kv_free_host(dkv_cache* c) {
  if (!c) return DKV_OK;
  if (c->reserved == kMagic) {
    if (c->k) (void)hipHostFree(c->k);
    if (c->v) (void)hipHostFree(c->v);
  }
  memset(c, 0, sizeof(*c));
  return DKV_OK;
}

int kv_append(const dkv_cache* c, const void* x, const void* wk, const void* wv, const int32_t* past_len,
              int32_t batch, int32_t T, int32_t D, void* stream) {
  int st = check_call(c, batch, T, D, past_len, {x, wk, wv});
  if (st) return st;
  if (T == 0) return DKV_OK;
  if ((st = check_cache_memory(c))) return st;
  return run_append(c, Paging{}, x, wk, wv, past_len, batch, T, D, reinterpret_cast<hipStream_t>(stream));
}

size_t attn_workspace_bytes(int32_t phase, const dkv_cache* c, int32_t batch, int32_t T, int32_t n_q_heads,
                            const int32_t* past_len) {
  (void)past_len;
  if (check_cache(c) || batch <= 0 || n_q_heads <= 0 || T < 0) return 0;
  if (phase == 1) return decode_ws_bytes(c, batch, n_q_heads, false);
  if (phase == 0) return prefill_layout(c, batch, T, n_q_heads).total;
  if (phase == 2) return 2 * staging_bytes(c) + prefill_layout(c, batch, T, n_q_heads).total;
  if (phase == 3) return 2 * staging_bytes(c) + decode_ws_bytes(c, batch, n_q_heads, false);
  return 0;
}

int attn_decode(const dkv_cache* c, const void* x, const void* wq, const void* wk, const void* wv,
                const int32_t* past_len, int32_t batch, int32_t D, int32_t n_q_heads, void* out, void* ws,
                size_t ws_bytes, void* stream) {
  return attn_decode_variant(c, x, wq, wk, wv, past_len, batch, D, n_q_heads, out, ws, ws_bytes, stream,
                             DKV_DECODE_ZEROCOPY);
}

int attn_decode_variant(const dkv_cache* c, const void* x, const void* wq, const void* wk, const void* wv,
                        const int32_t* past_len, int32_t batch, int32_t D, int32_t n_q_heads, void* out, void* ws,
                        size_t ws_bytes, void* stream, int32_t variant) {
  int st = check_call(c, batch, 1, D, past_len, {x, wq, wk, wv, out});
  if (st) return st;
  if ((st = check_heads(c, n_q_heads))) return st;
  if (D > kMaxD) return fail(DKV_ERR_UNSUPPORTED, "decode supports D <= %d", kMaxD);
  if (variant != DKV_DECODE_ZEROCOPY && variant != DKV_DECODE_STAGED)
    return fail(DKV_ERR_INVALID_ARG, "unknown decode variant %d", variant);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t sb = variant == DKV_DECODE_STAGED ? 2 * staging_bytes(c) : 0;
  const size_t need = sb + decode_ws_bytes(c, batch, n_q_heads, false);
  if (!ws || ws_bytes < need || !aligned16(ws))
    return fail(DKV_ERR_WORKSPACE, "workspace %zu bytes, need %zu (16-byte aligned)", ws_bytes, need);
  if ((st = check_cache_memory(c))) return st;
  if (variant == DKV_DECODE_ZEROCOPY)
    return run_decode(c, Paging{}, x, wq, wk, wv, past_len, batch, D, n_q_heads, out, ws, ws_bytes, s);
  const dkv_cache dev = staged_view(c, ws);
  if ((st = stage_in(c, dev, past_len, s))) return st;
  if ((st = run_decode(&dev, Paging{}, x, wq, wk, wv, past_len, batch, D, n_q_heads, out,
                       reinterpret_cast<char*>(ws) + sb, ws_bytes - sb, s)))
    return st;
  return stage_out(c, dev, past_len, 1, s);
}

namespace {
int check_rope(double theta) {
  if (!(theta > 1.0) || theta > 1e30)
    return fail(DKV_ERR_INVALID_ARG, "rope_theta must be a finite base > 1 (got %g)", theta);
  return DKV_OK;
}
}  // namespace

int attn_prefill_rope(const dkv_cache* c, const void* x, const void* wq, const void* wk, const void* wv,
                      const int32_t* past_len, int32_t batch, int32_t T, int32_t D, int32_t n_q_heads, void* out,
                      void* ws, size_t ws_bytes, double rope_theta, void* stream) {
  int st = check_call(c, batch, T, D, past_len, {x, wq, wk, wv, out});
  if (st) return st;
  if ((st = check_heads(c, n_q_heads))) return st;
  if ((st = check_rope(rope_theta))) return st;
  if (T == 0) return DKV_OK;
  const size_t need = prefill_layout(c, batch, T, n_q_heads).total;
  if (!ws || ws_bytes < need || !aligned16(ws))
    return fail(DKV_ERR_WORKSPACE, "workspace %zu bytes, need %zu (16-byte aligned)", ws_bytes, need);
  if ((st = check_cache_memory(c))) return st;
  return run_prefill(c, Paging{}, x, wq, wk, wv, past_len, batch, T, D, n_q_heads, out, ws, ws_bytes,
                     reinterpret_cast<hipStream_t>(stream), DKV_PREFILL_FUSED, rope_theta);
}

int attn_decode_rope(const dkv_cache* c, const void* x, const void* wq, const void* wk, const void* wv,
                     const int32_t* past_len, int32_t batch, int32_t D, int32_t n_q_heads, void* out, void* ws,
                     size_t ws_bytes, double rope_theta, void* stream) {
  int st = check_call(c, batch, 1, D, past_len, {x, wq, wk, wv, out});
  if (st) return st;
  if ((st = check_heads(c, n_q_heads))) return st;
  if (D > kMaxD) return fail(DKV_ERR_UNSUPPORTED, "decode supports D <= %d", kMaxD);
  if ((st = check_rope(rope_theta))) return st;
  const size_t need = decode_ws_bytes(c, batch, n_q_heads, false);
  if (!ws || ws_bytes < need || !aligned16(ws))
    return fail(DKV_ERR_WORKSPACE, "workspace %zu bytes, need %zu (16-byte aligned)", ws_bytes, need);
  if ((st = check_cache_memory(c))) return st;
  return run_decode(c, Paging{}, x, wq, wk, wv, past_len, batch, D, n_q_heads, out, ws, ws_bytes,
                    reinterpret_cast<hipStream_t>(stream), rope_theta);
}

int attn_decode_noalloc(const dkv_cache* c, const void* x, const void* wq, const void* wk, const void* wv,
                        const int32_t* past_len, int32_t batch, int32_t D, int32_t n_q_heads, void* out,
                        void* stream) {
  int st = check_call(c, batch, 1, D, past_len, {x, wq, wk, wv, out});
  if (st) return st;
  if ((st = check_heads(c, n_q_heads))) return st;
  if (D > kMaxD) return fail(DKV_ERR_UNSUPPORTED, "decode supports D <= %d", kMaxD);
  const size_t need = decode_ws_bytes(c, batch, n_q_heads, false);
  if (need > kNoAllocScratchBytes)
    return fail(DKV_ERR_WORKSPACE,
                "attn_decode_noalloc: this call needs %zu bytes of scratch, the library's device scratch holds %zu "
                "(use attn_decode with a workspace)", need, kNoAllocScratchBytes);
  if ((st = check_cache_memory(c))) return st;
  void* ws = nullptr;
  if ((st = scratch_for_current_device(&ws))) return st;
  // every byte the kernels read from the scratch is written earlier in the same call (the split
  // partials by the decode kernel, the queries by the projection pre-pass): nothing to clear
  return run_decode(c, Paging{}, x, wq, wk, wv, past_len, batch, D, n_q_heads, out, ws, kNoAllocScratchBytes,
                    reinterpret_cast<hipStream_t>(stream));
}

int attn_prefill(const dkv_cache* c, const void* x, const void* wq, const void* wk, const void* wv,
                 const int32_t* past_len, int32_t batch, int32_t T, int32_t D, int32_t n_q_heads, void* out,
                 void* ws, size_t ws_bytes, void* stream) {
  return attn_prefill_variant(c, x, wq, wk, wv, past_len, batch, T, D, n_q_heads, out, ws, ws_bytes, stream,
                              DKV_PREFILL_FUSED);
}

int attn_prefill_variant(const dkv_cache* c, const void* x, const void* wq, const void* wk, const void* wv,
                         const int32_t* past_len, int32_t batch, int32_t T, int32_t D, int32_t n_q_heads,
                         void* out, void* ws, size_t ws_bytes, void* stream, int32_t variant) {
  int st = check_call(c, batch, T, D, past_len, {x, wq, wk, wv, out});
  if (st) return st;
  if ((st = check_heads(c, n_q_heads))) return st;
  if (variant < DKV_PREFILL_FUSED || variant > DKV_PREFILL_PERSIST)
    return fail(DKV_ERR_INVALID_ARG, "unknown prefill variant %d", variant);
  // The persistent launch (workgroups handing the running state to each other through counters)
  // did not complete on the GPU and its cause was not found: it is disabled and no longer built.
  if (variant == DKV_PREFILL_PERSIST)
    return fail(DKV_ERR_UNSUPPORTED, "DKV_PREFILL_PERSIST is disabled (not built): its launch did not complete on "
                                     "the GPU");
  if (T == 0) return DKV_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t sb = variant == DKV_PREFILL_STAGED ? 2 * staging_bytes(c) : 0;
  const size_t need = sb + prefill_layout(c, batch, T, n_q_heads).total;
  if (!ws || ws_bytes < need || !aligned16(ws))
    return fail(DKV_ERR_WORKSPACE, "workspace %zu bytes, need %zu (16-byte aligned)", ws_bytes, need);
  if ((st = check_cache_memory(c))) return st;
  if (variant != DKV_PREFILL_STAGED)
    return run_prefill(c, Paging{}, x, wq, wk, wv, past_len, batch, T, D, n_q_heads, out, ws, ws_bytes, s, variant);
  const dkv_cache dev = staged_view(c, ws);
  if ((st = stage_in(c, dev, past_len, s))) return st;
  if ((st = run_prefill(&dev, Paging{}, x, wq, wk, wv, past_len, batch, T, D, n_q_heads, out,
                        reinterpret_cast<char*>(ws) + sb, ws_bytes - sb, s, DKV_PREFILL_FUSED)))
    return st;
  return stage_out(c, dev, past_len, T, s);
}

int kv_paged_alloc_host(dkv_paged_cache* out, int32_t n_pages, int32_t n_kv_heads, int32_t head_dim,
                        int32_t dtype) {
  if (!out) return fail(DKV_ERR_INVALID_ARG, "out is null");
  memset(out, 0, sizeof(*out));
  if (n_pages <= 0 || n_kv_heads <= 0) return fail(DKV_ERR_INVALID_ARG, "n_pages and n_kv_heads must be positive");
  if (dtype < DKV_F32 || dtype > DKV_BF16) return fail(DKV_ERR_UNSUPPORTED, "dtype %d", dtype);
  if (head_dim != 64 && head_dim != 128) return fail(DKV_ERR_UNSUPPORTED, "head_dim %d (built: 64, 128)", head_dim);
  const size_t bytes = (size_t)n_pages * n_kv_heads * kPageTokens * head_dim * elem_size(dtype);
  if (bytes / elem_size(dtype) / head_dim / kPageTokens / n_kv_heads != (size_t)n_pages)
    return fail(DKV_ERR_INVALID_ARG, "page pool size overflows");
  void *k = nullptr, *v = nullptr;
  const unsigned flags = hipHostMallocMapped | hipHostMallocCoherent;
  hipError_t e = hipHostMalloc(&k, bytes, flags);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(DKV_ERR_HOST_ALLOC, "hipHostMalloc(%zu bytes) for the K pages: %s", bytes, hipGetErrorString(e));
  }
  e = hipHostMalloc(&v, bytes, flags);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    (void)hipHostFree(k);
    return fail(DKV_ERR_HOST_ALLOC, "hipHostMalloc(%zu bytes) for the V pages: %s", bytes, hipGetErrorString(e));
  }
  out->k = k;
  out->v = v;
  out->n_pages = n_pages;
  out->n_kv_heads = n_kv_heads;
  out->head_dim = head_dim;
  out->dtype = dtype;
  out->reserved = kPagedMagic;
  return DKV_OK;
}

int kv_paged_free_host(dkv_paged_cache* c) {
  if (!c) return DKV_OK;
  if (c->reserved == kPagedMagic) {
    if (c->k) (void)hipHostFree(c->k);
    if (c->v) (void)hipHostFree(c->v);
  }
  memset(c, 0, sizeof(*c));
  return DKV_OK;
}

size_t attn_paged_workspace_bytes(int32_t phase, const dkv_paged_cache* c, int32_t batch, int32_t T,
                                  int32_t n_q_heads, int32_t max_pages) {
  if (check_paged(c) || batch <= 0 || batch > kMaxBatch || T < 0 || max_pages <= 0) return 0;
  const dkv_cache view = paged_view(c, batch, max_pages);
  const size_t tb = table_bytes(batch, max_pages);
  if (phase == 2) return tb;
  if (n_q_heads <= 0) return 0;
  if (phase == 1) return tb + decode_ws_bytes(&view, batch, n_q_heads, true);
  if (phase == 0) return tb + prefill_layout(&view, batch, T, n_q_heads, true).total;
  return 0;
}

int kv_paged_append(const dkv_paged_cache* c, const int32_t* block_table, int32_t max_pages, const void* x,
                    const void* wk, const void* wv, const int32_t* past_len, int32_t batch, int32_t T, int32_t D,
                    void* ws, size_t ws_bytes, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  dkv_cache view;
  Paging pg;
  void* rest;
  size_t rest_bytes;
  int st = paged_front(c, block_table, max_pages, past_len, batch, T, ws, ws_bytes, 0, view, rest, rest_bytes);
  if (st) return st;
  if ((st = check_call(&view, batch, T, D, past_len, {x, wk, wv}))) return st;
  if (T == 0) return DKV_OK;
  if ((st = check_paged_memory(c))) return st;
  hipError_t e;
  pg = stage_table(block_table, batch, max_pages, ws, s, e);
  if (e != hipSuccess) return hip_fail(e, "block table copy");
  return run_append(&view, pg, x, wk, wv, past_len, batch, T, D, s);
}

int attn_decode_paged(const dkv_paged_cache* c, const int32_t* block_table, int32_t max_pages, const void* x,
                      const void* wq, const void* wk, const void* wv, const int32_t* past_len, int32_t batch,
                      int32_t D, int32_t n_q_heads, void* out, void* ws, size_t ws_bytes, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  dkv_cache view;
  Paging pg;
  void* rest;
  size_t rest_bytes;
  int st = check_paged(c);
  if (st) return st;
  if (batch <= 0 || batch > kMaxBatch || max_pages <= 0)
    return fail(DKV_ERR_INVALID_ARG, "batch must be in [1, %d] and max_pages positive", kMaxBatch);
  const dkv_cache pre = paged_view(c, batch, max_pages);
  if (n_q_heads <= 0) return fail(DKV_ERR_INVALID_ARG, "n_q_heads must be positive");
  const size_t need = decode_ws_bytes(&pre, batch, n_q_heads, true);
  st = paged_front(c, block_table, max_pages, past_len, batch, 1, ws, ws_bytes, need, view, rest, rest_bytes);
  if (st) return st;
  if ((st = check_call(&view, batch, 1, D, past_len, {x, wq, wk, wv, out}))) return st;
  if ((st = check_heads(&view, n_q_heads))) return st;
  if (D > kMaxD) return fail(DKV_ERR_UNSUPPORTED, "decode supports D <= %d", kMaxD);
  if ((st = check_paged_memory(c))) return st;
  hipError_t e;
  pg = stage_table(block_table, batch, max_pages, ws, s, e);
  if (e != hipSuccess) return hip_fail(e, "block table copy");
  return run_decode(&view, pg, x, wq, wk, wv, past_len, batch, D, n_q_heads, out, rest, rest_bytes, s);
}

int attn_prefill_paged(const dkv_paged_cache* c, const int32_t* block_table, int32_t max_pages, const void* x,
                       const void* wq, const void* wk, const void* wv, const int32_t* past_len, int32_t batch,
                       int32_t T, int32_t D, int32_t n_q_heads, void* out, void* ws, size_t ws_bytes,
                       void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  dkv_cache view;
  Paging pg;
  void* rest;
  size_t rest_bytes;
  int st = check_paged(c);
  if (st) return st;
  if (batch <= 0 || batch > kMaxBatch || max_pages <= 0 || T < 0)
    return fail(DKV_ERR_INVALID_ARG, "batch must be in [1, %d], max_pages positive and T >= 0", kMaxBatch);
  if (n_q_heads <= 0) return fail(DKV_ERR_INVALID_ARG, "n_q_heads must be positive");
  const dkv_cache pre = paged_view(c, batch, max_pages);
  const size_t need = prefill_layout(&pre, batch, T, n_q_heads, true).total;
  st = paged_front(c, block_table, max_pages, past_len, batch, T, ws, ws_bytes, need, view, rest, rest_bytes);
  if (st) return st;
  if ((st = check_call(&view, batch, T, D, past_len, {x, wq, wk, wv, out}))) return st;
  if ((st = check_heads(&view, n_q_heads))) return st;
  if (T == 0) return DKV_OK;
  if ((st = check_paged_memory(c))) return st;
  hipError_t e;
  pg = stage_table(block_table, batch, max_pages, ws, s, e);
  if (e != hipSuccess) return hip_fail(e, "block table copy");
  return run_prefill(&view, pg, x, wq, wk, wv, past_len, batch, T, D, n_q_heads, out, rest, rest_bytes, s,
                     DKV_PREFILL_FUSED);
}

// ---- decode-loop helpers

namespace {
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}
int check_dtype(int32_t dtype) {
  return (dtype < DKV_F32 || dtype > DKV_BF16) ? fail(DKV_ERR_UNSUPPORTED, "dtype %d", dtype) : DKV_OK;
}
}  // namespace

int dkv_rmsnorm(const void* x, const void* weight, void* y, int32_t rows, int32_t D, float eps, int32_t dtype,
                void* stream) {
  int st = check_dtype(dtype);
  if (st) return st;
  if (!x || !weight || !y) return fail(DKV_ERR_INVALID_ARG, "a pointer is null");
  if (rows <= 0 || D <= 0) return fail(DKV_ERR_INVALID_ARG, "rows and D must be positive");
  if (!(eps >= 0.f)) return fail(DKV_ERR_INVALID_ARG, "eps must be >= 0");
  const size_t e = elem_size(dtype);
  if (x != y && overlaps(x, (size_t)rows * D * e, y, (size_t)rows * D * e))
    return fail(DKV_ERR_INVALID_ARG, "y overlaps x without being x");
  hipError_t err = launch_rmsnorm(dtype, x, weight, y, rows, D, eps, reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? DKV_OK : hip_fail(err, "rmsnorm launch");
}

int dkv_linear(const void* x, const void* w, const void* residual, void* y, int32_t rows, int32_t N, int32_t K,
               int32_t dtype, void* stream) {
  int st = check_dtype(dtype);
  if (st) return st;
  if (!x || !w || !y) return fail(DKV_ERR_INVALID_ARG, "a pointer is null");
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (residual && !aligned16(residual)))
    return fail(DKV_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  if (rows <= 0 || N <= 0 || K <= 0) return fail(DKV_ERR_INVALID_ARG, "rows, N and K must be positive");
  const size_t e = elem_size(dtype);
  if ((K * e) % 16 != 0) return fail(DKV_ERR_INVALID_ARG, "K=%d: rows of x and w must be whole 16-byte units", K);
  const size_t ny = (size_t)rows * N * e;
  if (overlaps(x, (size_t)rows * K * e, y, ny)) return fail(DKV_ERR_INVALID_ARG, "y overlaps x");
  if (residual && residual != y && overlaps(residual, ny, y, ny))
    return fail(DKV_ERR_INVALID_ARG, "y overlaps the residual without being it");
  hipError_t err = launch_linear(dtype, x, w, residual, y, rows, N, K, reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? DKV_OK : hip_fail(err, "linear launch");
}

int dkv_swiglu(const void* gate_up, void* y, int32_t rows, int32_t F, int32_t dtype, void* stream) {
  int st = check_dtype(dtype);
  if (st) return st;
  if (!gate_up || !y) return fail(DKV_ERR_INVALID_ARG, "a pointer is null");
  if (rows <= 0 || F <= 0) return fail(DKV_ERR_INVALID_ARG, "rows and F must be positive");
  const size_t e = elem_size(dtype);
  if (overlaps(gate_up, (size_t)rows * 2 * F * e, y, (size_t)rows * F * e))
    return fail(DKV_ERR_INVALID_ARG, "y overlaps gate_up");
  hipError_t err = launch_swiglu(dtype, gate_up, y, rows, F, reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? DKV_OK : hip_fail(err, "swiglu launch");
}

int dkv_hostlink_stream(void* host_ptr, size_t bytes, int32_t mode, int32_t n_wg, void* stream) {
  if (!host_ptr || !aligned16(host_ptr)) return fail(DKV_ERR_INVALID_ARG, "host_ptr null or misaligned");
  if (mode != 0 && mode != 1) return fail(DKV_ERR_INVALID_ARG, "mode must be 0 (read) or 1 (write)");
  if (n_wg <= 0 || bytes == 0 || bytes % (16 * (size_t)n_wg) != 0)
    return fail(DKV_ERR_INVALID_ARG, "bytes must be a positive multiple of 16 * n_wg");
  hipError_t e = launch_hostlink(host_ptr, bytes, mode, n_wg, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "hostlink launch");
  return DKV_OK;
}

}  // extern "C"
