// C ABI of the IceCache library: argument checks, layout sizing and the
// entry points declared in include/ice.h. Every check runs on the host before
// anything is enqueued; device work goes to the caller's stream.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <cstddef>
#include <string>
#include <vector>

#include "ice_launch.h"

using namespace ice;

// Build scratch of ice_build_noalloc: a fixed array in every device's global
// memory, loaded with the library and held until the process ends. In host
// code `scratch` only names the symbol; its device address is looked up once
// per device (hipGetSymbolAddress) and used in its place.
static __device__ __align__(256) char scratch[ICE_NOALLOC_SCRATCH_BYTES];

struct ice_index {
  ice_params p;
  DevLayout L;
  WsLayout W;
  void* blob;
  size_t blob_bytes;
  void* host_pool;        // host-pool mode: the caller's pinned V pool (host address)
  int32_t n_tokens;
  int32_t n_dense;        // heads flagged dense (ice_set_dense)
  std::vector<uint8_t> dense;       // the flags, host copy
  std::vector<uint8_t> head_built;  // heads built since the handle was created
  bool built;             // every head built
  // Level counts on the host. pos_ge[l][h]: the positions (< capacity) whose
  // own promotion draw in head h reaches level l >= 1, ascending. runs[h]:
  // the position ranges [t0, t1) of head h's tokens and the head whose draws
  // gave them their levels (a head built by reuse takes its source's levels
  // for the tokens it was built with); ltop[h]: its top level at build.
  struct Run {
    int32_t t0, t1, src;
  };
  std::vector<std::vector<int32_t>> pos_ge[ICE_MAX_LEVELS];
  std::vector<std::vector<Run>> runs;
  std::vector<int32_t> ltop;
  // Pipelined builds: the second stream and its events, made on the device
  // current at the first such build and kept until the handle is destroyed.
  hipStream_t side = nullptr;
  int side_dev = -1;
  std::vector<hipEvent_t> pev;
};

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(ICE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int check_params(const ice_params* p) {
  if (!p) return fail(ICE_ERR_ARG, "params is null");
  if (p->n_heads < 1) return fail(ICE_ERR_ARG, "n_heads must be >= 1");
  if (p->group < 1 || p->group > ICE_MAX_GROUP) return fail(ICE_ERR_ARG, "group must be in [1, %d]", ICE_MAX_GROUP);
  if (p->d != 64 && p->d != 128) return fail(ICE_ERR_DTYPE, "d must be 64 or 128");
  if (p->dtype != ICE_F32 && p->dtype != ICE_BF16) return fail(ICE_ERR_DTYPE, "dtype must be ICE_F32 or ICE_BF16");
  if (p->page_cap != ICE_PAGE_CAP) return fail(ICE_ERR_ARG, "page_cap must be %d", ICE_PAGE_CAP);
  if (p->levels < 1 || p->levels > ICE_MAX_LEVELS) return fail(ICE_ERR_ARG, "levels must be in [1, %d]", ICE_MAX_LEVELS);
  if (p->promote_log2 < 1 || p->promote_log2 > 16) return fail(ICE_ERR_ARG, "promote_log2 must be in [1, 16]");
  // at most 2^26 tokens per head keeps every page id below 2^27, the range a
  // page's selection key holds
  if (p->capacity < 1 || p->capacity > (1 << 26)) return fail(ICE_ERR_ARG, "capacity must be in [1, 2^26]");
  if (p->flags & ~(ICE_HOST_POOL | ICE_SPLIT_RESORT)) return fail(ICE_ERR_ARG, "unknown flags 0x%x", p->flags);
  if ((p->flags & ICE_HOST_POOL) && (p->flags & ICE_SPLIT_RESORT))
    return fail(ICE_ERR_ARG, "ICE_SPLIT_RESORT moves V rows: it needs the device V pool (no ICE_HOST_POOL)");
  if (p->resident < 0 || p->resident > ICE_MAX_RESIDENT)
    return fail(ICE_ERR_ARG, "resident must be in [0, %d]", ICE_MAX_RESIDENT);
  if (p->resident > 0 && (p->flags & ICE_HOST_POOL))
    return fail(ICE_ERR_ARG, "resident tokens need the device V pool (no ICE_HOST_POOL)");
  return ICE_OK;
}

int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

struct Cursor {
  int64_t off = 0;
  int64_t take(int64_t bytes) {
    const int64_t o = off;
    off = align256(off + std::max<int64_t>(bytes, 0));
    return o;
  }
};

// Page bound of one table: every owner's pages are full except its last, so
// pages = sum over owners of ceil(c/16) <= (points + 15 * owners) / 16.
int32_t page_bound(int64_t points, int64_t owners) {
  return (int32_t)((points + 15 * std::max<int64_t>(owners, 1) + 15) / 16);
}

void make_layout(const ice_params* p, DevLayout* L, WsLayout* W) {
  memset(L, 0, sizeof(*L));
  memset(W, 0, sizeof(*W));
  L->H = p->n_heads;
  L->G = p->group;
  L->d = p->d;
  L->dtype = p->dtype;
  L->L = p->levels;
  L->plog2 = p->promote_log2;
  L->cap = p->capacity;
  L->ntab = std::max(1, p->levels - 1);
  L->seed = p->seed;
  L->resort = (p->flags & ICE_SPLIT_RESORT) ? 1 : 0;
  L->elt = p->dtype == ICE_BF16 ? 2 : 4;
  // level counts over every position a head can ever hold
  L->ncap[0] = p->capacity;
  for (int h = 0; h < p->n_heads; ++h) {
    int32_t c[ICE_MAX_LEVELS] = {0, 0, 0, 0};
    for (int t = 0; t < p->capacity; ++t) {
      const int lv = draw_level(p->seed, h, t, p->levels, p->promote_log2);
      for (int l = 1; l <= lv; ++l) ++c[l];
    }
    for (int l = 1; l < p->levels; ++l) L->ncap[l] = std::max(L->ncap[l], c[l]);
  }
  for (int l = 0; l < L->ntab; ++l) {
    const int64_t owners = l + 1 < p->levels ? L->ncap[l + 1] : 0;
    L->pcap[l] = page_bound(L->ncap[l], owners);
  }
  L->topcap = p->levels >= 2 ? std::max(L->ncap[1], 1) : 0;
  L->res_pages = (p->resident + ICE_PAGE_CAP - 1) / ICE_PAGE_CAP;
  const int64_t d = p->d, elt = L->elt, cap = p->capacity;
  Cursor c;
  L->off_hdr = c.take(sizeof(Hdr));
  L->off_lev = c.take(cap);
  L->off_e = c.take(cap * 4);
  for (int l = 0; l < L->ntab; ++l) L->off_parent[l] = c.take(cap * 4);
  for (int l = 0; l < L->ntab; ++l) {
    // table 0 also holds the resident pages, after its pcap[0] pages
    const int64_t P = L->pcap[l] + (l == 0 ? L->res_pages : 0);
    L->off_pg_tok[l] = c.take(P * ICE_PAGE_CAP * 4);
    L->off_pg_cnt[l] = c.take(P * 4);
    L->off_pg_next[l] = c.take(P * 4);
    L->off_pg_owner[l] = c.take(P * 4);
    L->off_first[l] = c.take((cap + 1) * 4);
    L->off_tail[l] = c.take((cap + 1) * 4);
    L->off_orun[l] = c.take((cap + 1) * 4);
    L->off_ocnt[l] = c.take((cap + 1) * 4);
    L->off_pgK[l] = c.take(P * ICE_PAGE_CAP * d * elt);
    if (l == 0) {
      // host-pool mode keeps V out of the blob: the pool holds it per head
      if (p->flags & ICE_HOST_POOL) L->vpool_head_bytes = align256(P * ICE_PAGE_CAP * d * elt);
      else L->off_pgV = c.take(P * ICE_PAGE_CAP * d * elt);
    } else {
      L->off_pgE[l] = c.take(P * ICE_PAGE_CAP * 4);
    }
  }
  L->off_top_tok = c.take((int64_t)L->topcap * 4);
  L->off_top_K = c.take((int64_t)L->topcap * d * elt);
  L->off_top_E = c.take((int64_t)L->topcap * 4);
  L->head_bytes = c.off;

  // build workspace per head
  W->kp = p->dtype == ICE_BF16 ? p->d + 16 : p->d + 4;
  Cursor w;
  W->off_n2 = w.take(cap * 8);
  for (int l = 1; l < p->levels; ++l) W->off_rank[l] = w.take(cap * 4);
  for (int l = 1; l < p->levels; ++l) W->off_pts[l] = w.take((int64_t)L->ncap[l] * 4);
  for (int l = 0; l < p->levels; ++l) W->off_exact[l] = w.take((int64_t)L->ncap[l] * 4);
  W->off_cnts = w.take(2 * ICE_MAX_LEVELS * 4);
  W->off_blkcnt = w.take((cap + kLiftBlock - 1) / kLiftBlock * 2 * ICE_MAX_LEVELS * 4);
  const int64_t n1 = p->levels >= 2 ? L->ncap[1] : 0;
  // candidate operand rows, plus kGemmPadRows rows the parent GEMM may read
  // past the last candidate (its stage loads carry no bounds checks)
  W->off_opA = w.take((n1 + kGemmPadRows) * W->kp * elt);
  W->off_s1 = w.take(cap * 4);
  W->off_s2 = w.take(cap * 4);
  W->off_oloc = w.take(cap * 4);
  W->off_cnt = w.take((n1 + 1) * 4);
  W->off_fill = w.take((n1 + 1) * 4);
  W->off_cbase = w.take((n1 + 1) * 4);
  W->off_pbase = w.take((n1 + 1) * 4);
  W->off_brec = w.take(cap * 16);
  W->head_bytes = w.off;
  W->build_bytes = W->head_bytes * p->n_heads;
  W->pdci_bytes = align256((int64_t)p->n_heads * ICE_PDCI_MAX_KEYS * n1 * 24);
}

bool host_mode(const DevLayout& L) { return L.vpool_head_bytes > 0; }
int64_t page_bytes(const DevLayout& L) { return (int64_t)ICE_PAGE_CAP * L.d * L.elt; }
// attention's workspace: nothing in the device-pool mode; in host-pool mode
// the V staging area of uni_stride pages per head
int64_t attend_ws_bytes(const DevLayout& L, int uni_stride) {
  const int64_t stage = host_mode(L) ? (int64_t)L.H * uni_stride * page_bytes(L) : 0;
  return align256(stage);
}
// the layout attention runs with: staged V in host-pool mode
DevLayout attend_layout(const DevLayout& L, void* ws, int uni_stride) {
  DevLayout A = L;
  if (host_mode(L)) {
    A.vstage = static_cast<const char*>(ws);
    A.vstage_pages = uni_stride;
  }
  return A;
}

int check_budget(const ice_index* idx, int32_t budget) {
  if (budget < ICE_PAGE_CAP || budget % ICE_PAGE_CAP != 0 || budget > ICE_MAX_BEAM * ICE_PAGE_CAP)
    return fail(ICE_ERR_ARG, "budget_tokens must be a positive multiple of %d, at most %d", ICE_PAGE_CAP,
                ICE_MAX_BEAM * ICE_PAGE_CAP);
  (void)idx;
  return ICE_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Tokens of head h at level >= l (l >= 1, at most its top level) once its
// runs extend to position t_end with its own draws.
int64_t level_count(const ice_index* idx, int h, int l, int32_t t_end) {
  int64_t c = 0;
  int32_t covered = 0;
  auto in_range = [&](int src, int32_t a, int32_t b) {
    const std::vector<int32_t>& v = idx->pos_ge[l][src];
    return (int64_t)(std::lower_bound(v.begin(), v.end(), b) - std::lower_bound(v.begin(), v.end(), a));
  };
  for (const auto& r : idx->runs[h]) {
    c += in_range(r.src, r.t0, r.t1);
    covered = std::max(covered, r.t1);
  }
  if (t_end > covered) c += in_range(h, covered, t_end);
  return c;
}

// Top level at build: the highest level holding a token of [0, n).
int32_t top_from_draws(const ice_index* idx, int h, int32_t n) {
  int32_t lt = 0;
  for (int l = 1; l < idx->p.levels; ++l) {
    const std::vector<int32_t>& v = idx->pos_ge[l][h];
    if (!v.empty() && v.front() < n) lt = l;
  }
  return lt;
}

// Records heads h0..h0+n_heads-1 as built from their own draws with n tokens.
void note_own_build(ice_index* idx, int h0, int n_heads, int32_t n) {
  for (int h = h0; h < h0 + n_heads; ++h) {
    idx->runs[h].clear();
    if (n > 0) idx->runs[h].push_back({0, n, h});
    idx->ltop[h] = top_from_draws(idx, h, n);
  }
}

}  // namespace

extern "C" {

const char* ice_last_error(void) { return g_err.c_str(); }

size_t ice_index_bytes(const ice_params* p) {
  if (check_params(p) != ICE_OK) return 0;
  DevLayout L;
  WsLayout W;
  make_layout(p, &L, &W);
  return (size_t)(L.head_bytes * p->n_heads);
}

size_t ice_workspace_bytes(const ice_params* p, int32_t max_budget_tokens) {
  if (check_params(p) != ICE_OK) return 0;
  if (max_budget_tokens < ICE_PAGE_CAP || max_budget_tokens % ICE_PAGE_CAP != 0 ||
      max_budget_tokens > ICE_MAX_BEAM * ICE_PAGE_CAP) {
    fail(ICE_ERR_ARG, "max_budget_tokens must be a positive multiple of %d", ICE_PAGE_CAP);
    return 0;
  }
  DevLayout L;
  WsLayout W;
  make_layout(p, &L, &W);
  const int64_t att = attend_ws_bytes(L, p->group * (max_budget_tokens / ICE_PAGE_CAP));
  return (size_t)std::max<int64_t>(W.build_bytes + W.pdci_bytes, att);
}

size_t ice_host_pool_bytes(const ice_params* p) {
  if (check_params(p) != ICE_OK || !(p->flags & ICE_HOST_POOL)) return 0;
  DevLayout L;
  WsLayout W;
  make_layout(p, &L, &W);
  return (size_t)(L.vpool_head_bytes * p->n_heads);
}

int ice_create(const ice_params* p, void* index_dev, size_t index_bytes, ice_index** out) {
  if (!out) return fail(ICE_ERR_ARG, "out is null");
  *out = nullptr;
  int rc = check_params(p);
  if (rc) return rc;
  if (!index_dev) return fail(ICE_ERR_ARG, "index blob is null");
  if (((uintptr_t)index_dev & 255u) != 0) return fail(ICE_ERR_ARG, "index blob must be 256-byte aligned");
  ice_index* idx = new (std::nothrow) ice_index;
  if (!idx) return fail(ICE_ERR_ARG, "out of host memory");
  idx->p = *p;
  make_layout(p, &idx->L, &idx->W);
  if (index_bytes < (size_t)(idx->L.head_bytes * p->n_heads)) {
    delete idx;
    return fail(ICE_ERR_CAPACITY, "index blob has %zu bytes, needs %lld", index_bytes,
                (long long)(idx->L.head_bytes * p->n_heads));
  }
  idx->blob = index_dev;
  idx->blob_bytes = index_bytes;
  idx->host_pool = nullptr;
  idx->n_tokens = 0;
  idx->n_dense = 0;
  idx->dense.assign(p->n_heads, 0);
  idx->head_built.assign(p->n_heads, 0);
  idx->built = false;
  for (int l = 1; l < p->levels; ++l) idx->pos_ge[l].assign(p->n_heads, {});
  for (int h = 0; h < p->n_heads; ++h)
    for (int t = 0; t < p->capacity; ++t) {
      const int lv = draw_level(p->seed, h, t, p->levels, p->promote_log2);
      for (int l = 1; l <= lv; ++l) idx->pos_ge[l][h].push_back(t);
    }
  idx->runs.assign(p->n_heads, {});
  idx->ltop.assign(p->n_heads, 0);
  *out = idx;
  return ICE_OK;
}

void ice_destroy(ice_index* idx) {
  if (!idx) return;
  for (hipEvent_t e : idx->pev) (void)hipEventDestroy(e);
  if (idx->side) (void)hipStreamDestroy(idx->side);
  delete idx;
}

int ice_attach_host_pool(ice_index* idx, void* host_pool, size_t host_pool_bytes) {
  if (!idx) return fail(ICE_ERR_ARG, "index is null");
  if (!host_mode(idx->L)) return fail(ICE_ERR_STATE, "the index was created without ICE_HOST_POOL");
  if (!host_pool) return fail(ICE_ERR_ARG, "host pool is null");
  if (((uintptr_t)host_pool & 255u) != 0) return fail(ICE_ERR_ARG, "host pool must be 256-byte aligned");
  const size_t need = (size_t)(idx->L.vpool_head_bytes * idx->p.n_heads);
  if (host_pool_bytes < need)
    return fail(ICE_ERR_CAPACITY, "host pool has %zu bytes, needs %zu", host_pool_bytes, need);
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, host_pool);
  if (e != hipSuccess || attr.type != hipMemoryTypeHost) {
    (void)hipGetLastError();
    return fail(ICE_ERR_ARG, "host pool is not pinned host memory (allocate it with hipHostMalloc)");
  }
  void* dev = nullptr;
  e = hipHostGetDevicePointer(&dev, host_pool, 0);
  if (e != hipSuccess || !dev) return hip_fail(e, "hipHostGetDevicePointer of the host pool");
  idx->host_pool = host_pool;
  idx->L.vpool = static_cast<char*>(dev);
  return ICE_OK;
}

int32_t ice_n_tokens(const ice_index* idx) { return idx ? idx->n_tokens : -1; }

}  // extern "C"

namespace {

// Pipelined builds. The level-0 parent search keeps the matrix cores busy and
// leaves HBM mostly idle, while the lift before it and the pack, page copies
// and upper levels after it are HBM-bound. Heads are independent (each has
// its own part of the blob and of the workspace), so a build of many heads is
// cut into ranges of heads and run as a two-stream pipeline: the caller's
// stream runs the ranges' level-0 searches back to back, and the side stream
// runs each range's lift ahead of its search and the rest of its build after
// it, overlapping the next range's search. The result is the one-stream
// build's: every kernel sees the same heads and the same order within a head.
#ifndef ICE_BUILD_CHUNKS
#define ICE_BUILD_CHUNKS 4     // ranges per pipelined build
#endif
constexpr int kMaxBuildChunks = 16;
constexpr int kMinChunkHeads = 8;  // fewer heads per range: one stream
static_assert(ICE_BUILD_CHUNKS >= 2 && ICE_BUILD_CHUNKS <= kMaxBuildChunks, "build ranges");

hipError_t ensure_side(ice_index* idx);

// Ranges a build of n_heads heads runs over (1: on the caller's stream alone,
// also under stream capture, on a device other than the side stream's, and
// when the side stream cannot be made). A query that fails leaves no error
// behind for the build's own launch checks.
int build_chunks(ice_index* idx, int n_heads, hipStream_t s) {
  if (idx->p.levels < 2) return 1;  // no parent search to overlap
  const int c = std::min(ICE_BUILD_CHUNKS, n_heads / kMinChunkHeads);
  if (c < 2) return 1;
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  int dev = -1;
  if (hipStreamIsCapturing(s, &st) != hipSuccess || hipGetDevice(&dev) != hipSuccess || ensure_side(idx) != hipSuccess) {
    (void)hipGetLastError();
    return 1;
  }
  if (st != hipStreamCaptureStatusNone || dev != idx->side_dev) return 1;
  return c;
}

// The side stream (default priority, not synchronising with the null stream)
// and 2 + 2 * kMaxBuildChunks events without timing, made once per handle on
// the current device.
hipError_t ensure_side(ice_index* idx) {
  if (idx->side) return hipSuccess;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::vector<hipEvent_t> ev(2 + 2 * kMaxBuildChunks, nullptr);
  size_t made = 0;
  for (; made < ev.size() && e == hipSuccess; ++made) e = hipEventCreateWithFlags(&ev[made], hipEventDisableTiming);
  hipStream_t t = nullptr;
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&t, hipStreamNonBlocking);
  if (e != hipSuccess) {
    for (size_t i = 0; i < made; ++i)
      if (ev[i]) (void)hipEventDestroy(ev[i]);
    return e;
  }
  idx->pev = std::move(ev);
  idx->side = t;
  idx->side_dev = dev;
  return hipSuccess;
}

// The build of the range L (already offset to its first head: blob, ws, K,
// V) as `chunks` ranges on the caller's stream s and the side stream (made
// by build_chunks). s
// continues after all of it (the side stream's last event), also when a
// launch fails part way.
hipError_t build_pipelined(ice_index* idx, const DevLayout& L, char* blob, const void* K, const void* V, int n,
                           int64_t hstride, char* ws, bool keep, hipStream_t s, int chunks) {
  hipError_t e = hipSuccess;
  const int per = (L.H + chunks - 1) / chunks;
  chunks = (L.H + per - 1) / per;
  hipStream_t t = idx->side;
  // pev[0]: fork, pev[1]: join, pev[2 + 2c]: range c lifted, pev[3 + 2c]: range c searched
  hipEvent_t* ev = idx->pev.data();
  auto part = [&](int c, BuildPart what, hipStream_t st) -> hipError_t {
    const int a = c * per;
    DevLayout R = L;
    R.H = std::min(per, L.H - a);
    R.h0 = L.h0 + a;
    if (R.vpool) R.vpool += (int64_t)a * L.vpool_head_bytes;
    const int64_t kv = (int64_t)a * hstride * L.elt;
    return launch_build(R, idx->W, blob + (int64_t)a * L.head_bytes, static_cast<const char*>(K) + kv,
                        static_cast<const char*>(V) + kv, n, hstride, ws + (int64_t)a * idx->W.head_bytes, keep, st,
                        nullptr, nullptr, what);
  };
  if ((e = hipEventRecord(ev[0], s)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(t, ev[0], 0)) != hipSuccess) return e;
  // the lifts first, so that no search waits behind another range's rest
  for (int c = 0; c < chunks && e == hipSuccess; ++c) {
    if ((e = part(c, BuildPart::kLift, t)) != hipSuccess) break;
    e = hipEventRecord(ev[2 + 2 * c], t);
  }
  for (int c = 0; c < chunks && e == hipSuccess; ++c) {
    if ((e = hipStreamWaitEvent(s, ev[2 + 2 * c], 0)) != hipSuccess) break;
    if ((e = part(c, BuildPart::kParent0, s)) != hipSuccess) break;
    if ((e = hipEventRecord(ev[3 + 2 * c], s)) != hipSuccess) break;
    if ((e = hipStreamWaitEvent(t, ev[3 + 2 * c], 0)) != hipSuccess) break;
    e = part(c, BuildPart::kRest, t);
  }
  hipError_t j = hipEventRecord(ev[1], t);
  if (j == hipSuccess) j = hipStreamWaitEvent(s, ev[1], 0);
  return e != hipSuccess ? e : j;
}

// pipeline: allow the two-stream build (ice_build_noalloc keeps to one stream)
int build_range(ice_index* idx, const void* K, const void* V, int32_t n_tokens, int64_t head_stride, int32_t h0,
                int32_t n_heads, void* ws, size_t ws_bytes, void* stream, const PdciArgs* pd,
                hipEvent_t* ev = nullptr, bool pipeline = true) {
  if (!idx) return fail(ICE_ERR_ARG, "index is null");
  const int H = idx->p.n_heads;
  if (h0 < 0 || n_heads < 1 || h0 > H - n_heads)
    return fail(ICE_ERR_ARG, "heads [%d, %d) outside [0, %d)", h0, h0 + n_heads, H);
  if (n_tokens < 0) return fail(ICE_ERR_ARG, "n_tokens must be >= 0");
  if (n_tokens > idx->p.capacity)
    return fail(ICE_ERR_CAPACITY, "n_tokens %d exceeds capacity %d", n_tokens, idx->p.capacity);
  bool any_built = false, range_built = true;
  for (int h = 0; h < H; ++h) any_built |= idx->head_built[h] != 0;
  for (int h = h0; h < h0 + n_heads; ++h) range_built &= idx->head_built[h] != 0;
  if (n_heads < H && any_built && n_tokens != idx->n_tokens)
    return fail(ICE_ERR_ARG, "every head holds %d tokens; a build of some heads must keep that count", idx->n_tokens);
  if (n_tokens > 0) {
    if (!K || !V) return fail(ICE_ERR_ARG, "K or V is null");
    if (head_stride < (int64_t)n_tokens * idx->p.d) return fail(ICE_ERR_ARG, "head_stride smaller than n_tokens*d");
    if (!aligned16(K) || !aligned16(V) || (head_stride * idx->L.elt) % 16 != 0)
      return fail(ICE_ERR_ARG, "K, V and the head stride must be 16-byte aligned");
  }
  if (!ws || ws_bytes < (size_t)idx->W.build_bytes)
    return fail(ICE_ERR_CAPACITY, "workspace has %zu bytes, build needs %lld", ws_bytes,
                (long long)idx->W.build_bytes);
  if (((uintptr_t)ws & 255u) != 0) return fail(ICE_ERR_ARG, "workspace must be 256-byte aligned");
  if (host_mode(idx->L) && !idx->L.vpool) return fail(ICE_ERR_STATE, "build before ice_attach_host_pool");
  // the range as an index of its own: blob, workspace and host pool start at
  // head h0, and the promotion draws use the absolute head numbers
  DevLayout L = idx->L;
  L.H = n_heads;
  L.h0 = h0;
  if (L.vpool) L.vpool += (int64_t)h0 * L.vpool_head_bytes;
  char* blob = static_cast<char*>(idx->blob) + (int64_t)h0 * L.head_bytes;
  char* wsr = static_cast<char*>(ws) + (int64_t)h0 * idx->W.head_bytes;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int chunks = pipeline && !pd && !ev && n_tokens > 0 ? build_chunks(idx, n_heads, s) : 1;
  hipError_t e = chunks > 1
                     ? build_pipelined(idx, L, blob, K, V, n_tokens, head_stride, wsr, range_built, s, chunks)
                     : launch_build(L, idx->W, blob, K, V, n_tokens, head_stride, wsr, range_built, s, pd, ev);
  if (e != hipSuccess) return hip_fail(e, "ice_build launch");
  if (!range_built)     // headers were cleared: no dense flags there any more
    for (int h = h0; h < h0 + n_heads; ++h) {
      idx->n_dense -= idx->dense[h];
      idx->dense[h] = 0;
    }
  for (int h = h0; h < h0 + n_heads; ++h) idx->head_built[h] = 1;
  note_own_build(idx, h0, n_heads, n_tokens);
  idx->n_tokens = n_tokens;
  bool all = true;
  for (int h = 0; h < H; ++h) all &= idx->head_built[h] != 0;
  idx->built = all;
  return ICE_OK;
}

}  // namespace

extern "C" {

int ice_build_heads(ice_index* idx, const void* K, const void* V, int32_t n_tokens, int64_t head_stride, int32_t h0,
                    int32_t n_heads, void* ws, size_t ws_bytes, void* stream) {
  return build_range(idx, K, V, n_tokens, head_stride, h0, n_heads, ws, ws_bytes, stream, nullptr);
}

int ice_build_pdci(ice_index* idx, const void* K, const void* V, int32_t n_tokens, int64_t head_stride,
                   const float* dirs, int32_t m, int32_t l, int32_t visits, int32_t cands, void* ws, size_t ws_bytes,
                   void* stream) {
  if (!idx) return fail(ICE_ERR_ARG, "index is null");
  if (l < 1 || l > ICE_PDCI_MAX_L || m < 1 || m * l > ICE_PDCI_MAX_KEYS)
    return fail(ICE_ERR_ARG, "P-DCI needs 1 <= l <= %d and 1 <= m, m*l <= %d", ICE_PDCI_MAX_L, ICE_PDCI_MAX_KEYS);
  if (visits < 1 || cands < 1) return fail(ICE_ERR_ARG, "visits and cands must be >= 1");
  if (!dirs) return fail(ICE_ERR_ARG, "dirs is null");
  const WsLayout& W = idx->W;
  if (!ws || ws_bytes < (size_t)(W.build_bytes + W.pdci_bytes))
    return fail(ICE_ERR_CAPACITY, "workspace has %zu bytes, a P-DCI build needs %lld", ws_bytes,
                (long long)(W.build_bytes + W.pdci_bytes));
  PdciArgs P;
  P.dirs = dirs;
  P.m = m;
  P.l = l;
  P.mk = m * l;
  P.visits = visits;
  P.cands = cands;
  P.stride = idx->p.levels >= 2 ? idx->L.ncap[1] : 0;
  const int64_t n_el = (int64_t)idx->p.n_heads * ICE_PDCI_MAX_KEYS * P.stride;
  char* base = static_cast<char*>(ws) + W.build_bytes;
  P.keys = reinterpret_cast<double*>(base);
  P.skeys = reinterpret_cast<double*>(base + n_el * 8);
  P.sidx = reinterpret_cast<int32_t*>(base + n_el * 16);
  P.posof = reinterpret_cast<int32_t*>(base + n_el * 20);
  return build_range(idx, K, V, n_tokens, head_stride, 0, idx->p.n_heads, ws, ws_bytes, stream, &P);
}

int ice_build_reuse(ice_index* idx, const void* K, const void* V, int32_t n_tokens, int64_t head_stride, int32_t h0,
                    int32_t n_heads, int32_t src_h0, void* ws, size_t ws_bytes, void* stream) {
  if (!idx) return fail(ICE_ERR_ARG, "index is null");
  const int H = idx->p.n_heads;
  if (h0 < 0 || n_heads < 1 || h0 > H - n_heads || src_h0 < 0 || src_h0 > H - n_heads)
    return fail(ICE_ERR_ARG, "heads [%d, %d) or source heads [%d, %d) outside [0, %d)", h0, h0 + n_heads, src_h0,
                src_h0 + n_heads, H);
  if (h0 < src_h0 + n_heads && src_h0 < h0 + n_heads) return fail(ICE_ERR_ARG, "head ranges overlap");
  for (int h = src_h0; h < src_h0 + n_heads; ++h)
    if (!idx->head_built[h]) return fail(ICE_ERR_STATE, "source head %d is not built", h);
  if (n_tokens != idx->n_tokens)
    return fail(ICE_ERR_ARG, "the source heads hold %d tokens, not %d", idx->n_tokens, n_tokens);
  if (n_tokens > 0) {
    if (!K || !V) return fail(ICE_ERR_ARG, "K or V is null");
    if (head_stride < (int64_t)n_tokens * idx->p.d) return fail(ICE_ERR_ARG, "head_stride smaller than n_tokens*d");
    if (!aligned16(K) || !aligned16(V) || (head_stride * idx->L.elt) % 16 != 0)
      return fail(ICE_ERR_ARG, "K, V and the head stride must be 16-byte aligned");
  }
  if (!ws || ws_bytes < (size_t)idx->W.build_bytes)
    return fail(ICE_ERR_CAPACITY, "workspace has %zu bytes, build needs %lld", ws_bytes,
                (long long)idx->W.build_bytes);
  if (((uintptr_t)ws & 255u) != 0) return fail(ICE_ERR_ARG, "workspace must be 256-byte aligned");
  bool range_built = true;
  for (int h = h0; h < h0 + n_heads; ++h) range_built &= idx->head_built[h] != 0;
  DevLayout L = idx->L;
  L.H = n_heads;
  L.h0 = h0;
  if (L.vpool) L.vpool += (int64_t)h0 * L.vpool_head_bytes;
  char* blob = static_cast<char*>(idx->blob) + (int64_t)h0 * L.head_bytes;
  const char* src = static_cast<const char*>(idx->blob) + (int64_t)src_h0 * L.head_bytes;
  char* wsr = static_cast<char*>(ws) + (int64_t)h0 * idx->W.head_bytes;
  hipError_t e = launch_build_reuse(L, idx->W, blob, src, K, V, n_tokens, head_stride, wsr, range_built,
                                    static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ice_build_reuse launch");
  if (!range_built)
    for (int h = h0; h < h0 + n_heads; ++h) {
      idx->n_dense -= idx->dense[h];
      idx->dense[h] = 0;
    }
  for (int h = h0; h < h0 + n_heads; ++h) {
    idx->head_built[h] = 1;
    // the layout, levels included, is the source's
    idx->runs[h] = idx->runs[src_h0 + (h - h0)];
    idx->ltop[h] = idx->ltop[src_h0 + (h - h0)];
  }
  bool all = true;
  for (int h = 0; h < H; ++h) all &= idx->head_built[h] != 0;
  idx->built = all;
  return ICE_OK;
}

int ice_build(ice_index* idx, const void* K, const void* V, int32_t n_tokens, int64_t head_stride, void* ws,
              size_t ws_bytes, void* stream) {
  if (!idx) return fail(ICE_ERR_ARG, "index is null");
  return ice_build_heads(idx, K, V, n_tokens, head_stride, 0, idx->p.n_heads, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up on the first
// call on that device (with it current) and kept for the process.
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "ice_build_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(ICE_ERR_ARG, "ice_build_noalloc: device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return hip_fail(e, "ice_build_noalloc: hipGetSymbolAddress(scratch)");
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return ICE_OK;
}

}  // namespace

extern "C" {

int ice_build_noalloc(ice_index* idx, const void* K, const void* V, int32_t n_tokens, int64_t head_stride,
                      void* stream) {
  if (!idx) return fail(ICE_ERR_ARG, "index is null");
  if (idx->W.build_bytes > (int64_t)ICE_NOALLOC_SCRATCH_BYTES)
    return fail(ICE_ERR_CAPACITY, "ice_build_noalloc: the build needs %lld bytes of scratch, the library holds %lld",
                (long long)idx->W.build_bytes, (long long)ICE_NOALLOC_SCRATCH_BYTES);
  void* ptr = nullptr;
  const int rc = scratch_address(&ptr);
  if (rc != ICE_OK) return rc;
  return build_range(idx, K, V, n_tokens, head_stride, 0, idx->p.n_heads, ptr, (size_t)ICE_NOALLOC_SCRATCH_BYTES,
                     stream, nullptr, nullptr, false);
}

int ice_build_timed(ice_index* idx, const void* K, const void* V, int32_t n_tokens, int64_t head_stride, void* ws,
                    size_t ws_bytes, void* stream, float* phase_ms) {
  if (!idx) return fail(ICE_ERR_ARG, "index is null");
  if (!phase_ms) return fail(ICE_ERR_ARG, "phase_ms is null");
  hipEvent_t ev[ICE_BUILD_PHASES + 1] = {};
  int rc = ICE_OK;
  hipError_t e = hipSuccess;
  int made = 0;
  for (; made <= ICE_BUILD_PHASES && e == hipSuccess; ++made) e = hipEventCreate(&ev[made]);
  if (e != hipSuccess) {
    --made;
    rc = hip_fail(e, "ice_build_timed event");
  } else {
    rc = build_range(idx, K, V, n_tokens, head_stride, 0, idx->p.n_heads, ws, ws_bytes, stream, nullptr, ev);
    if (rc == ICE_OK) {
      e = hipEventSynchronize(ev[ICE_BUILD_PHASES]);
      for (int i = 0; i < ICE_BUILD_PHASES && e == hipSuccess; ++i) e = hipEventElapsedTime(&phase_ms[i], ev[i], ev[i + 1]);
      if (e != hipSuccess) rc = hip_fail(e, "ice_build_timed timing");
    }
  }
  for (int i = 0; i < made; ++i) (void)hipEventDestroy(ev[i]);
  return rc;
}

int ice_insert(ice_index* idx, const void* k_new, const void* v_new, int32_t n_new, void* ws, size_t ws_bytes,
               void* stream) {
  (void)ws;
  (void)ws_bytes;
  if (!idx) return fail(ICE_ERR_ARG, "index is null");
  if (!idx->built) return fail(ICE_ERR_STATE, "insert before build");
  if (n_new < 0) return fail(ICE_ERR_ARG, "n_new must be >= 0");
  if (n_new == 0) return ICE_OK;
  if (!k_new || !v_new) return fail(ICE_ERR_ARG, "k_new or v_new is null");
  if (!aligned16(k_new)) return fail(ICE_ERR_ARG, "k_new must be 16-byte aligned");
  if ((int64_t)idx->n_tokens + n_new > idx->p.capacity)
    return fail(ICE_ERR_CAPACITY, "insert of %d tokens exceeds capacity %d (holds %d)", n_new, idx->p.capacity,
                idx->n_tokens);
  // A head built from its own draws stays within the tables sized from those
  // draws. A head built by reuse holds its source's levels for its first
  // tokens and its own after them, which can outgrow the tables: its level
  // counts after the insert are checked against their bounds first.
  const int32_t t_end = idx->n_tokens + n_new;
  for (int h = 0; h < idx->p.n_heads; ++h) {
    bool own = true;
    for (const auto& r : idx->runs[h]) own &= r.src == h;
    if (own) continue;
    for (int l = 1; l <= idx->ltop[h]; ++l) {
      const int64_t c = level_count(idx, h, l, t_end);
      if (c > idx->L.ncap[l])
        return fail(ICE_ERR_CAPACITY,
                    "head %d (built by reuse) would hold %lld tokens at level %d, its tables hold %d; nothing inserted",
                    h, (long long)c, l, idx->L.ncap[l]);
    }
  }
  hipError_t e = launch_insert(idx->L, idx->blob, k_new, v_new, n_new, idx->n_tokens,
                               static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ice_insert launch");
  for (int h = 0; h < idx->p.n_heads; ++h) {
    auto& rv = idx->runs[h];
    if (!rv.empty() && rv.back().src == h && rv.back().t1 == idx->n_tokens) rv.back().t1 = t_end;
    else rv.push_back({idx->n_tokens, t_end, h});
  }
  idx->n_tokens += n_new;
  return ICE_OK;
}

int ice_select(const ice_index* idx, const void* Q, int32_t budget_tokens, int32_t beam, int32_t* sel,
               int32_t* uni, int32_t* n_uni, int32_t* trace, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  if (!idx) return fail(ICE_ERR_ARG, "index is null");
  if (!idx->built) return fail(ICE_ERR_STATE, "select before build");
  int rc = check_budget(idx, budget_tokens);
  if (rc) return rc;
  if (beam < 1 || beam > ICE_MAX_BEAM) return fail(ICE_ERR_ARG, "beam must be in [1, %d]", ICE_MAX_BEAM);
  if (!Q || !sel || !uni || !n_uni) return fail(ICE_ERR_ARG, "Q, sel, uni or n_uni is null");
  if (!aligned16(Q)) return fail(ICE_ERR_ARG, "Q must be 16-byte aligned");
  hipError_t e = launch_select(idx->L, idx->blob, Q, budget_tokens, beam, sel, uni, n_uni, trace,
                               static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ice_select launch");
  return ICE_OK;
}

int ice_attend(const ice_index* idx, const void* Q, const int32_t* uni, const int32_t* n_uni, int32_t uni_stride,
               float scale, float* O, float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (!idx) return fail(ICE_ERR_ARG, "index is null");
  if (!idx->built) return fail(ICE_ERR_STATE, "attend before build");
  if (!Q || !uni || !n_uni || !O) return fail(ICE_ERR_ARG, "Q, uni, n_uni or O is null");
  if (uni_stride < 1 || uni_stride > ICE_MAX_GROUP * ICE_MAX_BEAM)
    return fail(ICE_ERR_ARG, "uni_stride must be in [1, %d]", ICE_MAX_GROUP * ICE_MAX_BEAM);
  const int64_t need = attend_ws_bytes(idx->L, uni_stride);
  if (need > 0 && (!ws || ws_bytes < (size_t)need))
    return fail(ICE_ERR_CAPACITY, "workspace has %zu bytes, attend needs %lld", ws_bytes, (long long)need);
  if (need > 0 && ((uintptr_t)ws & 255u) != 0) return fail(ICE_ERR_ARG, "workspace must be 256-byte aligned");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const DevLayout A = attend_layout(idx->L, ws, uni_stride);
  hipError_t e = hipSuccess;
  if (host_mode(idx->L)) e = launch_gather_v(A, idx->blob, uni, n_uni, uni_stride, s);
  if (e == hipSuccess) e = launch_attend(A, idx->blob, Q, uni, n_uni, uni_stride, scale, O, lse, ws, s);
  if (e != hipSuccess) return hip_fail(e, "ice_attend launch");
  return ICE_OK;
}
int ice_set_resident(ice_index* idx, const void* K, const void* V, int32_t n, int64_t head_stride, void* stream) {
  if (!idx) return fail(ICE_ERR_ARG, "index is null");
  if (!idx->built) return fail(ICE_ERR_STATE, "resident tokens before build");
  if (n < 0 || n > idx->p.resident) return fail(ICE_ERR_ARG, "n must be in [0, %d] (params.resident)", idx->p.resident);
  if (n > 0) {
    if (!K || !V) return fail(ICE_ERR_ARG, "K or V is null");
    if (head_stride < (int64_t)n * idx->p.d) return fail(ICE_ERR_ARG, "head_stride must be >= n*d");
    if (!aligned16(K) || !aligned16(V) || (head_stride * idx->L.elt) % 16 != 0)
      return fail(ICE_ERR_ARG, "K, V and the head stride must be 16-byte aligned");
  }
  if (idx->L.res_pages == 0) return ICE_OK;   // nothing resident, nothing to clear
  hipError_t e = launch_set_resident(idx->L, idx->blob, K, V, n, head_stride, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ice_set_resident launch");
  return ICE_OK;
}

int ice_set_dense(ice_index* idx, const uint8_t* dense, void* stream) {
  if (!idx) return fail(ICE_ERR_ARG, "index is null");
  if (!idx->built) return fail(ICE_ERR_STATE, "dense flags before build");
  std::vector<int32_t> flags(idx->p.n_heads, 0);
  int n_dense = 0;
  if (dense)
    for (int h = 0; h < idx->p.n_heads; ++h) n_dense += (flags[h] = dense[h] ? 1 : 0);
  if (n_dense > 0 && host_mode(idx->L)) return fail(ICE_ERR_ARG, "dense heads need the device V pool (no ICE_HOST_POOL)");
  // the stream's earlier work finishes first, then one strided copy into the headers
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e == hipSuccess)
    e = hipMemcpy2D(static_cast<char*>(idx->blob) + idx->L.off_hdr + offsetof(Hdr, dense), (size_t)idx->L.head_bytes,
                    flags.data(), sizeof(int32_t), sizeof(int32_t), (size_t)idx->p.n_heads, hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(e, "ice_set_dense copy");
  idx->n_dense = n_dense;
  for (int h = 0; h < idx->p.n_heads; ++h) idx->dense[h] = (uint8_t)flags[h];
  return ICE_OK;
}

int ice_decode(const ice_index* idx, const void* Q, int32_t budget_tokens, int32_t beam, int32_t* sel, int32_t* uni,
               int32_t* n_uni, float scale, float* O, float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (!idx) return fail(ICE_ERR_ARG, "index is null");
  if (!idx->built) return fail(ICE_ERR_STATE, "decode before build");
  int rc = check_budget(idx, budget_tokens);
  if (rc) return rc;
  if (beam < 1 || beam > ICE_MAX_BEAM) return fail(ICE_ERR_ARG, "beam must be in [1, %d]", ICE_MAX_BEAM);
  if (!Q || !sel || !uni || !n_uni || !O) return fail(ICE_ERR_ARG, "Q, sel, uni, n_uni or O is null");
  if (!aligned16(Q)) return fail(ICE_ERR_ARG, "Q must be 16-byte aligned");
  const int uni_stride = idx->p.group * (budget_tokens / ICE_PAGE_CAP);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (!host_mode(idx->L) && idx->n_dense == 0 && decode_fused(idx->L, budget_tokens, beam)) {
    hipError_t e = launch_decode(idx->L, idx->blob, Q, budget_tokens, beam, sel, uni, n_uni, scale, O, lse, s);
    if (e != hipSuccess) return hip_fail(e, "ice_decode launch");
    return ICE_OK;
  }
  const int64_t need = attend_ws_bytes(idx->L, uni_stride);
  if (need > 0 && (!ws || ws_bytes < (size_t)need))
    return fail(ICE_ERR_CAPACITY, "workspace has %zu bytes, attend needs %lld", ws_bytes, (long long)need);
  if (need > 0 && ((uintptr_t)ws & 255u) != 0) return fail(ICE_ERR_ARG, "workspace must be 256-byte aligned");
  hipError_t e = launch_select(idx->L, idx->blob, Q, budget_tokens, beam, sel, uni, n_uni, nullptr, s);
  if (e != hipSuccess) return hip_fail(e, "ice_decode select launch");
  const DevLayout A = attend_layout(idx->L, ws, uni_stride);
  if (host_mode(idx->L)) {
    e = launch_gather_v(A, idx->blob, uni, n_uni, uni_stride, s);
    if (e != hipSuccess) return hip_fail(e, "ice_decode gather launch");
  }
  e = launch_attend(A, idx->blob, Q, uni, n_uni, uni_stride, scale, O, lse, ws, s);
  if (e != hipSuccess) return hip_fail(e, "ice_decode attend launch");
  return ICE_OK;
}

size_t ice_export_bytes(const ice_index* idx, int32_t what, int32_t level) {
  if (!idx) return 0;
  const DevLayout& L = idx->L;
  const int64_t cap = L.cap, elt = L.elt, d = L.d;
  const bool tab_ok = level >= 0 && level < L.ntab;
  switch (what) {
    case ICE_EXP_LEVEL: return cap;
    case ICE_EXP_LIFT: return cap * 4;
    case ICE_EXP_PARENT: return tab_ok ? cap * 4 : 0;
    case ICE_EXP_PAGE_TOK: return tab_ok ? (size_t)L.pcap[level] * ICE_PAGE_CAP * 4 : 0;
    case ICE_EXP_PAGE_CNT:
    case ICE_EXP_PAGE_NEXT:
    case ICE_EXP_PAGE_OWNER: return tab_ok ? (size_t)L.pcap[level] * 4 : 0;
    case ICE_EXP_OWNER_FIRST:
    case ICE_EXP_OWNER_TAIL:
    case ICE_EXP_OWNER_RUN:
    case ICE_EXP_OWNER_COUNT: return tab_ok ? (cap + 1) * 4 : 0;
    case ICE_EXP_TOP: return (size_t)L.topcap * 4;
    case ICE_EXP_PAGE_K: return tab_ok ? (size_t)L.pcap[level] * ICE_PAGE_CAP * d * elt : 0;
    case ICE_EXP_PAGE_V: return level == 0 ? (size_t)L.pcap[0] * ICE_PAGE_CAP * d * elt : 0;
    case ICE_EXP_HEADER: return sizeof(ice_head_stats);
    default: return 0;
  }
}

int ice_export(const ice_index* idx, int32_t head, int32_t what, int32_t level, void* dst, size_t dst_bytes,
               void* stream) {
  if (!idx || !dst) return fail(ICE_ERR_ARG, "index or dst is null");
  if (head < 0 || head >= idx->p.n_heads) return fail(ICE_ERR_ARG, "head out of range");
  const size_t n = ice_export_bytes(idx, what, level);
  if (n == 0) return fail(ICE_ERR_ARG, "nothing to export for what=%d level=%d", what, level);
  if (dst_bytes < n) return fail(ICE_ERR_ARG, "dst has %zu bytes, needs %zu", dst_bytes, n);
  const DevLayout& L = idx->L;
  int64_t off = 0;
  switch (what) {
    case ICE_EXP_LEVEL: off = L.off_lev; break;
    case ICE_EXP_LIFT: off = L.off_e; break;
    case ICE_EXP_PARENT: off = L.off_parent[level]; break;
    case ICE_EXP_PAGE_TOK: off = L.off_pg_tok[level]; break;
    case ICE_EXP_PAGE_CNT: off = L.off_pg_cnt[level]; break;
    case ICE_EXP_PAGE_NEXT: off = L.off_pg_next[level]; break;
    case ICE_EXP_PAGE_OWNER: off = L.off_pg_owner[level]; break;
    case ICE_EXP_OWNER_FIRST: off = L.off_first[level]; break;
    case ICE_EXP_OWNER_TAIL: off = L.off_tail[level]; break;
    case ICE_EXP_OWNER_RUN: off = L.off_orun[level]; break;
    case ICE_EXP_OWNER_COUNT: off = L.off_ocnt[level]; break;
    case ICE_EXP_TOP: off = L.off_top_tok; break;
    case ICE_EXP_PAGE_K: off = L.off_pgK[level]; break;
    case ICE_EXP_PAGE_V: off = L.off_pgV; break;
    case ICE_EXP_HEADER: off = L.off_hdr; break;
    default: return fail(ICE_ERR_ARG, "unknown export %d", what);
  }
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ice_export sync");
  const char* src = static_cast<const char*>(idx->blob) + (int64_t)head * L.head_bytes + off;
  if (what == ICE_EXP_PAGE_V && host_mode(L)) {
    if (!idx->host_pool) return fail(ICE_ERR_STATE, "no host pool attached");
    src = static_cast<const char*>(idx->host_pool) + (int64_t)head * L.vpool_head_bytes;
  }
  if (what != ICE_EXP_PAGE_V) {
    e = hipMemcpy(dst, src, n, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "ice_export copy");
    return ICE_OK;
  }
  // V pages are stored [page][slot group][dim][4 slots]; hand them out as
  // [page][slot][dim] rows
  std::vector<char> raw(n);
  e = hipMemcpy(raw.data(), src, n, host_mode(L) ? hipMemcpyHostToHost : hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "ice_export copy");
  const int64_t elt = L.elt, D = L.d, pages = (int64_t)n / (ICE_PAGE_CAP * D * elt);
  char* out = static_cast<char*>(dst);
  for (int64_t pg = 0; pg < pages; ++pg)
    for (int sl = 0; sl < ICE_PAGE_CAP; ++sl)
      for (int64_t dd = 0; dd < D; ++dd)
        memcpy(out + ((pg * ICE_PAGE_CAP + sl) * D + dd) * elt,
                    raw.data() + (((pg * 4 + sl / 4) * D + dd) * 4 + sl % 4) * elt, elt);
  return ICE_OK;
}

}  // extern "C"
