// Decode-time page selection: beam descent through the levels, top-k pages
// per query head, union over the GQA group.
//
// Follows the papernotes.org IceCache notes, key design 2 (search: the k
// nearest points at the top level, then recurse into their children level by
// level) and key design 3 (each head selects its own top-k pages; query heads
// that share a KV head use the union of their pages), and the aitangshan.cn
// IceCache article, section 6 (the union over a GQA group). With the query
// lifted as [q, 0], the lifted distance |q|^2 + M^2 - 2 q.k ranks exactly like
// q.k descending, which is what is scored. A page scores its best token.
//
// One block per head; each of its G query heads gets W waves (W = 4 for
// G <= 4, else 16/G). At every level a query's candidate rows are split over
// its waves: a wave scores 16 rows per pass with 4 lanes per row (bf16 dot2 on
// gfx950), issuing the loads of several 16-row groups before any arithmetic.
// Keys pack (score, ~id) into 64 bits, so "score descending, id ascending" is
// plain unsigned order. Each wave keeps its top list in registers, one key per
// lane: a chunk of 64 candidates is bitonic-sorted across the wave (ascending)
// and merged by taking max(list[i], chunk[i]) (the 64 largest of both, as a
// bitonic sequence) followed by a 6-step bitonic merge; the W lists of a
// query (at most 64 keys together) are read into one wave as bitonic runs and
// merged in 11 steps. A compare-exchange step is one lane exchange (DPP or
// permlane swap), one 64-bit compare and two selects on the VALU. Lists
// longer than 64 keys (beams or budgets beyond 64 entries)
// use a slower LDS list instead. The block ends with the union of its query
// heads' pages, ascending.
#include "ice_launch.h"
#include "attend_mfma.h"

#include <type_traits>

namespace ice {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxWaves = 16;

// Waves per query head: 16 waves per block, which fill a CU's registers (128
// VGPRs per wave), so each head's block runs on a CU of its own. With more
// heads than CUs such blocks run in rounds; launch_waves then halves the
// waves per query head when two blocks' LDS fits one CU, so that two heads
// share each CU and every head runs at once. The kernels take their wave
// count from the block size.
__host__ __device__ inline int waves_per_query(int G) { return G <= 4 ? 4 : 16 / G; }
constexpr int kCuLds = 160 * 1024;

// the device's compute units (current device, looked up once per device)
int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Waves of a selection block: waves_per_query(G) per query head, or half as
// many when the heads outnumber the CUs and lds(nw) bytes fit twice in a CU.
template <class LdsOf>
int launch_waves(const DevLayout& L, LdsOf lds) {
  const int w = waves_per_query(L.G);
  if (L.H > cu_count() && w >= 2 && 2 * lds((w / 2) * L.G) <= kCuLds) return (w / 2) * L.G;
  return w * L.G;
}
// LDS slots of the union's sort: the next power of two
__host__ __device__ inline int union_pad(int n) {
  int p = 64;
  while (p < n) p <<= 1;
  return p;
}

// ---- scoring geometry: 4 lanes per row, 16 rows per wave pass -------------
template <int D, class T>
struct Quarter {
  static constexpr int ROWB = D * (int)sizeof(T);
  static constexpr int NL = ROWB / 64;                // 16-byte loads per lane per row
  static constexpr int GB = NL >= 4 ? 2 : 4;          // row groups per load batch (keeps 128 VGPRs)
  static constexpr int GB0 = NL == 4 ? 3 : GB;        // pages per level-0 batch (keeps 128 VGPRs)
  V4 q[NL];
  int part;

  __device__ inline void load(const T* qrow, int lane) {
    part = lane & 3;
#pragma unroll
    for (int i = 0; i < NL; ++i)
      q[i] = *reinterpret_cast<const V4*>(reinterpret_cast<const char*>(qrow) + part * 16 + i * 64);
  }
  // this lane's 16-byte pieces part, part + 4, ... of `row` (the row's 4 lanes
  // read one contiguous 64-byte segment per load), or zeros when `ok` is false
  __device__ inline void fetch(bool ok, const T* row, V4* out) const {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      out[i] = V4{0, 0, 0, 0};
      if (ok) out[i] = *reinterpret_cast<const V4*>(reinterpret_cast<const char*>(row) + part * 16 + i * 64);
    }
  }
  // q.row from this lane's quarter, summed over the row's 4 lanes
  __device__ inline float dot(const V4* k) const {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      if constexpr (sizeof(T) == 2) {
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k[i].x), __builtin_bit_cast(bf16x2, q[i].x), s, false);
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k[i].y), __builtin_bit_cast(bf16x2, q[i].y), s, false);
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k[i].z), __builtin_bit_cast(bf16x2, q[i].z), s, false);
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k[i].w), __builtin_bit_cast(bf16x2, q[i].w), s, false);
      } else {
        s = fmaf(__uint_as_float(k[i].x), __uint_as_float(q[i].x), s);
        s = fmaf(__uint_as_float(k[i].y), __uint_as_float(q[i].y), s);
        s = fmaf(__uint_as_float(k[i].z), __uint_as_float(q[i].z), s);
        s = fmaf(__uint_as_float(k[i].w), __uint_as_float(q[i].w), s);
      }
    }
    s += xor_lane_f<1>(s);
    s += xor_lane_f<2>(s);
    return s;
  }
};

// max over the 16 rows of a pass (lanes 4r + part)
__device__ inline float rows_max(float s) {
  s = fmaxf(s, xor_lane_f<4>(s));
  s = fmaxf(s, xor_lane_f<8>(s));
  s = fmaxf(s, xor_lane_f<16>(s));
  s = fmaxf(s, xor_lane_f<32>(s));
  return s;
}

__device__ inline uint64_t shfl64(uint64_t v, int src) {
  const int lo = __shfl((int)(uint32_t)v, src, 64), hi = __shfl((int)(uint32_t)(v >> 32), src, 64);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ inline uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Lane masks of the networks, as compile-time constants: bit i is lane i's
// flag. The compare-exchanges take them through inverse ballots, so a
// direction costs one scalar operation and no vector work.
__host__ __device__ constexpr uint64_t lanes_where_zero(int m) {      // (lane & m) == 0
  uint64_t r = 0;
  for (int i = 0; i < 64; ++i)
    if ((i & m) == 0) r |= 1ull << i;
  return r;
}
// step (k, j) of a bitonic sort keeps the larger key where (lane & k) == 0
// and (lane & j) == 0 agree (blocks of k lanes alternate direction)
__host__ __device__ constexpr uint64_t sort_keep_max(int k, int j) {
  return ~(lanes_where_zero(k) ^ lanes_where_zero(j));
}

// Compare-exchange of lanes i and i ^ j: a lane whose bit is set in
// `keep_max` (a wave-uniform mask) keeps the larger of its key and its
// partner's, the other the smaller. For j = 16, 32 the permlane swap leaves
// the pair's two keys in (a, b) of both lanes, in the same order, which is
// all a compare-exchange needs.
template <int j>
__device__ inline uint64_t cx64(uint64_t x, uint64_t keep_max) {
  uint64_t a = x, b;
  if constexpr (j >= 16) {
    const int lo = (int)(uint32_t)x, hi = (int)(uint32_t)(x >> 32);
    int pl0, pl1, ph0, ph1;
    if constexpr (j == 16) {
      const auto pl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
      const auto ph = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
      pl0 = pl[0]; pl1 = pl[1]; ph0 = ph[0]; ph1 = ph[1];
    } else {
      static_assert(j == 32, "exchange distance");
      const auto pl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
      const auto ph = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
      pl0 = pl[0]; pl1 = pl[1]; ph0 = ph[0]; ph1 = ph[1];
    }
    a = ((uint64_t)(uint32_t)ph0 << 32) | (uint32_t)pl0;
    b = ((uint64_t)(uint32_t)ph1 << 32) | (uint32_t)pl1;
  } else {
    b = xor_lane_u64<j>(x);
  }
  return (a > b) == __builtin_amdgcn_inverse_ballot_w64(keep_max) ? a : b;
}
// step (k, j) of a bitonic sort; flip = 0 sorts descending, ~0 ascending
template <int k, int j>
__device__ inline uint64_t sort_step(uint64_t x, uint64_t flip) {
  return cx64<j>(x, sort_keep_max(k, j) ^ flip);
}
// Sorts one key per lane across the wave: descending (lane 0 largest) when
// `desc` (wave-uniform), else ascending.
__device__ inline uint64_t wave_sort(uint64_t x, bool desc) {
  const uint64_t flip = __builtin_amdgcn_readfirstlane((int)desc) ? 0ull : ~0ull;
  x = sort_step<2, 1>(x, flip);
  x = sort_step<4, 2>(x, flip);
  x = sort_step<4, 1>(x, flip);
  x = sort_step<8, 4>(x, flip);
  x = sort_step<8, 2>(x, flip);
  x = sort_step<8, 1>(x, flip);
  x = sort_step<16, 8>(x, flip);
  x = sort_step<16, 4>(x, flip);
  x = sort_step<16, 2>(x, flip);
  x = sort_step<16, 1>(x, flip);
  x = sort_step<32, 16>(x, flip);
  x = sort_step<32, 8>(x, flip);
  x = sort_step<32, 4>(x, flip);
  x = sort_step<32, 2>(x, flip);
  x = sort_step<32, 1>(x, flip);
  x = sort_step<64, 32>(x, flip);
  x = sort_step<64, 16>(x, flip);
  x = sort_step<64, 8>(x, flip);
  x = sort_step<64, 4>(x, flip);
  x = sort_step<64, 2>(x, flip);
  x = sort_step<64, 1>(x, flip);
  return x;
}
// Sorts lanes 0..15 descending (10 steps; the other lanes are sorted in
// 16-lane blocks of their own).
__device__ inline uint64_t sort16_desc(uint64_t x) {
  x = sort_step<2, 1>(x, 0ull);
  x = sort_step<4, 2>(x, 0ull);
  x = sort_step<4, 1>(x, 0ull);
  x = sort_step<8, 4>(x, 0ull);
  x = sort_step<8, 2>(x, 0ull);
  x = sort_step<8, 1>(x, 0ull);
  x = sort_step<16, 8>(x, 0ull);
  x = sort_step<16, 4>(x, 0ull);
  x = sort_step<16, 2>(x, 0ull);
  x = sort_step<16, 1>(x, 0ull);
  return x;
}
// Sorts a bitonic sequence across the wave, descending.
__device__ inline uint64_t bitonic_merge_desc(uint64_t t) {
  t = cx64<32>(t, lanes_where_zero(32));
  t = cx64<16>(t, lanes_where_zero(16));
  t = cx64<8>(t, lanes_where_zero(8));
  t = cx64<4>(t, lanes_where_zero(4));
  t = cx64<2>(t, lanes_where_zero(2));
  t = cx64<1>(t, lanes_where_zero(1));
  return t;
}
// Top 64 of a descending list and an ascending chunk, descending: their
// lane-wise maximum holds the 64 largest as a bitonic sequence.
__device__ inline uint64_t wave_merge(uint64_t list_desc, uint64_t chunk_asc) {
  return bitonic_merge_desc(umax64(list_desc, chunk_asc));
}
// Merges the descending lists of W waves (W = 2 or 4, at most 64 / W keys
// each; list w at lists + 64 w) into one descending list. The lists sit side
// by side in segments of 64 / W lanes, every second one read backwards, so
// each pair of segments is a bitonic sequence.
__device__ inline uint64_t merge_lists(const uint64_t* lists, int W, int lane) {
  if (W == 4) {
    const int sg = lane >> 4, i = lane & 15;
    uint64_t x = lists[sg * 64 + ((sg & 1) ? 15 - i : i)];
    // pairs of segments into 32-lane runs, the first descending, the second ascending
    x = cx64<16>(x, sort_keep_max(32, 16));
    x = cx64<8>(x, sort_keep_max(32, 8));
    x = cx64<4>(x, sort_keep_max(32, 4));
    x = cx64<2>(x, sort_keep_max(32, 2));
    x = cx64<1>(x, sort_keep_max(32, 1));
    return bitonic_merge_desc(x);
  }
  const int sg = lane >> 5, i = lane & 31;
  return bitonic_merge_desc(lists[sg * 64 + (sg ? 31 - i : i)]);
}

// ---- LDS layout ------------------------------------------------------------
// Per wave: its LDS top list (long lists only), a chunk of 64 keys and the 64
// (page, valid rows) pairs of the current round. Per query head: the owner
// table of its kept list (page offsets, first page, run and last-page count)
// and, for long lists, the merged list. Then small counters and the union's
// sort area.
struct SelLds {
  int lcap;           // list capacity = max(beam, pages per query)
  int wave_bytes;
  int off_comb;       // register lists: [kMaxWaves][64] u64
  int off_query;      // LDS lists: [G][lcap] u64 merged lists
  int off_meta;       // [G][meta_ints] owner tables
  int meta_ints;
  int off_misc;       // wn[kMaxWaves], qn[ICE_MAX_GROUP], qp[ICE_MAX_GROUP], qbar[ICE_MAX_GROUP]
  int off_sel;        // [G * kpg rounded up to a power of two] i32: selections, then the union's sort
  int total;
};

__host__ __device__ inline SelLds sel_lds(int G, int lcap, int kpg, bool big) {
  SelLds s;
  s.lcap = lcap;
  s.wave_bytes = (big ? lcap * 8 : 0) + 64 * 8 + 2 * 64 * 4;
  s.off_comb = kMaxWaves * s.wave_bytes;
  s.off_query = s.off_comb + (big ? 0 : kMaxWaves * 64 * 8);
  s.off_meta = s.off_query + (big ? G * lcap * 8 : 0);
  s.meta_ints = 3 * lcap + 2;
  s.off_misc = s.off_meta + G * s.meta_ints * 4;
  s.off_sel = s.off_misc + (kMaxWaves + 3 * ICE_MAX_GROUP) * 4;
  s.total = s.off_sel + union_pad(G * kpg) * 4;
  return s;
}

struct WaveArea {
  uint64_t* list;      // LDS top list, lcap keys (long lists only)
  uint64_t* chunk;     // 64 keys
  int32_t* cand;       // page ids of the round
  int32_t* cval;       // their valid rows
};

__device__ inline WaveArea wave_area(char* smem, const SelLds& S, int wv, bool big) {
  char* b = smem + wv * S.wave_bytes;
  WaveArea a;
  a.list = reinterpret_cast<uint64_t*>(b);
  a.chunk = a.list + (big ? S.lcap : 0);
  a.cand = reinterpret_cast<int32_t*>(a.chunk + 64);
  a.cval = a.cand + 64;
  return a;
}

// the owner table of a query head's kept list: off[i] = first page index of
// kept owner i among the query's pages (off[n] = their total), fst[i] = its
// first page, rl[i] = (pages in its build run) * 32 + (rows of its last page)
struct OwnerTable {
  int32_t* off;
  int32_t* fst;
  int32_t* rl;
};

__device__ inline OwnerTable owner_table(char* smem, const SelLds& S, int g) {
  int32_t* m = reinterpret_cast<int32_t*>(smem + S.off_meta) + g * S.meta_ints;
  return OwnerTable{m, m + S.lcap + 1, m + 2 * S.lcap + 1};
}

__device__ inline uint64_t readlane64(uint64_t v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

__device__ inline int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(v, d, 64);
    if (lane >= d) v += y;
  }
  return v;
}

// Barrier of the W waves of one query head: an LDS arrival counter that only
// grows (each wave waits for its target, W more per barrier). The wait is
// bounded: past kSpinLimit polls it counts a timeout in the head's header and
// goes on, so the kernel always ends.
constexpr int kSpinLimit = 1 << 20;

__device__ inline void query_sync(int* ctr, int& target, int W, int* timeouts) {
  target += W;
  if (W == 1) {
    wave_sync();
    return;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  if (__lane_id() == 0) atomicAdd(ctr, 1);
  int spins = 0;
  while (__atomic_load_n(ctr, __ATOMIC_RELAXED) < target) {
    if (++spins > kSpinLimit) {
      if (__lane_id() == 0) atomicAdd(timeouts, 1);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// ---- wave top lists --------------------------------------------------------
// Register list (cap <= 64): lane i holds entry i, 0 = empty.
struct RegTop {
  uint64_t L;
  int cap, n;
  __device__ inline void init(int c) {
    L = 0ull;
    cap = c;
    n = 0;
  }
  __device__ inline void push(const WaveArea&, uint64_t x, int lane) {
    const uint64_t thr = n == cap ? readlane64(L, cap - 1) : 0ull;
    const uint64_t live = __ballot(x > thr);
    if (live == 0) return;
    // the first chunk is sorted descending into the list, later ones
    // ascending and merged with it
    uint64_t t = wave_sort(x, n == 0);
    if (n > 0) t = wave_merge(L, t);
    L = lane < cap ? t : 0ull;
    n = min(cap, n + __popcll(live));
  }
  // First push of at most 16 keys, in lanes 0..15 (the other lanes empty).
  __device__ inline void push16(uint64_t x, int lane) {
    const uint64_t live = __ballot(x != 0ull);
    if (live == 0) return;
    const uint64_t t = sort16_desc(x);
    L = lane < cap ? t : 0ull;
    n = min(cap, __popcll(live));
  }
};

// LDS list (any cap up to ICE_MAX_BEAM), sorted descending. A push ranks
// every entry of the list and of the chunk within their union and rewrites
// the list in place (all reads happen before the writes).
struct LdsTop {
  int n, cap;
  __device__ inline void init(int c) {
    n = 0;
    cap = c;
  }
  __device__ void push(const WaveArea& a, uint64_t x, int lane) {
    a.chunk[lane] = x;
    wave_sync();
    uint64_t* Lc = a.list;
    const uint64_t thr = n == cap ? Lc[cap - 1] : 0ull;
    const bool live = x > thr;
    const uint64_t live_mask = __ballot(live);
    if (live_mask == 0) {
      wave_sync();
      return;
    }
    int rc = 0;
    for (int j = 0; j < 64; ++j) rc += a.chunk[j] > x;
    int lo = 0, hi = n;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (Lc[mid] > x) lo = mid + 1;
      else hi = mid;
    }
    uint64_t y[ICE_MAX_BEAM / 64];
    int c[ICE_MAX_BEAM / 64];
#pragma unroll
    for (int k = 0; k < ICE_MAX_BEAM / 64; ++k) {
      const int i = lane + 64 * k;
      y[k] = i < n ? Lc[i] : 0ull;
      c[k] = 0;
      if (i < n)
        for (int j = 0; j < 64; ++j) c[k] += a.chunk[j] > y[k];
    }
    wave_sync();
#pragma unroll
    for (int k = 0; k < ICE_MAX_BEAM / 64; ++k) {
      const int i = lane + 64 * k;
      if (i < n && i + c[k] < cap) Lc[i + c[k]] = y[k];
    }
    if (live && lo + rc < cap) Lc[lo + rc] = x;
    n = min(cap, n + __popcll(live_mask));
    wave_sync();
  }
};

// Page (level-0) keys: the low word is (~page << 5) | valid rows, so equal
// scores still rank by ascending page id and a selected page's row count
// comes with it (page ids stay below 2^27, rows 1 .. 16).
__device__ inline uint32_t page_key_lo(int pg, int rows) { return ((~(uint32_t)pg) << 5) | (uint32_t)rows; }
__device__ inline int32_t key_page(uint64_t k) { return (int32_t)(0x07ffffffu - ((uint32_t)k >> 5)); }
__device__ inline int32_t key_rows(uint64_t k) { return (int32_t)(k & 31u); }

// v[lane] = val for one lane: v_writelane_b32, a vector-register write of a
// scalar value (val and lane are wave-uniform; the lane index goes through
// m0, which this code uses for nothing else)
__device__ inline void write_lane(uint32_t& v, uint32_t val, int lane) {
  const int l = __builtin_amdgcn_readfirstlane(lane);
  const uint32_t x = (uint32_t)__builtin_amdgcn_readfirstlane((int)val);
  asm volatile("s_mov_b32 m0, %2\n\tv_writelane_b32 %0, %1, m0" : "+v"(v) : "s"(x), "s"(l) : "m0");
}

// number of keys greater than x in a descending list of n keys
__device__ inline int count_greater(const uint64_t* l, int n, uint64_t x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (l[mid] > x) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// Fills the wave's cand/cval with its pages of round t0: the query head's
// pages (all pages of its kept owners, owner by owner) are dealt to its W
// waves round-robin, wave j taking pages j, j + W, ...; lane l takes the
// wave's page t0 + l. An owner's pages are all full except its last; the
// pages of the build form one contiguous run from its first page, so only
// pages split off later by inserts are reached through next[]. Returns the
// number of pages of the round.
__device__ inline int deal_pages(const WaveArea& a, const OwnerTable& T, int n_own, int P, int j, int W, int t0,
                                 const int32_t* next, int lane) {
  const int mine = P > j ? (P - j + W - 1) / W : 0;
  const int nb = min(64, mine - t0);
  if (nb <= 0) return 0;
  if (lane < nb) {
    const int p = j + W * (t0 + lane);
    int lo = 0, hi = n_own - 1;      // last owner whose first page index is <= p
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (T.off[mid] <= p) lo = mid;
      else hi = mid - 1;
    }
    const int k = p - T.off[lo], np = T.off[lo + 1] - T.off[lo];
    const int run = max(1, T.rl[lo] >> 5), last = T.rl[lo] & 31;
    int pg = T.fst[lo] + min(k, run - 1);
    for (int s = run; s <= k; ++s) pg = next[pg];
    a.cand[lane] = pg;
    a.cval[lane] = k < np - 1 ? ICE_PAGE_CAP : last;
  }
  wave_sync();
  return nb;
}

// Keys of 4 row groups, one candidate per lane: group g, row r -> lane 16g + r.
// `ok[g]` is per lane (its row of group g), `row[g]` that row, `tok[g]` its id.
template <int D, class T>
__device__ inline uint64_t chunk_keys(const Quarter<D, T>& qs, const bool (&ok)[4], const T* const (&row)[4],
                                      const int (&tok)[4], int lane) {
  using QG = Quarter<D, T>;
  uint64_t key[4];
#pragma unroll
  for (int g0 = 0; g0 < 4; g0 += QG::GB) {
    V4 buf[QG::GB][QG::NL];
#pragma unroll
    for (int b = 0; b < QG::GB; ++b) qs.fetch(ok[g0 + b], row[g0 + b], buf[b]);
#pragma unroll
    for (int b = 0; b < QG::GB; ++b) {
      const float s = qs.dot(buf[b]);
      key[g0 + b] = ok[g0 + b] ? make_key(s, tok[g0 + b]) : 0ull;
    }
  }
  const int src = (lane & 15) * 4, grp = lane >> 4;
  const uint64_t x0 = shfl64(key[0], src), x1 = shfl64(key[1], src);
  const uint64_t x2 = shfl64(key[2], src), x3 = shfl64(key[3], src);
  return grp == 0 ? x0 : grp == 1 ? x1 : grp == 2 ? x2 : x3;
}

// The union of tot <= 64 selections (sel_all, LDS) by one wave: a 64-lane
// bitonic sort, then the first of each run of equal ids; writes urow
// (ascending, -1 padded to tot) and uni_lds (nullable). Returns its size.
__device__ inline int wave_union64(int tot, const int32_t* sel_all, int32_t* urow, int32_t* uni_lds, int lane) {
  int v = lane < tot ? sel_all[lane] : INT_MAX;
  if (v < 0) v = INT_MAX;
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      const int y = __shfl_xor(v, jj, 64);
      v = (((lane & k) == 0) == ((lane & jj) == 0)) ? min(v, y) : max(v, y);
    }
  }
  const int prev = __shfl_up(v, 1, 64);
  const bool keep = v != INT_MAX && (lane == 0 || v != prev);
  const uint64_t m = __ballot(keep);
  const int n = __popcll(m);
  if (keep) {
    const int pos = __popcll(m & ((1ull << lane) - 1ull));
    urow[pos] = v;
    if (uni_lds) uni_lds[pos] = v;
  }
  if (lane >= n && lane < tot) urow[lane] = -1;
  return n;
}

// Union over the group of the G*kpg selections in sel_all (LDS), ascending
// page id, -1 padded, into uni row h and n_uni[h]; uni_lds (nullable) gets a
// copy. Called by the whole block after a barrier; sel_all (union_pad(G*kpg)
// ints) and wn (kMaxWaves ints) are LDS scratch. Returns the union's size in
// every thread.
__device__ int write_union(int G, int kpg, int32_t* sel_all, int32_t* wn, int32_t* uni, int32_t* n_uni, int h,
                           int32_t* uni_lds) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // ---- union over the group, ascending page id, -1 padded
  const int tot = G * kpg;
  int32_t* urow = uni + (int64_t)h * tot;
  if (tot <= 64) {
    if (wv == 0) {
      const int n = wave_union64(tot, sel_all, urow, uni_lds, lane);
      if (lane == 0) {
        n_uni[h] = n;
        wn[0] = n;
      }
    }
    __syncthreads();
    return wn[0];
  }
  // long selections: bitonic sort of the padded list in LDS (empty = INT_MAX),
  // then keep the first of each run of equal ids
  const int P = union_pad(tot), nthr = blockDim.x, nw = nthr >> 6;
  for (int i = tid; i < P; i += nthr) {
    const int v = i < tot ? sel_all[i] : -1;
    sel_all[i] = v < 0 ? INT_MAX : v;
  }
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int i = tid; i < P; i += nthr) {
        const int l = i ^ jj;
        if (l > i) {
          const int a = sel_all[i], b = sel_all[l];
          if (((i & k) == 0) == (a > b)) {
            sel_all[i] = b;
            sel_all[l] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  int32_t* wcount = wn;   // per-wave counts of a round
  int base = 0;
  for (int r0 = 0; r0 < P; r0 += nthr) {
    const int i = r0 + tid;
    const int v = i < P ? sel_all[i] : INT_MAX;
    const bool keep = v != INT_MAX && (i == 0 || sel_all[i - 1] != v);
    const uint64_t m = __ballot(keep);
    if (lane == 0) wcount[wv] = __popcll(m);
    __syncthreads();
    int before = base, all = base;
    for (int w2 = 0; w2 < nw; ++w2) {
      before += w2 < wv ? wcount[w2] : 0;
      all += wcount[w2];
    }
    if (keep) {
      const int pos = before + __popcll(m & ((1ull << lane) - 1ull));
      urow[pos] = v;
      if (uni_lds) uni_lds[pos] = v;
    }
    base = all;
    __syncthreads();
  }
  for (int i = base + tid; i < tot; i += nthr) urow[i] = -1;
  if (tid == 0) n_uni[h] = base;
  return base;
}

// Claims of the fused decode step (LDS): a bit per page id of the head, per
// query head the pages it claimed first and their count, and the counter
// that deals the claimed pages out to the block's waves.
struct ClaimLds {
  uint32_t* bits;
  int32_t* pages;     // [G][kpg]: query head g's claims, then -1
  int32_t* rows;      // [G][kpg]: their valid rows
  int32_t* sel_rows;  // [G][kpg]: valid rows of the selected pages, in selection order
  int32_t* count;     // [G]: claims of query head g, -1 until they are published
  int32_t* done;      // query heads whose claims are complete (zero on entry)
  int32_t* next;      // the next chunk of pages to attend (zero on entry)
};

// Selection of head h by the whole block; returns the size of the group's
// union (in every thread). uni_lds (nullable, LDS outside the selection's
// area) receives a copy of the union. Ends with a block barrier, after which
// the selection's LDS area is free. With `cl` (the fused decode step) it
// writes no union: each query head's waves leave as soon as its lead has
// claimed the query head's pages that no lower query head selected
// (cl->pages, cl->count; the claim bits must be zero and the counts -1 on
// entry), and the caller writes the union with write_union after a block
// barrier.
template <int D, class T, bool BIG>
__device__ int select_head(const DevLayout& L, const void* blob, const T* Q, int budget, int beam, int32_t* sel,
                           int32_t* uni, int32_t* n_uni, int32_t* trace, char* smem, int h, int32_t* uni_lds,
                           const ClaimLds* cl = nullptr) {
  using QG = Quarter<D, T>;
  using Top = std::conditional_t<BIG, LdsTop, RegTop>;
  const int G = L.G, W = (int)(blockDim.x >> 6) / G;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = wv / W, j = wv % W;      // query head, wave within the query
  const bool lead = j == g % W;          // merges the query's lists (leads sit on different SIMDs)
  const int kpg = budget / ICE_PAGE_CAP;
  const SelLds S = sel_lds(G, max(beam, kpg), kpg, BIG);
  const WaveArea A = wave_area(smem, S, wv, BIG);
  const OwnerTable OT = owner_table(smem, S, g);
  uint64_t* comb = reinterpret_cast<uint64_t*>(smem + S.off_comb);
  uint64_t* qlist = reinterpret_cast<uint64_t*>(smem + S.off_query) + g * S.lcap;
  int32_t* wn = reinterpret_cast<int32_t*>(smem + S.off_misc);
  int32_t* qn = wn + kMaxWaves;
  int32_t* qp = qn + ICE_MAX_GROUP;
  int32_t* qbar = qp + ICE_MAX_GROUP;
  int32_t* sel_all = reinterpret_cast<int32_t*>(smem + S.off_sel);

  const void* hb = head_base(blob, L, h);
  const Hdr* hdr = at<Hdr>(hb, L.off_hdr);
  const int n_tok = hdr->n_tokens, Ltop = hdr->top_level;
  // the query heads progress independently between their own barriers
  int* timeouts = const_cast<int*>(&hdr->sync_timeouts);
  if (tid < ICE_MAX_GROUP) qbar[tid] = 0;
  __syncthreads();
  int bar_target = 0;
  auto qsync = [&]() { query_sync(&qbar[g], bar_target, W, timeouts); };

  QG qs;
  qs.load(Q + ((int64_t)h * G + g) * D, lane);
  const int row = lane >> 2;             // row of this lane inside a 16-row pass

  int32_t* tr = trace ? trace + ((int64_t)h * G + g) * L.L * beam : nullptr;
  if (tr && lead)
    for (int i = lane; i < L.L * beam; i += 64) tr[i] = -1;

  // Owner table of `nk` kept owners (lead wave): their pages in table `lvl`.
  // id_of(i) gives the token id (owner slot) of kept entry i.
  auto build_table = [&](int lvl, int nk, auto id_of) {
    const int32_t* firsts = at<int32_t>(hb, L.off_first[lvl]);
    const int32_t* runs = at<int32_t>(hb, L.off_orun[lvl]);
    const int32_t* cnts = at<int32_t>(hb, L.off_ocnt[lvl]);
    int base = 0;
    for (int c0 = 0; c0 < nk; c0 += 64) {
      const int i = c0 + lane;
      const int o = i < nk ? id_of(i) : -1;
      int cnt = 0, first = 0, run = 0;
      if (o >= 0) {
        cnt = cnts[o];
        first = firsts[o];
        run = runs[o];
      }
      const int np = (cnt + ICE_PAGE_CAP - 1) / ICE_PAGE_CAP;
      const int incl = wave_incl_scan(np, lane);
      if (i < nk) {
        OT.off[i] = base + incl - np;
        OT.fst[i] = first;
        OT.rl[i] = run * 32 + (np > 0 ? cnt - ICE_PAGE_CAP * (np - 1) : 0);
      }
      base += __builtin_amdgcn_readlane(incl, 63);
    }
    if (lane == 0) {
      OT.off[nk] = base;
      qn[g] = nk;
      qp[g] = base;
    }
  };

  // Merges the W wave lists of each query head into its kept list of at most
  // `cap` entries; the lead wave writes the trace row `cut` (cut >= 0) or the
  // selection (cut < 0), and the owner table of the kept points in table
  // `lvl` (lvl >= 0).
  auto combine = [&](Top& t, int cap, int cut, int lvl) {
    if constexpr (!BIG) {
      comb[wv * 64 + lane] = t.L;
      qsync();
      if (lead) {
        const uint64_t* ql0 = comb + (g * W) * 64;
        uint64_t r = ql0[lane];
        if ((W == 2 || W == 4) && W * cap <= 64) {
          r = merge_lists(ql0, W, lane);
        } else {
          for (int jj = 1; jj < W; ++jj) r = wave_merge(r, ql0[jj * 64 + 63 - lane]);
        }
        const uint64_t ql = lane < cap ? r : 0ull;
        const int qc = __popcll(__ballot(ql != 0ull));
        const int id = lane < qc ? (cut >= 0 ? key_id(ql) : key_page(ql)) : -1;
        if (cut >= 0) {
          if (tr && lane < beam) tr[cut * beam + lane] = id;
        } else if (lane < kpg) {
          // the fused step writes `sel` from sel_all once its attention is
          // done: a global store here would hold the claim behind it
          if (!cl) sel[((int64_t)h * G + g) * kpg + lane] = id;
          sel_all[g * kpg + lane] = id;
          if (cl) cl->sel_rows[g * kpg + lane] = lane < qc ? key_rows(ql) : 0;
        }
        if (lvl >= 0) build_table(lvl, qc, [&](int) { return id; });
      }
    } else {
      if (lane == 0) wn[wv] = t.n;
      qsync();
      int tot = 0;
      for (int jj = 0; jj < W; ++jj) tot += wn[g * W + jj];
      for (int i = lane; i < t.n; i += 64) {
        const uint64_t x = A.list[i];
        int rank = i;
        for (int jj = 0; jj < W; ++jj) {
          if (jj == j) continue;
          const int ow = g * W + jj;
          rank += count_greater(reinterpret_cast<const uint64_t*>(smem + ow * S.wave_bytes), wn[ow], x);
        }
        if (rank < cap) qlist[rank] = x;
      }
      qsync();
      if (lead) {
        const int qc = min(cap, tot);
        auto id_of = [&](int i) { return i < qc ? (cut >= 0 ? key_id(qlist[i]) : key_page(qlist[i])) : -1; };
        if (cut >= 0) {
          if (tr)
            for (int i = lane; i < beam; i += 64) tr[cut * beam + i] = id_of(i);
        } else {
          for (int i = lane; i < kpg; i += 64) {
            const int id = id_of(i);
            sel[((int64_t)h * G + g) * kpg + i] = id;
            sel_all[g * kpg + i] = id;
          }
        }
        if (lvl >= 0) build_table(lvl, qc, id_of);
      }
    }
    qsync();
  };

  int cut = 0;
  if (n_tok > 0 && Ltop >= 1) {
    // ---- top level: every point of the top list, 16-row groups split over the waves
    {
      const int n_top = hdr->n_top;
      const int32_t* top_tok = at<int32_t>(hb, L.off_top_tok);
      const T* top_K = at<T>(hb, L.off_top_K);
      const int ngroups = (n_top + 15) / 16;
      Top tl;
      tl.init(beam);
      for (int m0 = j; m0 < ngroups; m0 += 4 * W) {
        bool ok[4];
        const T* rp[4];
        int tk[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int r = (m0 + b * W) * 16 + row;
          ok[b] = r < n_top;
          const int rc = ok[b] ? r : 0;          // loads are unconditional so they batch
          rp[b] = top_K + (int64_t)rc * D;
          tk[b] = top_tok[rc];
        }
        tl.push(A, chunk_keys<D, T>(qs, ok, rp, tk, lane), lane);
      }
      combine(tl, beam, cut++, Ltop - 1);
    }
    // ---- levels Ltop-1 .. 1: the children of the kept points, every row scored
    for (int l = Ltop - 1; l >= 1; --l) {
      const int32_t* next = at<int32_t>(hb, L.off_pg_next[l]);
      const int32_t* pg_tok = at<int32_t>(hb, L.off_pg_tok[l]);
      const T* pgK = at<T>(hb, L.off_pgK[l]);
      const int n_own = qn[g], P = qp[g];
      Top tl;
      tl.init(beam);
      for (int t0 = 0, nb; (nb = deal_pages(A, OT, n_own, P, j, W, t0, next, lane)) > 0; t0 += 64) {
        for (int b0 = 0; b0 < nb; b0 += 4) {
          bool ok[4];
          const T* rp[4];
          int tk[4];
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int blk = b0 + b < nb ? A.cand[b0 + b] : -1;
            ok[b] = blk >= 0 && row < A.cval[b0 + b];
            const int64_t r = (int64_t)(blk >= 0 ? blk : 0) * ICE_PAGE_CAP + row;   // in the page: 16 slots exist
            rp[b] = pgK + r * D;
            tk[b] = pg_tok[r];
          }
          tl.push(A, chunk_keys<D, T>(qs, ok, rp, tk, lane), lane);
        }
        wave_sync();
      }
      combine(tl, beam, cut++, l - 1);
    }
  } else if (n_tok > 0) {
    // ---- root: the virtual root owns every token
    if (lead) build_table(0, 1, [&](int) { return L.cap; });
    qsync();
  }

  // ---- level 0: the pages of the kept level-1 points, one key per page
  {
    Top tl;
    tl.init(kpg);
    if (n_tok > 0) {
      const int32_t* next = at<int32_t>(hb, L.off_pg_next[0]);
      const T* pgK = at<T>(hb, L.off_pgK[0]);
      const int n_own = qn[g], P = qp[g];
      // page keys gather in lanes 0..fill-1: each is formed once on the scalar
      // unit and written into its lane
      uint32_t pk_hi = 0u, pk_lo = 0u;
      int fill = 0;
      for (int t0 = 0, nb; (nb = deal_pages(A, OT, n_own, P, j, W, t0, next, lane)) > 0; t0 += 64) {
        for (int b0 = 0; b0 < nb; b0 += QG::GB0) {
          V4 buf[QG::GB0][QG::NL];
          int pg[QG::GB0], cv[QG::GB0];
#pragma unroll
          for (int b = 0; b < QG::GB0; ++b) {
            // the same LDS word in every lane: uniform values
            pg[b] = __builtin_amdgcn_readfirstlane(b0 + b < nb ? A.cand[b0 + b] : -1);
            cv[b] = __builtin_amdgcn_readfirstlane(b0 + b < nb ? A.cval[b0 + b] : 0);
            const bool ok = pg[b] >= 0 && row < cv[b];
            qs.fetch(ok, pgK + ((int64_t)(ok ? pg[b] : 0) * ICE_PAGE_CAP + row) * D, buf[b]);
          }
#pragma unroll
          for (int b = 0; b < QG::GB0; ++b) {
            if (pg[b] < 0) continue;
            float s = qs.dot(buf[b]);
            if (row >= cv[b]) s = -INFINITY;
            s = rows_max(s);
            const uint32_t hi = ordered_bits(__int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(s))));
            const uint32_t lo = page_key_lo(__builtin_amdgcn_readfirstlane(pg[b]), cv[b]);
            write_lane(pk_hi, hi, fill);
            write_lane(pk_lo, lo, fill);
            if (++fill == 64) {
              tl.push(A, ((uint64_t)pk_hi << 32) | pk_lo, lane);
              pk_hi = pk_lo = 0u;
              fill = 0;
            }
          }
        }
        wave_sync();
      }
      if (fill) {
        const uint64_t pk = ((uint64_t)pk_hi << 32) | pk_lo;
        if constexpr (!BIG) {
          if (fill <= 16 && tl.n == 0) tl.push16(pk, lane);
          else tl.push(A, pk, lane);
        } else {
          tl.push(A, pk, lane);
        }
      }
    }
    combine(tl, kpg, -1, -1);
  }
  if (cl) {
    // the query head's selected pages that no lower query head of the group
    // selected, in selection order: these its waves attend. The lead first
    // waits for query head g-1 to publish; that one waited for g-2, and so
    // on, so the claim bits then hold exactly the lower query heads' pages
    // and the claims do not depend on which query head finished first (a
    // bounded wait: past kSpinLimit polls it counts a timeout and goes on).
    if (lead) {
      if (g > 0) {
        int spins = 0;
        while (__atomic_load_n(&cl->count[g - 1], __ATOMIC_RELAXED) < 0) {
          if (++spins > kSpinLimit) {
            if (lane == 0) atomicAdd(timeouts, 1);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      }
      const int p = lane < kpg ? sel_all[g * kpg + lane] : -1;
      const int pr = lane < kpg ? cl->sel_rows[g * kpg + lane] : 0;
      bool mine = false;
      if (p >= 0) {
        const uint32_t bit = 1u << (p & 31);
        mine = (atomicOr(&cl->bits[p >> 5], bit) & bit) == 0u;
      }
      const uint64_t mk = __ballot(mine);
      const int n = __popcll(mk);
      if (mine) {
        const int at_ = g * kpg + __popcll(mk & ((1ull << lane) - 1ull));
        cl->pages[at_] = p;
        cl->rows[at_] = pr;
      }
      if (lane >= n && lane < kpg) {
        cl->pages[g * kpg + lane] = -1;
        cl->rows[g * kpg + lane] = 0;
      }
      // publish: the pages are visible before the count
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      if (lane == 0) __atomic_store_n(&cl->count[g], n, __ATOMIC_RELAXED);
      // the last query head to finish sees every selection: it writes the
      // union right away when one wave can sort it
      int done = 0;
      if (lane == 0) done = atomicAdd(cl->done, 1);
      done = __shfl(done, 0, 64);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      if (done == G - 1 && G * kpg <= 64) {
        const int n = wave_union64(G * kpg, sel_all, uni + (int64_t)h * G * kpg, nullptr, lane);
        if (lane == 0) n_uni[h] = n;
      }
    }
    qsync();
    return 0;
  }
  __syncthreads();      // every query head's selection is in sel_all
  return write_union(G, kpg, sel_all, wn, uni, n_uni, h, uni_lds);
}

template <int D, class T, bool BIG>
__global__ __launch_bounds__(1024) void k_select(DevLayout L, const void* blob, const T* Q, int budget, int beam,
                                                 int32_t* sel, int32_t* uni, int32_t* n_uni, int32_t* trace) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  select_head<D, T, BIG>(L, blob, Q, budget, beam, sel, uni, n_uni, trace, smem, blockIdx.x, nullptr);
}

// ---- the fused decode step: selection, then attention over the union -------
// Each query head's waves attend the pages it claimed as soon as its own
// selection ends, while the block's other query heads are still selecting;
// the union is then exactly the claimed pages, each attended once, for all G
// query heads. The waves' partials are merged after one block barrier.
// LDS: the selection's area, attention's Q^T and partials, the claim bits
// (one per page id of the head), the claimed pages and their counts.
struct DecLds {
  int off_part, off_bits, off_pages, off_rows, off_sel_rows, off_count, words, total;
};
__host__ __device__ inline int align16(int x) { return (x + 15) & ~15; }
__host__ __device__ inline DecLds dec_lds(int G, int beam, int kpg, int nw, int D, int pcap0) {
  const SelLds S = sel_lds(G, max(beam, kpg), kpg, false);
  DecLds d;
  d.off_part = align16(S.total);
  d.off_bits = align16(d.off_part + mfma_attend::part_floats(nw, G, D) * 4);
  d.words = (pcap0 + 31) / 32;
  d.off_pages = align16(d.off_bits + d.words * 4);
  d.off_rows = d.off_pages + G * kpg * 4;
  d.off_sel_rows = d.off_rows + G * kpg * 4;
  d.off_count = d.off_sel_rows + G * kpg * 4;
  d.total = align16(d.off_count + (G + 2) * 4);
  return d;
}
constexpr int kDecodeMaxLds = 160 * 1024;

template <int D>
__global__ __launch_bounds__(1024) void k_decode(DevLayout L, const void* blob, const uint16_t* Q, int budget,
                                                 int beam, int32_t* sel, int32_t* uni, int32_t* n_uni, float scale,
                                                 float* O, float* lse) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int h = blockIdx.x, G = L.G, nw = blockDim.x >> 6, kpg = budget / ICE_PAGE_CAP;
  const DecLds DL = dec_lds(G, beam, kpg, nw, D, L.pcap[0]);
  float* part = reinterpret_cast<float*>(smem + DL.off_part);
  int32_t* cnt = reinterpret_cast<int32_t*>(smem + DL.off_count);
  ClaimLds cl{reinterpret_cast<uint32_t*>(smem + DL.off_bits), reinterpret_cast<int32_t*>(smem + DL.off_pages),
              reinterpret_cast<int32_t*>(smem + DL.off_rows), reinterpret_cast<int32_t*>(smem + DL.off_sel_rows), cnt,
              cnt + G, cnt + G + 1};
  const uint16_t* Qh = Q + (int64_t)h * G * D;
  // ordered before any use by the selection's first block barrier
  mfma_attend::stage_q<D>(Qh, G, part);
  for (int i = threadIdx.x; i < DL.words; i += blockDim.x) cl.bits[i] = 0u;
  if (threadIdx.x < G) cl.count[threadIdx.x] = -1;
  if (threadIdx.x == 0) *cl.done = *cl.next = 0;
  select_head<D, uint16_t, false>(L, blob, Q, budget, beam, sel, uni, n_uni, nullptr, smem, h, nullptr, &cl);
  // Attention: the claimed pages of all query heads, in query-head order,
  // then the head's resident pages, form a list of items cut into at most nw
  // chunks of consecutive items. The chunks are dealt out one at a time to
  // whichever wave asks next, so waves whose query head finished its
  // selection early take the chunks of the later ones. A wave attends its
  // chunk's pages in list order into fresh sums and leaves them in the
  // chunk's partial slot; the slots are merged in chunk order, so the result
  // does not depend on which wave took which chunk (bitwise deterministic). A
  // wave asks once its own selection has ended; it first waits for the query
  // heads whose claims its chunk holds to publish (a bounded wait: past
  // kSpinLimit polls it counts a timeout and skips their pages, so the
  // kernel always ends), then keeps the next page's loads in flight while it
  // attends the current one.
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  (void)wv;
  const void* hb = head_base(blob, L, h);
  const Hdr* hdr = at<Hdr>(hb, L.off_hdr);
  int* timeouts = const_cast<int*>(&hdr->sync_timeouts);
  const int n_pages = hdr->n_pages[0], n_res = hdr->n_resident;
  const int n_rp = min(L.res_pages, (n_res + ICE_PAGE_CAP - 1) / ICE_PAGE_CAP);
  const int n_claim = G * kpg, n_items = n_claim + n_rp;
  const int cs = max(1, (n_items + nw - 1) / nw);        // items per chunk
  const int n_chunks = (n_items + cs - 1) / cs;          // <= nw partial slots
  const char* pgK = at<char>(hb, L.off_pgK[0]);
  const char* pgV = v_pages(L, hb, h);
  const float c2 = scale * mfma_attend::kLog2e;
  for (;;) {
    int c = 0;
    if (lane == 0) c = atomicAdd(cl.next, 1);
    c = __builtin_amdgcn_readfirstlane(__shfl(c, 0, 64));
    if (c >= n_chunks) break;
    const int i0 = c * cs, i1 = min(n_items, (c + 1) * cs);
    // the query heads of the chunk's claims, each waited for once
    uint32_t gq_ok = 0u;
    if (i0 < n_claim) {
      const int g1 = (min(i1, n_claim) - 1) / kpg;
      for (int gq = i0 / kpg; gq <= g1; ++gq) {
        int spins = 0;
        bool ok = true;
        while (__atomic_load_n(&cl.count[gq], __ATOMIC_RELAXED) < 0) {
          if (++spins > kSpinLimit) {
            if (lane == 0) atomicAdd(timeouts, 1);
            ok = false;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        gq_ok |= ok ? 1u << gq : 0u;
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
    mfma_attend::WaveAcc<D> st;
    st.init();
    for (int k0 = i0; k0 < i1; k0 += 64) {
      // lane t: item k0 + t's page and valid rows (0 rows: nothing to attend)
      int my_pg = 0, my_n = 0;
      const int i = k0 + lane;
      if (i < i1) {
        if (i >= n_claim) {     // a resident page: nothing to wait for
          const int r = i - n_claim;
          my_pg = L.pcap[0] + r;
          my_n = min(ICE_PAGE_CAP, n_res - ICE_PAGE_CAP * r);
        } else if ((gq_ok >> (i / kpg)) & 1u) {
          const int pg = cl.pages[i], n = cl.rows[i];
          if (pg >= 0 && pg < n_pages && n > 0) {
            my_pg = pg;
            my_n = n;
          }
        }
      }
      const int nk = min(64, i1 - k0);
      // two K buffers with fixed roles in each half of an unrolled pair of
      // steps: the next page's K loads while the current page's V loads and
      // the current page is attended. The steps are straight-line code
      // (clamped indices, masked pages) so that the next page stays in flight.
      mfma_attend::MPage<D> bufA, bufB;
      auto issue = [&](int k, mfma_attend::MPage<D>& b) {
        const int kc = min(k, nk - 1);
        const int pg = __shfl(my_pg, kc, 64), n = k < nk ? __shfl(my_n, kc, 64) : 0;
        mfma_attend::mload_k<D>(pgK, pg, n, lane, b);
      };
      auto step = [&](int k, mfma_attend::MPage<D>& cur, mfma_attend::MPage<D>& nxt) {
        const int kc = min(k, nk - 1);
        const int pg = __shfl(my_pg, kc, 64), n = k < nk ? __shfl(my_n, kc, 64) : 0;
        uint2 v[mfma_attend::MGeo<D>::VC];
        mfma_attend::mload_v<D>(pgV, pg, n, lane, v);
        issue(k + 1, nxt);
        mfma_attend::page_update<D>(cur.k, v, n, c2, reinterpret_cast<const V4*>(part), lane, st.m, st.l, st.acc);
      };
      issue(0, bufA);
      for (int k = 0; k < nk; k += 2) {
        step(k, bufA, bufB);
        step(k + 1, bufB, bufA);
      }
    }
    mfma_attend::write_partial<D>(st, c, G, part, nw);
  }
  __syncthreads();
  mfma_attend::merge_partials<D>(G, part, nw, O + (int64_t)h * G * D, lse ? lse + (int64_t)h * G : nullptr,
                                 n_chunks);
  // the selections (the selection's LDS is untouched by the attention); a
  // union too long for one wave is written by the block from them
  const SelLds S = sel_lds(G, max(beam, kpg), kpg, false);
  const int32_t* sel_all = reinterpret_cast<const int32_t*>(smem + S.off_sel);
  for (int i = threadIdx.x; i < G * kpg; i += blockDim.x) sel[(int64_t)h * G * kpg + i] = sel_all[i];
  if (G * kpg > 64)
    write_union(G, kpg, reinterpret_cast<int32_t*>(smem + S.off_sel), reinterpret_cast<int32_t*>(smem + S.off_misc),
                uni, n_uni, h, nullptr);
}

template <int D, class T>
void launch_typed(const DevLayout& L, const void* blob, const void* Qv, int budget, int beam, int32_t* sel,
                  int32_t* uni, int32_t* n_uni, int32_t* trace, hipStream_t s) {
  const int kpg = budget / ICE_PAGE_CAP;
  const int lcap = beam > kpg ? beam : kpg;
  const bool big = lcap > 64;
  const SelLds S = sel_lds(L.G, lcap, kpg, big);
  const int nw = launch_waves(L, [&](int) { return S.total; });
  const dim3 grid((unsigned)L.H), block(64 * nw);
  const T* Q = static_cast<const T*>(Qv);
  if (big) k_select<D, T, true><<<grid, block, (size_t)S.total, s>>>(L, blob, Q, budget, beam, sel, uni, n_uni, trace);
  else k_select<D, T, false><<<grid, block, (size_t)S.total, s>>>(L, blob, Q, budget, beam, sel, uni, n_uni, trace);
}

template <int D>
void launch_decode_typed(const DevLayout& L, const void* blob, const void* Qv, int budget, int beam, int32_t* sel,
                         int32_t* uni, int32_t* n_uni, float scale, float* O, float* lse, hipStream_t s) {
  const int kpg = budget / ICE_PAGE_CAP;
  const int nw = launch_waves(L, [&](int n) { return dec_lds(L.G, beam, kpg, n, D, L.pcap[0]).total; });
  const DecLds DL = dec_lds(L.G, beam, kpg, nw, D, L.pcap[0]);
  k_decode<D><<<dim3((unsigned)L.H), dim3(64 * nw), (size_t)DL.total, s>>>(
      L, blob, static_cast<const uint16_t*>(Qv), budget, beam, sel, uni, n_uni, scale, O, lse);
}

}  // namespace

bool decode_fused(const DevLayout& L, int budget, int beam) {
  const int kpg = budget / ICE_PAGE_CAP;
  if (L.dtype != ICE_BF16 || (beam > kpg ? beam : kpg) > 64) return false;
  const int nw = launch_waves(L, [&](int n) { return dec_lds(L.G, beam, kpg, n, L.d, L.pcap[0]).total; });
  return dec_lds(L.G, beam, kpg, nw, L.d, L.pcap[0]).total <= kDecodeMaxLds;
}

hipError_t launch_decode(const DevLayout& L, const void* blob, const void* Q, int budget, int beam, int32_t* sel,
                         int32_t* uni, int32_t* n_uni, float scale, float* O, float* lse, hipStream_t s) {
  if (L.d == 128) launch_decode_typed<128>(L, blob, Q, budget, beam, sel, uni, n_uni, scale, O, lse, s);
  else launch_decode_typed<64>(L, blob, Q, budget, beam, sel, uni, n_uni, scale, O, lse, s);
  return hipGetLastError();
}

hipError_t launch_select(const DevLayout& L, const void* blob, const void* Q, int budget, int beam,
                         int32_t* sel, int32_t* uni, int32_t* n_uni, int32_t* trace, hipStream_t s) {
  if (L.dtype == ICE_BF16) {
    if (L.d == 128) launch_typed<128, uint16_t>(L, blob, Q, budget, beam, sel, uni, n_uni, trace, s);
    else launch_typed<64, uint16_t>(L, blob, Q, budget, beam, sel, uni, n_uni, trace, s);
  } else {
    if (L.d == 128) launch_typed<128, float>(L, blob, Q, budget, beam, sel, uni, n_uni, trace, s);
    else launch_typed<64, float>(L, blob, Q, budget, beam, sel, uni, n_uni, trace, s);
  }
  return hipGetLastError();
}

}  // namespace ice
