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
// lane: a chunk of 64 candidates is bitonic-sorted across the wave and merged
// by taking max(list[i], chunk[63-i]) (the 64 largest of both, as a bitonic
// sequence) followed by a 6-step bitonic merge; the W lists of a query merge
// the same way. All lane exchanges of these networks are DPP / permlane moves
// on the VALU. Lists longer than 64 keys (beams or budgets beyond 64 entries)
// use a slower LDS list instead. The block ends with the union of its query
// heads' pages, ascending.
#include "ice_launch.h"

#include <type_traits>

namespace ice {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxWaves = 16;
constexpr int kChainBatch = 64;     // pages gathered per round

__host__ __device__ inline int waves_per_query(int G) { return G <= 4 ? 4 : 16 / G; }
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
  static constexpr int PB = ROWB / 4;                 // bytes per lane per row
  static constexpr int NL = PB / 16;                  // 16-byte loads per lane per row
  static constexpr int GB = NL >= 8 ? 2 : 4;          // row groups per load batch
  V4 q[NL];
  int part;

  __device__ inline void load(const T* qrow, int lane) {
    part = lane & 3;
#pragma unroll
    for (int i = 0; i < NL; ++i)
      q[i] = *reinterpret_cast<const V4*>(reinterpret_cast<const char*>(qrow) + part * PB + i * 16);
  }
  // this lane's quarter of `row`, or zeros when `ok` is false
  __device__ inline void fetch(bool ok, const T* row, V4* out) const {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      out[i] = V4{0, 0, 0, 0};
      if (ok) out[i] = *reinterpret_cast<const V4*>(reinterpret_cast<const char*>(row) + part * PB + i * 16);
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
__device__ inline uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }

template <int k, int j>
__device__ inline uint64_t bitonic_step(uint64_t x, int lane) {
  const uint64_t y = xor_lane_u64<j>(x);
  return (((lane & k) == 0) == ((lane & j) == 0)) ? umax64(x, y) : umin64(x, y);
}
// Sorts one key per lane across the wave, descending (lane 0 largest).
__device__ inline uint64_t wave_sort_desc(uint64_t x, int lane) {
  x = bitonic_step<2, 1>(x, lane);
  x = bitonic_step<4, 2>(x, lane);
  x = bitonic_step<4, 1>(x, lane);
  x = bitonic_step<8, 4>(x, lane);
  x = bitonic_step<8, 2>(x, lane);
  x = bitonic_step<8, 1>(x, lane);
  x = bitonic_step<16, 8>(x, lane);
  x = bitonic_step<16, 4>(x, lane);
  x = bitonic_step<16, 2>(x, lane);
  x = bitonic_step<16, 1>(x, lane);
  x = bitonic_step<32, 16>(x, lane);
  x = bitonic_step<32, 8>(x, lane);
  x = bitonic_step<32, 4>(x, lane);
  x = bitonic_step<32, 2>(x, lane);
  x = bitonic_step<32, 1>(x, lane);
  x = bitonic_step<64, 32>(x, lane);
  x = bitonic_step<64, 16>(x, lane);
  x = bitonic_step<64, 8>(x, lane);
  x = bitonic_step<64, 4>(x, lane);
  x = bitonic_step<64, 2>(x, lane);
  x = bitonic_step<64, 1>(x, lane);
  return x;
}
template <int j>
__device__ inline uint64_t merge_step(uint64_t t, int lane) {
  const uint64_t y = xor_lane_u64<j>(t);
  return (lane & j) == 0 ? umax64(t, y) : umin64(t, y);
}
// Top 64 of two descending wave lists, descending.
__device__ inline uint64_t wave_merge_desc(uint64_t a, uint64_t b_sorted, int lane) {
  // b reversed: lane ^ 63 == 63 - lane
  uint64_t r = xor_lane_u64<1>(b_sorted);
  r = xor_lane_u64<2>(r);
  r = xor_lane_u64<4>(r);
  r = xor_lane_u64<8>(r);
  r = xor_lane_u64<16>(r);
  r = xor_lane_u64<32>(r);
  uint64_t t = umax64(a, r);
  t = merge_step<32>(t, lane);
  t = merge_step<16>(t, lane);
  t = merge_step<8>(t, lane);
  t = merge_step<4>(t, lane);
  t = merge_step<2>(t, lane);
  t = merge_step<1>(t, lane);
  return t;
}

// ---- LDS layout ------------------------------------------------------------
struct SelLds {
  int lcap;           // list capacity = max(beam, pages per query)
  int wave_bytes;     // per wave: [LDS lists: list[2][lcap] u64] chunk[64] u64, cand/cval[64] i32, 4 ints
  int off_comb;       // register lists: [2 parities][kMaxWaves][64] u64
  int off_query;      // LDS lists: [G][lcap] u64 query lists
  int off_wn;         // LDS lists: per wave count and buffer (2 ints)
  int off_qn;         // LDS lists: per query count
  int off_sel;        // [G][kpg] i32 selections (for the union)
  int total;
};

__host__ __device__ inline SelLds sel_lds(int G, int lcap, int kpg, bool big) {
  SelLds s;
  s.lcap = lcap;
  s.wave_bytes = (big ? 2 * lcap * 8 : 0) + 64 * 8 + 2 * kChainBatch * 4 + 16;
  s.off_comb = kMaxWaves * s.wave_bytes;
  s.off_query = s.off_comb + (big ? 0 : 2 * kMaxWaves * 64 * 8);
  s.off_wn = s.off_query + (big ? G * lcap * 8 : 0);
  s.off_qn = s.off_wn + kMaxWaves * 8;
  s.off_sel = s.off_qn + ICE_MAX_GROUP * 4;
  s.total = s.off_sel + union_pad(G * kpg) * 4;
  return s;
}

struct WaveArea {
  uint64_t* lists;     // two buffers of lcap keys each (LDS lists only)
  int lcap;
  uint64_t* chunk;
  int32_t* cand;       // gathered page / block ids
  int32_t* cval;       // their valid slots
  int32_t* ncand;
};

__device__ inline WaveArea wave_area(char* smem, const SelLds& S, int wv, bool big) {
  char* b = smem + wv * S.wave_bytes;
  WaveArea a;
  a.lists = reinterpret_cast<uint64_t*>(b);
  a.lcap = S.lcap;
  a.chunk = a.lists + (big ? 2 * S.lcap : 0);
  a.cand = reinterpret_cast<int32_t*>(a.chunk + 64);
  a.cval = a.cand + kChainBatch;
  a.ncand = a.cval + kChainBatch;
  return a;
}

// ---- wave top lists --------------------------------------------------------
// Register list (cap <= 64): lane i holds entry i, 0 = empty.
struct RegTop {
  uint64_t L;
  int cap;
  __device__ inline void init(int c) {
    L = 0ull;
    cap = c;
  }
  __device__ inline void push(const WaveArea&, uint64_t x, int lane) {
    const uint64_t thr = shfl64(L, cap - 1);   // 0 until the list is full
    if (__ballot(x > thr) == 0) return;
    const uint64_t t = wave_merge_desc(L, wave_sort_desc(x, lane), lane);
    L = lane < cap ? t : 0ull;
  }
};

// LDS list (any cap up to ICE_MAX_BEAM), sorted descending, double-buffered.
struct LdsTop {
  int cur, n, cap;
  __device__ inline void init(int c) {
    cur = 0;
    n = 0;
    cap = c;
  }
  __device__ void push(const WaveArea& a, uint64_t x, int lane) {
    a.chunk[lane] = x;
    wave_sync();
    const uint64_t* Lc = a.lists + cur * a.lcap;
    uint64_t* Nx = a.lists + (cur ^ 1) * a.lcap;
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
    for (int i = lane; i < n; i += 64) {
      const uint64_t y = Lc[i];
      int c = 0;
      for (int j = 0; j < 64; ++j) c += a.chunk[j] > y;
      if (i + c < cap) Nx[i + c] = y;
    }
    if (live && lo + rc < cap) Nx[lo + rc] = x;
    n = min(cap, n + __popcll(live_mask));
    cur ^= 1;
    wave_sync();
  }
};

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

// Walks the pages of one owner per lane. An owner's pages are all full except
// its last; the pages of the build form one contiguous run starting at
// first[], so they need no pointer chasing; only pages split off later by
// inserts are reached through next[].
struct OwnerWalk {
  int page, idx, first, run, cnt;
  __device__ inline void start(int owner_slot, const int32_t* firsts, const int32_t* runs, const int32_t* cnts) {
    page = -1;
    if (owner_slot < 0) return;
    first = firsts[owner_slot];
    run = runs[owner_slot];
    cnt = cnts[owner_slot];
    idx = 0;
    page = cnt > 0 ? first : -1;
  }
};

// Gathers up to kChainBatch (page, valid slots) pairs from this wave's lanes'
// owners; a lane resumes where the batch filled up. Returns the count.
__device__ inline int gather_pages(const WaveArea& a, OwnerWalk& w, const int32_t* next, int lane) {
  if (lane == 0) *a.ncand = 0;
  wave_sync();
  while (w.page >= 0) {
    const int slot = atomicAdd(a.ncand, 1);
    if (slot >= kChainBatch) break;
    a.cand[slot] = w.page;
    a.cval[slot] = min(ICE_PAGE_CAP, w.cnt - ICE_PAGE_CAP * w.idx);
    ++w.idx;
    if (w.idx * ICE_PAGE_CAP >= w.cnt) w.page = -1;
    else if (w.idx < w.run) w.page = w.first + w.idx;
    else w.page = next[w.page];
  }
  wave_sync();
  const int n = min(*a.ncand, kChainBatch);
  wave_sync();
  return n;
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

template <int D, class T, bool BIG>
__global__ __launch_bounds__(1024) void k_select(DevLayout L, const void* blob, const T* Q, int budget, int beam,
                                                 int32_t* sel, int32_t* uni, int32_t* n_uni, int32_t* trace) {
  using QG = Quarter<D, T>;
  using Top = std::conditional_t<BIG, LdsTop, RegTop>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int G = L.G, W = waves_per_query(G);
  const int h = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = wv / W, j = wv % W;      // query head, wave within the query
  const int kpg = budget / ICE_PAGE_CAP;
  const SelLds S = sel_lds(G, max(beam, kpg), kpg, BIG);
  const WaveArea A = wave_area(smem, S, wv, BIG);
  uint64_t* comb = reinterpret_cast<uint64_t*>(smem + S.off_comb);
  uint64_t* qlist = reinterpret_cast<uint64_t*>(smem + S.off_query) + g * S.lcap;
  int32_t* wn = reinterpret_cast<int32_t*>(smem + S.off_wn);
  int32_t* qn = reinterpret_cast<int32_t*>(smem + S.off_qn);
  int32_t* sel_all = reinterpret_cast<int32_t*>(smem + S.off_sel);

  const void* hb = head_base(blob, L, h);
  const Hdr* hdr = at<Hdr>(hb, L.off_hdr);
  const int n_tok = hdr->n_tokens, Ltop = hdr->top_level;

  QG qs;
  qs.load(Q + ((int64_t)h * G + g) * D, lane);
  const int row = lane >> 2;             // row of this lane inside a 16-row pass

  int32_t* tr = trace ? trace + ((int64_t)h * G + g) * L.L * beam : nullptr;
  if (tr && j == 0)
    for (int i = lane; i < L.L * beam; i += 64) tr[i] = -1;

  // the query head's kept list after each cut: a register list (lane i holds
  // entry i) or, for long lists, qlist in LDS
  uint64_t ql = 0ull;
  int qcount = 0, parity = 0;
  auto combine = [&](Top& t, int cap) {
    if constexpr (!BIG) {
      uint64_t* area = comb + parity * kMaxWaves * 64;
      area[wv * 64 + lane] = t.L;
      __syncthreads();
      uint64_t r = t.L;
      for (int jj = 0; jj < W; ++jj)
        if (jj != j) r = wave_merge_desc(r, area[(g * W + jj) * 64 + lane], lane);
      ql = lane < cap ? r : 0ull;
      qcount = __popcll(__ballot(ql != 0ull));
      parity ^= 1;
    } else {
      if (lane == 0) {
        wn[2 * wv] = t.n;
        wn[2 * wv + 1] = t.cur;
      }
      __syncthreads();
      const uint64_t* mine = A.lists + t.cur * A.lcap;
      int tot = 0;
      for (int jj = 0; jj < W; ++jj) tot += wn[2 * (g * W + jj)];
      for (int i = lane; i < t.n; i += 64) {
        const uint64_t x = mine[i];
        int rank = i;
        for (int jj = 0; jj < W; ++jj) {
          if (jj == j) continue;
          const int ow = g * W + jj;
          const uint64_t* other = reinterpret_cast<const uint64_t*>(smem + ow * S.wave_bytes) + wn[2 * ow + 1] * S.lcap;
          rank += count_greater(other, wn[2 * ow], x);
        }
        if (rank < cap) qlist[rank] = x;
      }
      if (j == 0 && lane == 0) qn[g] = min(cap, tot);
      __syncthreads();
      qcount = qn[g];
    }
  };
  // owner (token id) of kept entry oi, -1 past the list; every lane calls it
  auto kept = [&](int oi) -> int {
    if constexpr (!BIG) {
      const uint64_t k = shfl64(ql, oi & 63);
      return oi < qcount ? key_id(k) : -1;
    } else {
      return oi < qcount ? key_id(qlist[oi]) : -1;
    }
  };
  auto emit = [&](int32_t* dst, int n_out) {   // kept ids (rank order), -1 padded
    if constexpr (!BIG) {
      if (lane < n_out) dst[lane] = lane < qcount ? key_id(ql) : -1;
    } else {
      for (int i = lane; i < n_out; i += 64) dst[i] = i < qcount ? key_id(qlist[i]) : -1;
    }
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
      combine(tl, beam);
      if (tr && j == 0) emit(tr + cut * beam, beam);
      ++cut;
    }
    // ---- levels Ltop-1 .. 1: the children of the kept points
    for (int l = Ltop - 1; l >= 1; --l) {
      const int32_t* next = at<int32_t>(hb, L.off_pg_next[l]);
      const int32_t* pg_tok = at<int32_t>(hb, L.off_pg_tok[l]);
      const T* pgK = at<T>(hb, L.off_pgK[l]);
      OwnerWalk ow;
      ow.start(kept(j + W * lane), at<int32_t>(hb, L.off_first[l]), at<int32_t>(hb, L.off_orun[l]),
               at<int32_t>(hb, L.off_ocnt[l]));
      Top tl;
      tl.init(beam);
      for (int nb; (nb = gather_pages(A, ow, next, lane)) > 0;) {
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
      }
      combine(tl, beam);
      if (tr && j == 0) emit(tr + cut * beam, beam);
      ++cut;
    }
  }

  // ---- level 0: the pages of the kept level-1 points (every page at the root)
  {
    Top tl;
    tl.init(kpg);
    if (n_tok > 0) {
      const int32_t* next = at<int32_t>(hb, L.off_pg_next[0]);
      const T* pgK = at<T>(hb, L.off_pgK[0]);
      const int32_t* firsts = at<int32_t>(hb, L.off_first[0]);
      const int32_t* runs = at<int32_t>(hb, L.off_orun[0]);
      const int32_t* cnts = at<int32_t>(hb, L.off_ocnt[0]);
      OwnerWalk ow;
      int root_next = j, root_cnt = 0, n_pages = 0;
      if (Ltop >= 1) {
        ow.start(kept(j + W * lane), firsts, runs, cnts);
      } else {
        // root: chain order is page id order; the pages are split over the waves by id
        ow.page = -1;
        root_cnt = cnts[L.cap];
        n_pages = hdr->n_pages[0];
      }
      uint64_t pk = 0ull;
      int fill = 0;
      for (;;) {
        int nb;
        if (Ltop >= 1) {
          nb = gather_pages(A, ow, next, lane);
        } else {
          nb = min(kChainBatch, (n_pages - root_next + W - 1) / W);
          if (nb > 0) {
            for (int i = lane; i < nb; i += 64) {
              const int pg = root_next + i * W;
              A.cand[i] = pg;
              A.cval[i] = min(ICE_PAGE_CAP, root_cnt - ICE_PAGE_CAP * pg);
            }
            root_next += nb * W;
          }
          wave_sync();
        }
        if (nb <= 0) break;
        for (int b0 = 0; b0 < nb; b0 += QG::GB) {
          V4 buf[QG::GB][QG::NL];
          int pg[QG::GB], cv[QG::GB];
#pragma unroll
          for (int b = 0; b < QG::GB; ++b) {
            pg[b] = b0 + b < nb ? A.cand[b0 + b] : -1;
            cv[b] = b0 + b < nb ? A.cval[b0 + b] : 0;
            const bool ok = pg[b] >= 0 && row < cv[b];
            qs.fetch(ok, pgK + ((int64_t)(ok ? pg[b] : 0) * ICE_PAGE_CAP + row) * D, buf[b]);
          }
#pragma unroll
          for (int b = 0; b < QG::GB; ++b) {
            if (pg[b] < 0) continue;
            float s = qs.dot(buf[b]);
            if (row >= cv[b]) s = -INFINITY;
            s = rows_max(s);
            if (lane == fill) pk = make_key(s, pg[b]);
            if (++fill == 64) {
              tl.push(A, pk, lane);
              pk = 0ull;
              fill = 0;
            }
          }
        }
      }
      if (fill) tl.push(A, pk, lane);
    }
    combine(tl, kpg);
  }
  // ---- outputs of this query head
  if (j == 0) {
    emit(sel + ((int64_t)h * G + g) * kpg, kpg);
    emit(sel_all + g * kpg, kpg);
  }
  __syncthreads();
  // ---- union over the group, ascending page id, -1 padded
  const int tot = G * kpg;
  int32_t* urow = uni + (int64_t)h * tot;
  if (tot <= 64) {
    if (wv != 0) return;
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
    if (keep) urow[__popcll(m & ((1ull << lane) - 1ull))] = v;
    if (lane >= n && lane < tot) urow[lane] = -1;
    if (lane == 0) n_uni[h] = n;
    return;
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
    if (keep) urow[before + __popcll(m & ((1ull << lane) - 1ull))] = v;
    base = all;
    __syncthreads();
  }
  for (int i = base + tid; i < tot; i += nthr) urow[i] = -1;
  if (tid == 0) n_uni[h] = base;
}

template <int D, class T>
void launch_typed(const DevLayout& L, const void* blob, const void* Qv, int budget, int beam, int32_t* sel,
                  int32_t* uni, int32_t* n_uni, int32_t* trace, hipStream_t s) {
  const int kpg = budget / ICE_PAGE_CAP;
  const int lcap = beam > kpg ? beam : kpg;
  const bool big = lcap > 64;
  const SelLds S = sel_lds(L.G, lcap, kpg, big);
  const dim3 grid((unsigned)L.H), block(64 * waves_per_query(L.G) * L.G);
  const T* Q = static_cast<const T*>(Qv);
  if (big) k_select<D, T, true><<<grid, block, (size_t)S.total, s>>>(L, blob, Q, budget, beam, sel, uni, n_uni, trace);
  else k_select<D, T, false><<<grid, block, (size_t)S.total, s>>>(L, blob, Q, budget, beam, sel, uni, n_uni, trace);
}

}  // namespace

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
