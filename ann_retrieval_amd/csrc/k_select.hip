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
// One block of 16 waves per head; each query head gets W = 16/G waves. At
// every level the candidate rows are split over the query's waves: a wave
// scores 16 rows per pass with 4 lanes per row (bf16 dot2 on gfx950), with
// the loads of several 16-row groups in flight before any arithmetic, and
// folds every 64 candidate keys into its own top list in LDS. The W wave lists
// of a query are then merged by rank (binary search in the other sorted
// lists). Keys pack (score, ~id) into 64 bits, so "score descending, id
// ascending" is plain unsigned order.
#include "ice_launch.h"

namespace ice {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 16;
constexpr int kChainBatch = 64;

// Scoring geometry: 4 lanes per row, 16 rows per wave pass; each lane holds a
// quarter of the query and reads a quarter of every row.
template <int D, class T>
struct Quarter {
  static constexpr int ROWB = D * (int)sizeof(T);
  static constexpr int PB = ROWB / 4;                 // bytes per lane per row
  static constexpr int NL = PB / 16;                  // 16-byte loads per lane per row
  static constexpr int GB = NL >= 16 ? 1 : 16 / NL;   // row groups per load batch
  V4 q[NL];
  int part;

  __device__ inline void load(const T* qrow, int lane) {
    part = lane & 3;
#pragma unroll
    for (int i = 0; i < NL; ++i)
      q[i] = *reinterpret_cast<const V4*>(reinterpret_cast<const char*>(qrow) + part * PB + i * 16);
  }
  // loads this lane's quarter of `row`, or zeros when `ok` is false
  __device__ inline void fetch(bool ok, const T* row, V4* out) const {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      out[i] = V4{0, 0, 0, 0};
      if (ok) out[i] = *reinterpret_cast<const V4*>(reinterpret_cast<const char*>(row) + part * PB + i * 16);
    }
  }
  // partial dot of this lane's quarter; quad_sum completes it
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
    return s;
  }
};

__device__ inline float quad_sum(float s) {
  s += __shfl_xor(s, 1, 64);
  s += __shfl_xor(s, 2, 64);
  return s;
}
// max over the 16 rows of a pass (lanes 4r + part)
__device__ inline float rows_max(float s) {
  s = fmaxf(s, __shfl_xor(s, 4, 64));
  s = fmaxf(s, __shfl_xor(s, 8, 64));
  s = fmaxf(s, __shfl_xor(s, 16, 64));
  s = fmaxf(s, __shfl_xor(s, 32, 64));
  return s;
}

// ---- LDS layout (bytes), shared by the launcher and the kernel --------------
struct SelLds {
  int lcap;           // list capacity = max(beam, pages per query)
  int wave_bytes;     // per wave: list[2][lcap] u64, chunk[64] u64, cand[64] i32, 4 ints
  int off_query;      // per query: list[lcap] u64
  int off_wn;         // per wave: list count and current buffer (2 ints)
  int off_qn;         // per query: list count
  int off_sel;        // [G][kpg] i32
  int off_flag;       // [G][kpg] i32
  int total;
};

__host__ __device__ inline SelLds sel_lds(int G, int lcap, int kpg) {
  SelLds s;
  s.lcap = lcap;
  s.wave_bytes = 2 * lcap * 8 + 64 * 8 + kChainBatch * 4 + 16;
  s.off_query = kWaves * s.wave_bytes;
  s.off_wn = s.off_query + G * lcap * 8;
  s.off_qn = s.off_wn + kWaves * 8;
  s.off_sel = s.off_qn + ICE_MAX_GROUP * 4;
  s.off_flag = s.off_sel + G * kpg * 4;
  s.total = s.off_flag + G * kpg * 4;
  return s;
}

struct WaveArea {
  uint64_t* lists;     // two buffers of lcap keys each
  int lcap;
  uint64_t* chunk;
  int32_t* cand;
  int32_t* ncand;
};

__device__ inline WaveArea wave_area(char* smem, const SelLds& S, int wv) {
  char* b = smem + wv * S.wave_bytes;
  WaveArea a;
  a.lists = reinterpret_cast<uint64_t*>(b);
  a.lcap = S.lcap;
  a.chunk = a.lists + 2 * S.lcap;
  a.cand = reinterpret_cast<int32_t*>(a.chunk + 64);
  a.ncand = a.cand + kChainBatch;
  return a;
}

// Wave-local sorted (descending) top list of at most `cap` keys.
struct TopList {
  int cur, n, cap;
};

// Merges the 64 keys in `a.chunk` (0 = empty) into the list.
__device__ void merge_chunk(const WaveArea& a, TopList& tl, int lane) {
  wave_sync();
  const uint64_t* Lc = a.lists + tl.cur * a.lcap;
  uint64_t* Nx = a.lists + (tl.cur ^ 1) * a.lcap;
  const uint64_t x = a.chunk[lane];
  const uint64_t thr = tl.n == tl.cap ? Lc[tl.cap - 1] : 0ull;
  const bool live = x > thr;
  const uint64_t live_mask = __ballot(live);
  if (live_mask == 0) {
    wave_sync();
    return;
  }
  int rc = 0;
  for (int j = 0; j < 64; ++j) rc += a.chunk[j] > x;
  int lo = 0, hi = tl.n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (Lc[mid] > x) lo = mid + 1;
    else hi = mid;
  }
  for (int i = lane; i < tl.n; i += 64) {
    const uint64_t y = Lc[i];
    int c = 0;
    for (int j = 0; j < 64; ++j) c += a.chunk[j] > y;
    if (i + c < tl.cap) Nx[i + c] = y;
  }
  if (live && lo + rc < tl.cap) Nx[lo + rc] = x;
  tl.n = min(tl.cap, tl.n + __popcll(live_mask));
  tl.cur ^= 1;
  wave_sync();
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

// Gathers up to kChainBatch page ids from the chains in `cur` (lane-owned
// entries); each lane resumes its walk where the batch filled up.
__device__ inline int gather_chains(const WaveArea& a, int32_t (&cur)[ICE_MAX_BEAM / 64], const int32_t* next,
                                    int lane) {
  if (lane == 0) *a.ncand = 0;
  wave_sync();
#pragma unroll
  for (int e = 0; e < ICE_MAX_BEAM / 64; ++e) {
    while (cur[e] >= 0) {
      const int slot = atomicAdd(a.ncand, 1);
      if (slot >= kChainBatch) break;
      a.cand[slot] = cur[e];
      cur[e] = next[cur[e]];
    }
  }
  wave_sync();
  const int n = min(*a.ncand, kChainBatch);
  wave_sync();
  return n;
}

template <int D, class T>
__global__ __launch_bounds__(1024) void k_select(DevLayout L, const void* blob, const T* Q, int budget, int beam,
                                                 int W, int32_t* sel, int32_t* uni, int32_t* n_uni, int32_t* trace) {
  using QG = Quarter<D, T>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int h = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int G = L.G;
  const int g = wv / W, j = wv % W;      // query head, wave within the query
  const int kpg = budget / ICE_PAGE_CAP;
  const SelLds S = sel_lds(G, max(beam, kpg), kpg);
  const WaveArea A = wave_area(smem, S, wv);
  uint64_t* qlist = reinterpret_cast<uint64_t*>(smem + S.off_query) + g * S.lcap;
  int32_t* wn = reinterpret_cast<int32_t*>(smem + S.off_wn);
  int32_t* qn = reinterpret_cast<int32_t*>(smem + S.off_qn);
  int32_t* sel_all = reinterpret_cast<int32_t*>(smem + S.off_sel);
  int32_t* first_flag = reinterpret_cast<int32_t*>(smem + S.off_flag);

  const void* hb = head_base(blob, L, h);
  const Hdr* hdr = at<Hdr>(hb, L.off_hdr);
  const int n_tok = hdr->n_tokens, Ltop = hdr->top_level;

  QG qs;
  qs.load(Q + ((int64_t)h * G + g) * D, lane);
  const int row = lane >> 2;             // row of this lane inside a 16-row pass

  int32_t* tr = trace ? trace + ((int64_t)h * G + g) * L.L * beam : nullptr;
  if (tr && j == 0)
    for (int i = lane; i < L.L * beam; i += 64) tr[i] = -1;

  // Merges the W wave lists of every query into its query list (all waves).
  auto combine = [&](TopList& tl, int cap) {
    if (lane == 0) {
      wn[2 * wv] = tl.n;
      wn[2 * wv + 1] = tl.cur;
    }
    __syncthreads();
    const uint64_t* mine = A.lists + tl.cur * A.lcap;
    int tot = 0;
    for (int jj = 0; jj < W; ++jj) tot += wn[2 * (g * W + jj)];
    for (int i = lane; i < tl.n; i += 64) {
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
  };
  auto emit_trace = [&](int cut) {
    if (tr && j == 0)
      for (int i = lane; i < qn[g]; i += 64) tr[cut * beam + i] = key_id(qlist[i]);
  };

  int cut = 0;
  int32_t cur[ICE_MAX_BEAM / 64];
  if (n_tok > 0 && Ltop >= 1) {
    // ---- top level: every point of the top list, 16-row groups split over the query's waves
    {
      const int n_top = hdr->n_top;
      const int32_t* top_tok = at<int32_t>(hb, L.off_top_tok);
      const T* top_K = at<T>(hb, L.off_top_K);
      const int ngroups = (n_top + 15) / 16;
      TopList tl{0, 0, beam};
      int fill = 0;
      for (int m0 = j; m0 < ngroups; m0 += W * QG::GB) {
        V4 buf[QG::GB][QG::NL];
#pragma unroll
        for (int b = 0; b < QG::GB; ++b) {
          const int r = (m0 + b * W) * 16 + row;
          qs.fetch(r < n_top, top_K + (int64_t)(r < n_top ? r : 0) * D, buf[b]);
        }
#pragma unroll
        for (int b = 0; b < QG::GB; ++b) {
          const int r = (m0 + b * W) * 16 + row;
          const float s = quad_sum(qs.dot(buf[b]));
          if ((lane & 3) == 0) A.chunk[fill + row] = r < n_top ? make_key(s, top_tok[r]) : 0ull;
          fill += 16;
          if (fill == 64) {
            merge_chunk(A, tl, lane);
            fill = 0;
          }
        }
      }
      if (fill) {
        if (lane >= fill) A.chunk[lane] = 0ull;
        merge_chunk(A, tl, lane);
      }
      combine(tl, beam);
      emit_trace(cut++);
    }
    // ---- levels Ltop-1 .. 1: the children of the kept points
    for (int l = Ltop - 1; l >= 1; --l) {
      const int32_t* first = at<int32_t>(hb, L.off_first[l]);
      const int32_t* next = at<int32_t>(hb, L.off_pg_next[l]);
      const int32_t* pg_tok = at<int32_t>(hb, L.off_pg_tok[l]);
      const int32_t* pg_cnt = at<int32_t>(hb, L.off_pg_cnt[l]);
      const T* pgK = at<T>(hb, L.off_pgK[l]);
      const int nq = qn[g];
#pragma unroll
      for (int e = 0; e < ICE_MAX_BEAM / 64; ++e) {
        const int oi = j + W * (lane + 64 * e);
        cur[e] = oi < nq ? first[key_id(qlist[oi])] : -1;
      }
      __syncthreads();   // every wave has read the old query list
      TopList tl{0, 0, beam};
      int fill = 0;
      for (int nb; (nb = gather_chains(A, cur, next, lane)) > 0;) {
        for (int b0 = 0; b0 < nb; b0 += QG::GB) {
          V4 buf[QG::GB][QG::NL];
          int blk[QG::GB];
#pragma unroll
          for (int b = 0; b < QG::GB; ++b) {
            blk[b] = b0 + b < nb ? A.cand[b0 + b] : -1;
            const bool ok = blk[b] >= 0 && row < pg_cnt[blk[b]];
            qs.fetch(ok, pgK + ((int64_t)(ok ? blk[b] : 0) * 16 + row) * D, buf[b]);
          }
#pragma unroll
          for (int b = 0; b < QG::GB; ++b) {
            const bool ok = blk[b] >= 0 && row < pg_cnt[blk[b]];
            const float s = quad_sum(qs.dot(buf[b]));
            if ((lane & 3) == 0)
              A.chunk[fill + row] = ok ? make_key(s, pg_tok[(int64_t)blk[b] * 16 + row]) : 0ull;
            fill += 16;
            if (fill == 64) {
              merge_chunk(A, tl, lane);
              fill = 0;
            }
          }
        }
      }
      if (fill) {
        if (lane >= fill) A.chunk[lane] = 0ull;
        merge_chunk(A, tl, lane);
      }
      combine(tl, beam);
      emit_trace(cut++);
    }
  }

  // ---- level 0: the pages of the kept level-1 points (every page at the root)
  {
    TopList tl{0, 0, kpg};
    if (n_tok > 0) {
      const int32_t* next = at<int32_t>(hb, L.off_pg_next[0]);
      const int32_t* pg_cnt = at<int32_t>(hb, L.off_pg_cnt[0]);
      const T* pgK = at<T>(hb, L.off_pgK[0]);
      const int32_t* first = at<int32_t>(hb, L.off_first[0]);
      const int n_pages = hdr->n_pages[0];
      if (Ltop >= 1) {
        const int nq = qn[g];
#pragma unroll
        for (int e = 0; e < ICE_MAX_BEAM / 64; ++e) {
          const int oi = j + W * (lane + 64 * e);
          cur[e] = oi < nq ? first[key_id(qlist[oi])] : -1;
        }
      }
      __syncthreads();
      int fill = 0;
      // root: the pages are split over the waves by id, no chain walk
      int root_next = j;
      for (;;) {
        int nb;
        if (Ltop >= 1) {
          nb = gather_chains(A, cur, next, lane);
        } else {
          nb = min(kChainBatch, (n_pages - root_next + W - 1) / W);
          if (nb > 0) {
            for (int i = lane; i < nb; i += 64) A.cand[i] = root_next + i * W;
            root_next += nb * W;
          }
          wave_sync();
        }
        if (nb <= 0) break;
        for (int b0 = 0; b0 < nb; b0 += QG::GB) {
          V4 buf[QG::GB][QG::NL];
          int pg[QG::GB];
#pragma unroll
          for (int b = 0; b < QG::GB; ++b) {
            pg[b] = b0 + b < nb ? A.cand[b0 + b] : -1;
            const bool ok = pg[b] >= 0 && row < pg_cnt[pg[b]];
            qs.fetch(ok, pgK + ((int64_t)(ok ? pg[b] : 0) * 16 + row) * D, buf[b]);
          }
#pragma unroll
          for (int b = 0; b < QG::GB; ++b) {
            if (pg[b] < 0) continue;
            float s = quad_sum(qs.dot(buf[b]));
            if (row >= pg_cnt[pg[b]]) s = -INFINITY;
            s = rows_max(s);
            if (lane == 0) A.chunk[fill] = make_key(s, pg[b]);
            if (++fill == 64) {
              merge_chunk(A, tl, lane);
              fill = 0;
            }
          }
        }
      }
      if (fill) {
        if (lane >= fill) A.chunk[lane] = 0ull;
        merge_chunk(A, tl, lane);
      }
    } else {
      __syncthreads();
    }
    combine(tl, kpg);
  }

  // ---- outputs of this query head
  if (j == 0) {
    int32_t* srow = sel + ((int64_t)h * G + g) * kpg;
    for (int i = lane; i < kpg; i += 64) {
      const int v = i < qn[g] ? key_id(qlist[i]) : -1;
      srow[i] = v;
      sel_all[g * kpg + i] = v;
    }
  }
  __syncthreads();
  // ---- union over the group, ascending page id
  const int tot = G * kpg;
  for (int i = tid; i < tot; i += blockDim.x) {
    const int v = sel_all[i];
    bool f = v >= 0;
    for (int k = 0; k < i && f; ++k) f = sel_all[k] != v;
    first_flag[i] = f;
  }
  __syncthreads();
  int32_t* urow = uni + (int64_t)h * tot;
  int nf = 0;
  for (int k = 0; k < tot; ++k) nf += first_flag[k];
  for (int i = tid; i < tot; i += blockDim.x) {
    if (first_flag[i]) {
      const int v = sel_all[i];
      int pos = 0;
      for (int k = 0; k < tot; ++k) pos += first_flag[k] && sel_all[k] < v;
      urow[pos] = v;
    }
    if (i >= nf) urow[i] = -1;
  }
  if (tid == 0) n_uni[h] = nf;
}

}  // namespace

hipError_t launch_select(const DevLayout& L, const void* blob, const void* Q, int budget, int beam,
                         int32_t* sel, int32_t* uni, int32_t* n_uni, int32_t* trace, hipStream_t s) {
  const int kpg = budget / ICE_PAGE_CAP;
  const int W = kWaves / L.G;
  const SelLds S = sel_lds(L.G, beam > kpg ? beam : kpg, kpg);
  const dim3 grid((unsigned)L.H), block((unsigned)(64 * W * L.G));
  const size_t lds = (size_t)S.total;
  if (L.dtype == ICE_BF16) {
    const uint16_t* q = static_cast<const uint16_t*>(Q);
    if (L.d == 128) k_select<128, uint16_t><<<grid, block, lds, s>>>(L, blob, q, budget, beam, W, sel, uni, n_uni, trace);
    else k_select<64, uint16_t><<<grid, block, lds, s>>>(L, blob, q, budget, beam, W, sel, uni, n_uni, trace);
  } else {
    const float* q = static_cast<const float*>(Q);
    if (L.d == 128) k_select<128, float><<<grid, block, lds, s>>>(L, blob, q, budget, beam, W, sel, uni, n_uni, trace);
    else k_select<64, float><<<grid, block, lds, s>>>(L, blob, q, budget, beam, W, sel, uni, n_uni, trace);
  }
  return hipGetLastError();
}

size_t select_lds_bytes(int G, int budget, int beam) {
  const int kpg = budget / ICE_PAGE_CAP;
  return (size_t)sel_lds(G, beam > kpg ? beam : kpg, kpg).total;
}

}  // namespace ice
