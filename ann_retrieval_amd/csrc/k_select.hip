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
// One block per head, one wave per query head. Candidates stream through a
// per-wave top list in LDS: every 64 candidate keys are merged into the list
// by rank counting. Keys pack (score, ~id) into 64 bits so that the order
// "score descending, id ascending" is plain integer order.
#include "ice_launch.h"

namespace ice {
namespace {

constexpr int kChainBatch = 64;   // page/block ids gathered per round

struct WaveLds {
  uint64_t list[2][ICE_MAX_BEAM];
  uint64_t chunk[64];
  int32_t cand[kChainBatch];
  int32_t ncand;
  int32_t pad;
};

// Sorted top list of at most `cap` keys (descending), double-buffered.
struct TopList {
  WaveLds* w;
  int cur, n, cap;
  __device__ uint64_t* data() { return w->list[cur]; }
};

// Merges the 64 keys in w->chunk (0 = empty) into the list.
__device__ void merge_chunk(TopList& tl, int lane) {
  WaveLds* w = tl.w;
  wave_sync();
  const uint64_t* L = w->list[tl.cur];
  uint64_t* N = w->list[tl.cur ^ 1];
  const uint64_t x = w->chunk[lane];
  const uint64_t thr = tl.n == tl.cap ? L[tl.cap - 1] : 0ull;
  const bool live = x > thr;
  const uint64_t live_mask = __ballot(live);
  if (live_mask == 0) {
    wave_sync();
    return;
  }
  // rank of x among the chunk and among the list
  int rc = 0;
  for (int j = 0; j < 64; ++j) rc += w->chunk[j] > x;
  int lo = 0, hi = tl.n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (L[mid] > x) lo = mid + 1;
    else hi = mid;
  }
  const int pos = lo + rc;
  // new positions of the list entries (only live chunk keys can overtake)
  for (int i = lane; i < tl.n; i += 64) {
    const uint64_t y = L[i];
    int c = 0;
    for (int j = 0; j < 64; ++j) c += w->chunk[j] > y;
    if (i + c < tl.cap) N[i + c] = y;
  }
  if (live && pos < tl.cap) N[pos] = x;
  const int nl = __popcll(live_mask);
  tl.n = min(tl.cap, tl.n + nl);
  tl.cur ^= 1;
  wave_sync();
}

template <int D, class T>
struct Scorer {
  using G = RowGeo<D, T>;
  float q[G::EPL];
  int slice;   // lane % LPR

  __device__ inline void load(const T* qrow, int lane) {
    slice = lane % G::LPR;
    const V4 v = *reinterpret_cast<const V4*>(reinterpret_cast<const char*>(qrow) + slice * 16);
    Elt<T>::unpack(v, q);
  }
  // Partial dot of this lane's slice of `row` (all lanes of a row group
  // then hold the full score after group_sum).
  __device__ inline float partial(const T* row) const {
    const V4 v = *reinterpret_cast<const V4*>(reinterpret_cast<const char*>(row) + slice * 16);
    float f[G::EPL];
    Elt<T>::unpack(v, f);
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < G::EPL; ++i) s = fmaf(q[i], f[i], s);
    return s;
  }
};

// Gathers up to kChainBatch page ids from the chains of the owners in
// `owners` (lane i walks the chains of owners i, i+64, ...). `cur` keeps each
// lane's position so the walk resumes where the batch filled up. Returns
// false when every chain is exhausted and nothing was gathered.
__device__ inline bool gather_chains(WaveLds* w, int32_t (&cur)[ICE_MAX_BEAM / 64], int n_own,
                                     const int32_t* next, int lane) {
  if (lane == 0) w->ncand = 0;
  wave_sync();
  for (int e = 0; e < ICE_MAX_BEAM / 64; ++e) {
    if (lane + 64 * e >= n_own) continue;
    while (cur[e] >= 0) {
      const int slot = atomicAdd(&w->ncand, 1);
      if (slot >= kChainBatch) break;
      w->cand[slot] = cur[e];
      cur[e] = next[cur[e]];
    }
  }
  wave_sync();
  const int n = min(w->ncand, kChainBatch);
  wave_sync();
  if (lane == 0) w->ncand = n;
  wave_sync();
  return n > 0;
}

template <int D, class T>
__global__ void k_select(DevLayout L, const void* blob, const T* Q, int budget, int beam, int32_t* sel,
                         int32_t* uni, int32_t* n_uni, int32_t* trace) {
  using G = RowGeo<D, T>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int h = blockIdx.x;
  const int g = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int NG = blockDim.x >> 6;
  const int kpg = budget / ICE_PAGE_CAP;
  WaveLds* w = reinterpret_cast<WaveLds*>(smem) + g;
  int32_t* sel_all = reinterpret_cast<int32_t*>(reinterpret_cast<WaveLds*>(smem) + NG);
  int32_t* first_flag = sel_all + NG * kpg;

  const void* hb = head_base(blob, L, h);
  const Hdr* hdr = at<Hdr>(hb, L.off_hdr);
  const int n_tok = hdr->n_tokens, Ltop = hdr->top_level;
  const int cap = L.cap;

  Scorer<D, T> sc;
  sc.load(Q + ((int64_t)h * NG + g) * D, lane);

  int32_t* tr = trace ? trace + ((int64_t)h * NG + g) * L.L * beam : nullptr;
  if (tr)
    for (int i = lane; i < L.L * beam; i += 64) tr[i] = -1;

  TopList tl{w, 0, 0, beam};
  int32_t cur[ICE_MAX_BEAM / 64];
  int cut = 0;

  if (n_tok > 0 && Ltop >= 1) {
    // ---- top level: score every point of the top list
    const int n_top = hdr->n_top;
    const int32_t* top_tok = at<int32_t>(hb, L.off_top_tok);
    const T* top_K = at<T>(hb, L.off_top_K);
    for (int r0 = 0; r0 < n_top; r0 += 64) {
#pragma unroll 4
      for (int sub = 0; sub < 64; sub += G::RPP) {
        const int rr = sub + lane / G::LPR;
        const int r = r0 + rr;
        float s = 0.0f;
        if (r < n_top) s = sc.partial(top_K + (int64_t)r * D);
        s = group_sum<G::LPR>(s);
        if ((lane % G::LPR) == 0) w->chunk[rr] = r < n_top ? make_key(s, top_tok[r]) : 0ull;
      }
      merge_chunk(tl, lane);
    }
    if (tr)
      for (int i = lane; i < tl.n; i += 64) tr[cut * beam + i] = key_id(tl.data()[i]);
    ++cut;
    // ---- levels Ltop-1 .. 1: children of the kept points
    for (int l = Ltop - 1; l >= 1; --l) {
      const int32_t* first = at<int32_t>(hb, L.off_first[l]);
      const int32_t* next = at<int32_t>(hb, L.off_pg_next[l]);
      const int32_t* pg_tok = at<int32_t>(hb, L.off_pg_tok[l]);
      const int32_t* pg_cnt = at<int32_t>(hb, L.off_pg_cnt[l]);
      const T* pgK = at<T>(hb, L.off_pgK[l]);
      const int n_own = tl.n;
      for (int e = 0; e < ICE_MAX_BEAM / 64; ++e)
        cur[e] = lane + 64 * e < n_own ? first[key_id(tl.data()[lane + 64 * e])] : -1;
      TopList nx{w, tl.cur ^ 1, 0, beam};
      // the old list stays readable in buffer tl.cur while the new one is
      // built: copy the kept owners out first (gathering is done by `cur`).
      wave_sync();
      nx.cur = tl.cur;  // reuse both buffers for the new list
      nx.n = 0;
      while (gather_chains(w, cur, n_own, next, lane)) {
        const int nb = w->ncand;
        for (int b0 = 0; b0 < nb; b0 += 4) {
          // 4 blocks x 16 slots = one chunk of 64 candidates
#pragma unroll 4
          for (int sub = 0; sub < 64; sub += G::RPP) {
            const int rr = sub + lane / G::LPR;
            const int bi = b0 + rr / ICE_PAGE_CAP, slot = rr % ICE_PAGE_CAP;
            const int blk = bi < nb ? w->cand[bi] : -1;
            const bool ok = blk >= 0 && slot < pg_cnt[blk];
            float s = 0.0f;
            if (ok) s = sc.partial(pgK + ((int64_t)blk * ICE_PAGE_CAP + slot) * D);
            s = group_sum<G::LPR>(s);
            if ((lane % G::LPR) == 0)
              w->chunk[rr] = ok ? make_key(s, pg_tok[(int64_t)blk * ICE_PAGE_CAP + slot]) : 0ull;
          }
          merge_chunk(nx, lane);
        }
      }
      tl = nx;
      if (tr)
        for (int i = lane; i < tl.n; i += 64) tr[cut * beam + i] = key_id(tl.data()[i]);
      ++cut;
    }
  }

  // ---- level 0: pages of the kept level-1 points (or every page at the root)
  TopList pl{w, 0, 0, kpg};
  if (n_tok > 0) {
    const int32_t* next = at<int32_t>(hb, L.off_pg_next[0]);
    const int32_t* pg_cnt = at<int32_t>(hb, L.off_pg_cnt[0]);
    const T* pgK = at<T>(hb, L.off_pgK[0]);
    const int32_t* first = at<int32_t>(hb, L.off_first[0]);
    int n_own;
    if (Ltop == 0) {
      n_own = 1;
      for (int e = 0; e < ICE_MAX_BEAM / 64; ++e) cur[e] = (lane == 0 && e == 0) ? first[cap] : -1;
    } else {
      n_own = tl.n;
      for (int e = 0; e < ICE_MAX_BEAM / 64; ++e)
        cur[e] = lane + 64 * e < n_own ? first[key_id(tl.data()[lane + 64 * e])] : -1;
    }
    pl.cur = tl.cur;
    wave_sync();
    int filled = 0;   // page keys in the chunk
    while (gather_chains(w, cur, n_own, next, lane)) {
      const int nb = w->ncand;
      for (int b = 0; b < nb; ++b) {
        const int pg = w->cand[b];
        const int cnt = pg_cnt[pg];
        float best = -INFINITY;
#pragma unroll
        for (int sub = 0; sub < ICE_PAGE_CAP; sub += G::RPP) {
          const int slot = sub + lane / G::LPR;
          float s = 0.0f;
          if (slot < cnt) s = sc.partial(pgK + ((int64_t)pg * ICE_PAGE_CAP + slot) * D);
          s = group_sum<G::LPR>(s);
          if (slot < cnt) best = fmaxf(best, s);
        }
#pragma unroll
        for (int m = G::LPR; m < 64; m <<= 1) best = fmaxf(best, __shfl_xor(best, m, 64));
        if (lane == 0) w->chunk[filled] = make_key(best, pg);
        if (++filled == 64) {
          merge_chunk(pl, lane);
          filled = 0;
        }
      }
    }
    if (filled > 0) {
      if (lane >= filled) w->chunk[lane] = 0ull;
      merge_chunk(pl, lane);
    }
  }
  // ---- outputs of this query head
  int32_t* srow = sel + ((int64_t)h * NG + g) * kpg;
  for (int i = lane; i < kpg; i += 64) {
    const int v = i < pl.n ? key_id(pl.data()[i]) : -1;
    srow[i] = v;
    sel_all[g * kpg + i] = v;
  }
  __syncthreads();
  // ---- union over the group, ascending page id
  const int tot = NG * kpg;
  for (int i = threadIdx.x; i < tot; i += blockDim.x) {
    const int v = sel_all[i];
    bool f = v >= 0;
    for (int j = 0; j < i && f; ++j) f = sel_all[j] != v;
    first_flag[i] = f;
  }
  __syncthreads();
  int32_t* urow = uni + (int64_t)h * tot;
  int nf = 0;
  for (int j = 0; j < tot; ++j) nf += first_flag[j];
  for (int i = threadIdx.x; i < tot; i += blockDim.x) {
    if (first_flag[i]) {
      const int v = sel_all[i];
      int pos = 0;
      for (int j = 0; j < tot; ++j) pos += first_flag[j] && sel_all[j] < v;
      urow[pos] = v;
    }
    if (i >= nf) urow[i] = -1;
  }
  if (threadIdx.x == 0) n_uni[h] = nf;
}

}  // namespace

hipError_t launch_select(const DevLayout& L, const void* blob, const void* Q, int budget, int beam,
                         int32_t* sel, int32_t* uni, int32_t* n_uni, int32_t* trace, hipStream_t s) {
  const int kpg = budget / ICE_PAGE_CAP;
  const size_t lds = sizeof(WaveLds) * L.G + sizeof(int32_t) * 2 * L.G * kpg;
  const dim3 grid((unsigned)L.H), block((unsigned)(64 * L.G));
  if (L.dtype == ICE_BF16) {
    const uint16_t* q = static_cast<const uint16_t*>(Q);
    if (L.d == 128) k_select<128, uint16_t><<<grid, block, lds, s>>>(L, blob, q, budget, beam, sel, uni, n_uni, trace);
    else k_select<64, uint16_t><<<grid, block, lds, s>>>(L, blob, q, budget, beam, sel, uni, n_uni, trace);
  } else {
    const float* q = static_cast<const float*>(Q);
    if (L.d == 128) k_select<128, float><<<grid, block, lds, s>>>(L, blob, q, budget, beam, sel, uni, n_uni, trace);
    else k_select<64, float><<<grid, block, lds, s>>>(L, blob, q, budget, beam, sel, uni, n_uni, trace);
  }
  return hipGetLastError();
}

size_t select_lds_bytes(int G, int budget) {
  return sizeof(WaveLds) * G + sizeof(int32_t) * 2 * G * (budget / ICE_PAGE_CAP);
}

}  // namespace ice
