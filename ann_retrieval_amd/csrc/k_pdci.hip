// Nearest parent by Prioritized DCI: the approximate search the pages' tree
// is built on, as a build option beside the exact MFMA search.
//
// The papernotes.org notes (key design 2) put M-DCI on P-DCI: no space
// partitioning; several indices each project the points onto a random
// direction and order them by how far the projection lies from the query's;
// a priority queue visits the closest first. The aitangshan.cn article
// (section 3) names it as the prior work the tree extends. The structure
// follows the published method (Li and Malik, ICML 2017): m composite indices
// of l simple indices; a composite index yields a point once all l of its
// simple indices have visited it, and stops after `visits` visits (once it
// has a candidate) or `cands` candidates; all candidates are then ranked by
// their lifted distance.
//
// Per level, for every head at once:
//  1. k_pdci_project: fp64 keys of every candidate parent (a point one level
//     up) in every simple index, from the stored rows and the fp32 lift
//     coordinate. The products are exact in fp64.
//  2. k_pdci_rank: each simple index sorted by (key, candidate) by counting,
//     in LDS tiles, how many keys precede each key: sorted keys, the sorted
//     candidates and each candidate's position.
//  3. k_pdci_search: one thread per child. Per composite index, l walkers
//     start at the child's key in their sorted lists and move outward; each
//     visit takes the walker front with the smallest |key - child key| (ties
//     by simple index, then candidate). A visited candidate is complete when
//     its position in every other list of the composite lies between that
//     list's two walker fronts (the walkers have visited exactly that range).
//     Complete candidates are scored like the insert's parent search (fp32
//     lifted inner product from the rows, ties to the lower token id).
#include "ice_launch.h"

#include <math.h>

namespace ice {
namespace {

constexpr int kPdciThreads = 256;
constexpr int kRankTile = 4096;   // keys per LDS tile of the ranking

struct PdciView {
  bool skip;
  int n_cand, n_child;
  const int32_t* cand;    // candidate parents (points of level+1), ascending token id
  const int32_t* child;   // points of exactly `level`, ascending token id
  const float* e;
  Hdr* hdr;
  char* wh;
};

__device__ inline PdciView pdci_view(const DevLayout& L, const WsLayout& W, void* blob, void* ws, int level, int h) {
  PdciView v;
  void* hb = head_base(blob, L, h);
  v.hdr = at<Hdr>(hb, L.off_hdr);
  v.wh = static_cast<char*>(ws) + (int64_t)h * W.head_bytes;
  v.skip = level >= v.hdr->top_level;
  const int32_t* cnts = at<int32_t>(v.wh, W.off_cnts);
  v.n_cand = v.skip ? 0 : cnts[level + 1];
  v.n_child = v.skip ? 0 : cnts[ICE_MAX_LEVELS + level];
  v.cand = at<int32_t>(v.wh, W.off_pts[level + 1]);
  v.child = at<int32_t>(v.wh, W.off_exact[level]);
  v.e = at<float>(hb, L.off_e);
  return v;
}

// Keys of one lifted row in the first `mk` simple indices (directions staged
// in LDS as [mk][D+1]); NaN keys become +inf and -0 becomes +0, so the keys
// are totally ordered.
template <int D, class T>
__device__ inline void row_keys(const T* row, float e, const float* sd, int mk, double (&key)[ICE_PDCI_MAX_KEYS]) {
#pragma unroll
  for (int k = 0; k < ICE_PDCI_MAX_KEYS; ++k) key[k] = 0.0;
  for (int i = 0; i < D; ++i) {
    const double x = (double)Elt<T>::load(row, i);
#pragma unroll
    for (int k = 0; k < ICE_PDCI_MAX_KEYS; ++k)
      if (k < mk) key[k] = fma(x, (double)sd[k * (D + 1) + i], key[k]);
  }
  const double xe = (double)e;
#pragma unroll
  for (int k = 0; k < ICE_PDCI_MAX_KEYS; ++k) {
    if (k < mk) key[k] = fma(xe, (double)sd[k * (D + 1) + D], key[k]);
    key[k] = key[k] != key[k] ? INFINITY : key[k] + 0.0;
  }
}

template <int D>
__device__ inline void stage_dirs(const PdciArgs& P, float* sd) {
  for (int i = threadIdx.x; i < P.mk * (D + 1); i += blockDim.x) sd[i] = P.dirs[i];
  __syncthreads();
}

template <int D, class T>
__global__ __launch_bounds__(kPdciThreads) void k_pdci_project(DevLayout L, WsLayout W, PdciArgs P, void* blob,
                                                                const T* K, int64_t hstride, void* ws, int level) {
  const int h = blockIdx.y;
  __shared__ float sd[ICE_PDCI_MAX_KEYS * (D + 1)];
  stage_dirs<D>(P, sd);
  const PdciView v = pdci_view(L, W, blob, ws, level, h);
  const int c = blockIdx.x * kPdciThreads + threadIdx.x;
  if (c >= v.n_cand) return;
  const int t = v.cand[c];
  double key[ICE_PDCI_MAX_KEYS];
  row_keys<D, T>(K + (int64_t)h * hstride + (int64_t)t * D, v.e[t], sd, P.mk, key);
#pragma unroll
  for (int k = 0; k < ICE_PDCI_MAX_KEYS; ++k)
    if (k < P.mk) P.keys[((int64_t)h * ICE_PDCI_MAX_KEYS + k) * P.stride + c] = key[k];
}

// Rank of every key of one simple index under (key, candidate): grid (tiles
// of the list, simple index, head).
__global__ __launch_bounds__(kPdciThreads) void k_pdci_rank(DevLayout L, WsLayout W, PdciArgs P, void* blob, void* ws,
                                                            int level) {
  const int k = blockIdx.y, h = blockIdx.z;
  const PdciView v = pdci_view(L, W, blob, ws, level, h);
  const int n = v.n_cand;
  const int64_t base = ((int64_t)h * ICE_PDCI_MAX_KEYS + k) * P.stride;
  const int c = blockIdx.x * kPdciThreads + threadIdx.x;
  const double kc = c < n ? P.keys[base + c] : 0.0;
  __shared__ double tile[kRankTile];
  int rank = 0;
  for (int t0 = 0; t0 < n; t0 += kRankTile) {
    const int m = min(kRankTile, n - t0);
    __syncthreads();
    for (int i = threadIdx.x; i < m; i += kPdciThreads) tile[i] = P.keys[base + t0 + i];
    __syncthreads();
    if (c < n)
      for (int i = 0; i < m; ++i) {
        const double ki = tile[i];
        rank += (ki < kc || (ki == kc && t0 + i < c)) ? 1 : 0;
      }
  }
  if (c < n) {
    P.skeys[base + rank] = kc;
    P.sidx[base + rank] = c;
    P.posof[base + c] = rank;
  }
}

// One walker front: |key - query key|, simple index, candidate, position.
struct Front {
  double d;
  int list, cand, pos;
};

__device__ inline bool before(const Front& a, const Front& b) {
  return a.d < b.d || (a.d == b.d && (a.list < b.list || (a.list == b.list && a.cand < b.cand)));
}

__device__ inline Front load_front(const PdciArgs& P, int64_t base, int n, int pos, double q, int list) {
  Front f;
  f.list = list;
  f.pos = pos;
  if (pos < 0 || pos >= n) {
    f.d = INFINITY;
    f.cand = 0x7fffffff;
  } else {
    f.d = fabs(P.skeys[base + pos] - q);
    f.cand = P.sidx[base + pos];
  }
  return f;
}

// fp32 lifted inner product of two rows (the insert's parent score)
template <int D, class T>
__device__ inline float row_score(const T* a, const T* b, float ea, float eb) {
  constexpr int PER = Elt<T>::per16;
  const V4* a4 = reinterpret_cast<const V4*>(a);
  const V4* b4 = reinterpret_cast<const V4*>(b);
  float s = 0.0f;
  for (int i = 0; i < D / PER; ++i) {
    float x[PER], y[PER];
    Elt<T>::unpack(a4[i], x);
    Elt<T>::unpack(b4[i], y);
#pragma unroll
    for (int j = 0; j < PER; ++j) s = fmaf(x[j], y[j], s);
  }
  return fmaf(ea, eb, s);
}

template <int D, class T>
__global__ __launch_bounds__(kPdciThreads) void k_pdci_search(DevLayout L, WsLayout W, PdciArgs P, void* blob,
                                                               const T* K, int64_t hstride, void* ws, int level) {
  const int h = blockIdx.y;
  __shared__ float sd[ICE_PDCI_MAX_KEYS * (D + 1)];
  stage_dirs<D>(P, sd);
  const PdciView v = pdci_view(L, W, blob, ws, level, h);
  const int i = blockIdx.x * kPdciThreads + threadIdx.x;
  if (i >= v.n_child) return;
  const int n = v.n_cand;
  const int t = v.child[i];
  const T* Kh = K + (int64_t)h * hstride;
  const T* rowt = Kh + (int64_t)t * D;
  const float et = v.e[t];
  double q[ICE_PDCI_MAX_KEYS];
  row_keys<D, T>(rowt, et, sd, P.mk, q);
  float best = -INFINITY, second = -INFINITY;
  int btok = 0x7fffffff;
  for (int j = 0; j < P.m; ++j) {
    Front lf[ICE_PDCI_MAX_L], rf[ICE_PDCI_MAX_L];
    int64_t base[ICE_PDCI_MAX_L];
#pragma unroll
    for (int s = 0; s < ICE_PDCI_MAX_L; ++s) {
      base[s] = ((int64_t)h * ICE_PDCI_MAX_KEYS + j * P.l + s) * P.stride;
      if (s < P.l) {
        const double qs = q[0];
        double qk = qs;
#pragma unroll
        for (int k = 0; k < ICE_PDCI_MAX_KEYS; ++k)
          if (k == j * P.l + s) qk = q[k];
        // first position whose key is not below the child's
        int lo = 0, hi = n;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (P.skeys[base[s] + mid] < qk) lo = mid + 1;
          else hi = mid;
        }
        lf[s] = load_front(P, base[s], n, lo - 1, qk, s);
        rf[s] = load_front(P, base[s], n, lo, qk, s);
      } else {
        lf[s] = rf[s] = Front{INFINITY, s, 0x7fffffff, -1};
      }
    }
    int visited = 0, found = 0;
    while (found < P.cands && (visited < P.visits || found == 0)) {
      Front b = lf[0];
      bool left = true;
#pragma unroll
      for (int s = 0; s < ICE_PDCI_MAX_L; ++s) {
        if (s > 0 && before(lf[s], b)) {
          b = lf[s];
          left = true;
        }
        if (before(rf[s], b)) {
          b = rf[s];
          left = false;
        }
      }
      if (!(b.d < INFINITY)) break;   // every walker has run off its list
      ++visited;
      bool done = true;
#pragma unroll
      for (int s = 0; s < ICE_PDCI_MAX_L; ++s) {
        if (s < P.l && s != b.list) {
          const int p = P.posof[base[s] + b.cand];
          done &= p > lf[s].pos && p < rf[s].pos;
        }
      }
      // the popped walker moves one step outward
#pragma unroll
      for (int s = 0; s < ICE_PDCI_MAX_L; ++s) {
        if (s == b.list) {
          double qk = q[0];
#pragma unroll
          for (int k = 0; k < ICE_PDCI_MAX_KEYS; ++k)
            if (k == j * P.l + s) qk = q[k];
          if (left) lf[s] = load_front(P, base[s], n, lf[s].pos - 1, qk, s);
          else rf[s] = load_front(P, base[s], n, rf[s].pos + 1, qk, s);
        }
      }
      if (done) {
        ++found;
        const int tok = v.cand[b.cand];
        if (tok != btok) {
          const float sc = row_score<D, T>(rowt, Kh + (int64_t)tok * D, et, v.e[tok]);
          if (sc > best || (sc == best && tok < btok)) {
            second = best;
            best = sc;
            btok = tok;
          } else {
            second = fmaxf(second, sc);
          }
        }
      }
    }
  }
  void* hb = head_base(blob, L, h);
  // no candidate at all only if every key was non-finite: take the first point
  const int par = btok != 0x7fffffff ? btok : v.cand[0];
  at<int32_t>(hb, L.off_parent[level])[t] = par;
  at<float>(v.wh, W.off_s1)[t] = best;
  at<float>(v.wh, W.off_s2)[t] = second;
  const float M2 = (float)v.hdr->M2;
  if (second > -INFINITY && (best - second) < 1e-4f * (M2 - second)) atomicAdd(&v.hdr->near_ties, 1);
}

inline unsigned blocks_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per < 1 ? 1 : (n + per - 1) / per); }

template <int D, class T>
hipError_t pdci_typed(const DevLayout& L, const WsLayout& W, const PdciArgs& P, void* blob, const void* Kv,
                      int64_t hstride, void* ws, int level, hipStream_t s) {
  const T* K = static_cast<const T*>(Kv);
  const unsigned H = (unsigned)L.H;
  const int nc = L.ncap[level + 1];
  k_pdci_project<D, T><<<dim3(blocks_for(nc, kPdciThreads), H), kPdciThreads, 0, s>>>(L, W, P, blob, K, hstride, ws,
                                                                                      level);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_pdci_rank<<<dim3(blocks_for(nc, kPdciThreads), (unsigned)P.mk, H), kPdciThreads, 0, s>>>(L, W, P, blob, ws,
                                                                                              level);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  k_pdci_search<D, T><<<dim3(blocks_for(L.ncap[level], kPdciThreads), H), kPdciThreads, 0, s>>>(L, W, P, blob, K,
                                                                                              hstride, ws, level);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_parent_pdci(const DevLayout& L, const WsLayout& W, const PdciArgs& P, void* blob, const void* K,
                              int64_t head_stride, void* ws, int level, hipStream_t s) {
  if (L.dtype == ICE_BF16) {
    if (L.d == 128) return pdci_typed<128, uint16_t>(L, W, P, blob, K, head_stride, ws, level, s);
    return pdci_typed<64, uint16_t>(L, W, P, blob, K, head_stride, ws, level, s);
  }
  if (L.d == 128) return pdci_typed<128, float>(L, W, P, blob, K, head_stride, ws, level, s);
  return pdci_typed<64, float>(L, W, P, blob, K, head_stride, ws, level, s);
}

}  // namespace ice
