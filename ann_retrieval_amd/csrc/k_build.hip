// Index build kernels: key norms and promotion levels, the lift and the
// level lists, the parent-GEMM operand, the deterministic page pack and the
// row copies into the page pool.
//
// What is computed follows the aitangshan.cn IceCache article, section 3
// (lift keys so inner product becomes Euclidean distance; random promotion
// into a pyramid of levels; each point's parent is its most similar point one
// level up; points sharing a parent share a page) and the papernotes.org
// IceCache notes, key designs 1-2 (each node is one physical page).
#include "ice_launch.h"

#include <math.h>

namespace ice {
namespace {

constexpr int kScanThreads = 1024;

// Exclusive prefix sum over the 1024 threads of a block. `total` receives the
// block sum. `lds` needs 16 ints.
__device__ inline int block_scan_excl(int v, int* lds, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int y = __shfl_up(x, m, 64);
    if (lane >= m) x += y;
  }
  if (lane == 63) lds[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
    const int s = lds[w];
    if (w < wave) before += s;
    all += s;
  }
  __syncthreads();
  total = all;
  return before + x - v;
}

__global__ void k_fill_heads(void* base, int64_t head_bytes, int64_t off, int64_t n, int32_t value) {
  int32_t* p = at<int32_t>(static_cast<char*>(base) + (int64_t)blockIdx.y * head_bytes, off);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = value;
}

// Several fills of every head region in one launch: range z of `f` is
// n[z] int32 words at byte offset off[z], set to val[z].
constexpr int kMaxFills = 2 + 5 * (ICE_MAX_LEVELS - 1);   // header (two ranges) + five per table
struct FillSet {
  int count = 0;
  int64_t off[kMaxFills], n[kMaxFills];
  int32_t val[kMaxFills];
  void add(int64_t o, int64_t words, int32_t v) {
    off[count] = o;
    n[count] = words;
    val[count] = v;
    ++count;
  }
};
__global__ void k_fill_set(void* base, int64_t head_bytes, FillSet f) {
  const int z = blockIdx.z;
  int32_t* p = at<int32_t>(static_cast<char*>(base) + (int64_t)blockIdx.y * head_bytes, f.off[z]);
  const int32_t value = f.val[z];
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < f.n[z]; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = value;
}

// Flag f of a token at level lv (lv = -1: no token) in the level lists:
// f < ICE_MAX_LEVELS: lv >= f; else lv == f - ICE_MAX_LEVELS (levels < NL).
__device__ inline bool level_flag(int f, int lv, int NL) {
  return f < ICE_MAX_LEVELS ? f < NL && lv >= f : f - ICE_MAX_LEVELS < NL && lv == f - ICE_MAX_LEVELS;
}
constexpr int kLevelFlags = 2 * ICE_MAX_LEVELS;

// |k|^2 in fp64 (exact products for bf16 and fp32 inputs), the promotion
// level (unless `draw` is false: a layout taken from another head keeps its
// levels), the per-head maximum M^2, and the block's count of every level
// flag. One block covers kNormTokens tokens of a head, every wave a quarter
// of them with all its row loads in flight.
constexpr int kNormTokens = kLiftBlock;
template <int D, class T>
__global__ __launch_bounds__(256) void k_norm_level(DevLayout L, WsLayout W, void* blob, const T* K,
                                                    int64_t hstride, int n, void* ws, bool draw) {
  using G = RowGeo<D, T>;
  static_assert(kNormTokens == 256, "four waves, one token per thread in the level counts");
  constexpr int PW = kNormTokens / 4;     // tokens per wave
  const int h = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const T* Kh = K + (int64_t)h * hstride;
  void* hb = head_base(blob, L, h);
  double* n2 = at<double>(static_cast<char*>(ws) + (int64_t)h * W.head_bytes, W.off_n2);
  int8_t* lev = at<int8_t>(hb, L.off_lev);
  double mx = 0.0;
  const int base = blockIdx.x * kNormTokens + wave * PW;
#pragma unroll
  for (int r0 = 0; r0 < PW; r0 += G::RPP) {
    const int t = base + r0 + lane / G::LPR;
    double acc = 0.0;
    if (t < n) {
      const V4 v = *reinterpret_cast<const V4*>(reinterpret_cast<const char*>(Kh + (int64_t)t * D) +
                                                (lane % G::LPR) * 16);
      float f[G::EPL];
      Elt<T>::unpack(v, f);
#pragma unroll
      for (int i = 0; i < G::EPL; ++i) acc += (double)f[i] * (double)f[i];
    }
    acc = group_sum_d<G::LPR>(acc);
    if (t < n && (lane % G::LPR) == 0) {
      n2[t] = acc;
      mx = fmax(mx, acc);
    }
  }
  // level of token blockIdx.x * kNormTokens + threadIdx.x, and the block's
  // count of each level flag
  __shared__ int fc[4][kLevelFlags];
  {
    const int t = blockIdx.x * kNormTokens + (int)threadIdx.x;
    int lv = -1;
    if (t < n) {
      if (draw) {
        lv = draw_level(L.seed, L.h0 + h, t, L.L, L.plog2);
        lev[t] = (int8_t)lv;
      } else {
        lv = lev[t];
      }
    }
#pragma unroll
    for (int f = 0; f < kLevelFlags; ++f) {
      const uint64_t m = __ballot(level_flag(f, lv, L.L));
      if (lane == 0) fc[wave][f] = __popcll(m);
    }
  }
  __shared__ double red[4];
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) mx = fmax(mx, __shfl_xor(mx, m, 64));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  if (threadIdx.x < kLevelFlags)
    at<int32_t>(static_cast<char*>(ws) + (int64_t)h * W.head_bytes, W.off_blkcnt)[blockIdx.x * kLevelFlags + threadIdx.x] =
        fc[0][threadIdx.x] + fc[1][threadIdx.x] + fc[2][threadIdx.x] + fc[3][threadIdx.x];
  if (threadIdx.x == 0) {
    const double b = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
    // Non-negative doubles order like their bit patterns.
    if (b > 0.0)
      atomicMax(reinterpret_cast<unsigned long long*>(&at<Hdr>(hb, L.off_hdr)->M2),
                (unsigned long long)__double_as_longlong(b));
  }
}

// The stable level lists from the per-block flag counts, in two steps.
// k_lift_scan (one block per head): each flag's counts become the counts of
// the blocks before (an exclusive scan over the token blocks); the totals
// give the level sizes, the top level and the header's counts.
__global__ __launch_bounds__(kScanThreads) void k_lift_scan(DevLayout L, WsLayout W, void* blob, void* ws, int n) {
  const int h = blockIdx.x, tid = threadIdx.x;
  void* hb = head_base(blob, L, h);
  char* wh = static_cast<char*>(ws) + (int64_t)h * W.head_bytes;
  Hdr* hdr = at<Hdr>(hb, L.off_hdr);
  int32_t* bc = at<int32_t>(wh, W.off_blkcnt);
  const int nblk = (n + kNormTokens - 1) / kNormTokens;
  __shared__ int lds[16];
  __shared__ int tot[kLevelFlags];
  for (int f = 0; f < kLevelFlags; ++f) {
    int run = 0;
    for (int b0 = 0; b0 < nblk; b0 += kScanThreads) {
      const int b = b0 + tid;
      const int c = b < nblk ? bc[b * kLevelFlags + f] : 0;
      int total;
      const int ex = block_scan_excl(c, lds, total);
      if (b < nblk) bc[b * kLevelFlags + f] = run + ex;
      run += total;
    }
    if (tid == 0) tot[f] = run;
  }
  __syncthreads();
  if (tid == 0) {
    const int NL = L.L;
    int Ltop = 0;
    for (int l = 1; l < NL; ++l)
      if (tot[l] > 0) Ltop = l;
    int32_t* cnts = at<int32_t>(wh, W.off_cnts);
    for (int l = 0; l < ICE_MAX_LEVELS; ++l) {
      cnts[l] = l < NL ? tot[l] : 0;
      cnts[ICE_MAX_LEVELS + l] = l < NL ? tot[ICE_MAX_LEVELS + l] : 0;
    }
    hdr->n_tokens = n;
    hdr->top_level = Ltop;
    hdr->n_top = Ltop >= 1 ? tot[Ltop] : 0;
  }
}

// k_lift_scatter (one block per kNormTokens tokens): the lift coordinate
// e = sqrt(max(0, M^2 - |k|^2)) of each token, and its place in every level
// list it belongs to: pts[l] (level >= l, ascending) with rank[l], exact[l]
// (level == l), and the top list (the top level's points, ascending).
__global__ __launch_bounds__(kNormTokens) void k_lift_scatter(DevLayout L, WsLayout W, void* blob, void* ws, int n) {
  const int h = blockIdx.y, blk = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  void* hb = head_base(blob, L, h);
  char* wh = static_cast<char*>(ws) + (int64_t)h * W.head_bytes;
  const Hdr* hdr = at<Hdr>(hb, L.off_hdr);
  const int NL = L.L, Ltop = hdr->top_level;
  const int t = blk * kNormTokens + tid;
  const bool valid = t < n;
  const int lv = valid ? at<int8_t>(hb, L.off_lev)[t] : -1;
  if (valid) at<float>(hb, L.off_e)[t] = (float)sqrt(fmax(0.0, hdr->M2 - at<double>(wh, W.off_n2)[t]));
  __shared__ int wc[kNormTokens / 64][kLevelFlags];
  uint64_t masks[kLevelFlags];
#pragma unroll
  for (int f = 0; f < kLevelFlags; ++f) {
    masks[f] = __ballot(level_flag(f, lv, NL));
    if (lane == 0) wc[wave][f] = __popcll(masks[f]);
  }
  __syncthreads();
  const int32_t* before = at<int32_t>(wh, W.off_blkcnt) + blk * kLevelFlags;
#pragma unroll
  for (int f = 0; f < kLevelFlags; ++f) {
    int pos = before[f] + __popcll(masks[f] & ((1ull << lane) - 1ull));
    for (int w = 0; w < wave; ++w) pos += wc[w][f];
    const bool fl = (masks[f] >> lane) & 1ull;
    if (f >= 1 && f < NL) {
      if (fl) at<int32_t>(wh, W.off_pts[f])[pos] = t;
      if (valid) at<int32_t>(wh, W.off_rank[f])[t] = fl ? pos : -1;
      if (fl && f == Ltop) at<int32_t>(hb, L.off_top_tok)[pos] = t;
    } else if (f >= ICE_MAX_LEVELS && fl) {
      at<int32_t>(wh, W.off_exact[f - ICE_MAX_LEVELS])[pos] = t;
    }
  }
}

// Operand rows of the candidate parents (points of level `level`+1):
// bf16: [key (D) | e0 e1 e0 e2 e0 e1 | 0 ...] with e = e0+e1+e2 split in
// bf16 parts, so that one extra MFMA step adds e_child * e_parent to the
// key inner product; then kGemmPadRows padding rows [0 ... 0 | -3.4e38 in
// the step's last column], which the children's 1 in that column turns
// into scores below any candidate's. fp32: [key | e | 0 0 0].
template <int D, class T>
__global__ void k_gather_opA(DevLayout L, WsLayout W, const void* blob, const T* K, int64_t hstride, void* ws,
                             int level) {
  const int h = blockIdx.y;
  const void* hb = head_base(blob, L, h);
  if (level >= at<Hdr>(hb, L.off_hdr)->top_level) return;
  char* wh = static_cast<char*>(ws) + (int64_t)h * W.head_bytes;
  const int n_cand = at<int32_t>(wh, W.off_cnts)[level + 1];
  const int32_t* pts = at<int32_t>(wh, W.off_pts[level + 1]);
  const float* e = at<float>(hb, L.off_e);
  T* opA = at<T>(wh, W.off_opA);
  const T* Kh = K + (int64_t)h * hstride;
  // one 16-byte piece of a row per thread
  constexpr int EPP = 16 / (int)sizeof(T);     // elements per piece
  const int ppr = W.kp / EPP;                  // pieces per row
  const int64_t total = (int64_t)(n_cand + (sizeof(T) == 2 ? kGemmPadRows : 0)) * ppr;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int r = (int)(i / ppr), q = (int)(i % ppr);
    union {
      V4 v;
      T x[EPP];
    } out;
    out.v = V4{0, 0, 0, 0};
    if (r >= n_cand) {                                     // bf16 padding row
      if (q == ppr - 1) out.x[EPP - 1] = T(0xFF7F);
    } else {
      const int tok = pts[r];
      if (q < D / EPP) {
        out.v = *reinterpret_cast<const V4*>(Kh + (int64_t)tok * D + q * EPP);
      } else if (q == D / EPP) {
        if constexpr (sizeof(T) == 4) {
          out.x[0] = e[tok];
        } else {
          const float ev = e[tok];
          const uint16_t p0 = f32_to_bf16(ev);
          const float r1 = ev - bf16_to_f32(p0);
          const uint16_t p1 = f32_to_bf16(r1);
          const uint16_t p2 = f32_to_bf16(r1 - bf16_to_f32(p1));
          out.x[0] = p0;
          out.x[1] = p1;
          out.x[2] = p0;
          out.x[3] = p2;
          out.x[4] = p0;
          out.x[5] = p1;
        }
      }
    }
    *reinterpret_cast<V4*>(opA + i * EPP) = out.v;
  }
}

// ---- page pack -------------------------------------------------------------
// Level-`level` points are grouped by owner (their level-(level+1) parent),
// owners walked in ascending token id; inside an owner the owner itself comes
// first, then its children by descending parent score (= ascending lifted
// distance), equal scores by ascending token id; every owner's run is cut into
// pages of 16 with consecutive ids. With no promoted point (root mode) a
// virtual root owns every token in token order.

struct PackView {
  bool skip, root;
  int n_pts, n_own;
  const int32_t* pts;   // nullptr at level 0 (point index = token id)
};

__device__ inline PackView pack_view(const DevLayout& L, const WsLayout& W, const void* hb, const char* wh,
                                     int level) {
  PackView v;
  const Hdr* hdr = at<Hdr>(hb, L.off_hdr);
  const int Ltop = hdr->top_level;
  v.root = Ltop == 0;
  v.skip = v.root ? level != 0 : level >= Ltop;
  const int32_t* cnts = at<int32_t>(wh, W.off_cnts);
  v.n_pts = level == 0 ? hdr->n_tokens : cnts[level];
  v.n_own = v.root ? 1 : cnts[level + 1];
  v.pts = level == 0 ? nullptr : at<int32_t>(wh, W.off_pts[level]);
  return v;
}

// Owner table and page metadata from the owners' member counts cnt[o]
// (global or LDS): a block-wide scan over the owners in chunks of the block
// gives each owner its first bucket position cbase and first page pbase
// (written to the workspace, and to base_lds when given); every owner slot
// gets its first / tail page, run and count, every page its owner, next
// page and count, and the empty token slots -1. Called by the whole block.
__device__ void write_owner_table(const DevLayout& L, const WsLayout& W, void* hb, char* wh, const PackView& v,
                                  int level, const int32_t* cnt, int32_t* base_lds) {
  __shared__ int lds[16];
  int32_t* cnt_g = at<int32_t>(wh, W.off_cnt);
  int32_t* cbase = at<int32_t>(wh, W.off_cbase);
  int32_t* pbase = at<int32_t>(wh, W.off_pbase);
  int32_t* fill = at<int32_t>(wh, W.off_fill);
  const int32_t* owners = v.root ? nullptr : at<int32_t>(wh, W.off_pts[level + 1]);
  int32_t* pg_tok = at<int32_t>(hb, L.off_pg_tok[level]);
  int32_t* pg_cnt = at<int32_t>(hb, L.off_pg_cnt[level]);
  int32_t* pg_next = at<int32_t>(hb, L.off_pg_next[level]);
  int32_t* pg_owner = at<int32_t>(hb, L.off_pg_owner[level]);
  int32_t* first = at<int32_t>(hb, L.off_first[level]);
  int32_t* tail = at<int32_t>(hb, L.off_tail[level]);
  int32_t* orun = at<int32_t>(hb, L.off_orun[level]);
  int32_t* ocnt = at<int32_t>(hb, L.off_ocnt[level]);
  int runc = 0, runp = 0;
  for (int b0 = 0; b0 < v.n_own; b0 += kScanThreads) {
    const int o = b0 + threadIdx.x;
    const int c = o < v.n_own ? cnt[o] : 0;
    const int np = (c + ICE_PAGE_CAP - 1) / ICE_PAGE_CAP;
    int totc, totp;
    const int cb = runc + block_scan_excl(c, lds, totc);
    const int pb = runp + block_scan_excl(np, lds, totp);
    if (o < v.n_own) {
      if (cnt != cnt_g) cnt_g[o] = c;
      cbase[o] = cb;
      pbase[o] = pb;
      fill[o] = 0;
      if (base_lds) base_lds[o] = cb;
      const int tok = v.root ? ICE_ROOT : owners[o];
      const int slot = v.root ? L.cap : tok;
      first[slot] = np ? pb : -1;
      tail[slot] = np ? pb + np - 1 : -1;
      orun[slot] = np;
      ocnt[slot] = c;
      for (int j = 0; j < np; ++j) {
        const int p = pb + j;
        const int pc = min(ICE_PAGE_CAP, c - j * ICE_PAGE_CAP);
        pg_owner[p] = tok;
        pg_next[p] = j + 1 < np ? p + 1 : -1;
        pg_cnt[p] = pc;
        for (int s2 = pc; s2 < ICE_PAGE_CAP; ++s2) pg_tok[(int64_t)p * ICE_PAGE_CAP + s2] = -1;
      }
    }
    runc += totc;
    runp += totp;
  }
  if (threadIdx.x == 0) at<Hdr>(hb, L.off_hdr)->n_pages[level] = runp;
}

__global__ __launch_bounds__(kScanThreads) void k_pack_scan(DevLayout L, WsLayout W, void* blob, void* ws,
                                                           int level) {
  const int h = blockIdx.x;
  void* hb = head_base(blob, L, h);
  char* wh = static_cast<char*>(ws) + (int64_t)h * W.head_bytes;
  const PackView v = pack_view(L, W, hb, wh, level);
  if (v.skip) return;
  write_owner_table(L, W, hb, wh, v, level, at<int32_t>(wh, W.off_cnt), nullptr);
}

// Owner slot of point i of the level (its owner's position in the next
// level's point list; 0 in root mode). An owner is its own parent.
__device__ inline int point_owner(const DevLayout& L, const WsLayout& W, void* hb, char* wh, const PackView& v,
                                  int level, int i, int& t) {
  t = v.pts ? v.pts[i] : i;
  if (v.root) return 0;
  int32_t* parent = at<int32_t>(hb, L.off_parent[level]);
  const int8_t* lev = at<int8_t>(hb, L.off_lev);
  int ow;
  if (lev[t] >= level + 1) {
    ow = t;
    parent[t] = t;
    at<float>(wh, W.off_s1)[t] = INFINITY;   // the owner leads its own run
  } else {
    ow = parent[t];
  }
  return at<int32_t>(wh, W.off_rank[level + 1])[ow];
}

// Owners per head the one-block pack keeps in LDS (two int32 arrays).
constexpr int kPackLdsOwners = 8192;

// The pack's grouping of one head in one block, for heads whose owners fit
// the LDS: every point's owner and the owners' counts (LDS atomics), the
// owner table (write_owner_table), then every point's (score, token) into a
// slot of its owner's bucket (LDS atomics). k_pack_rank then orders each
// bucket; the virtual root (root mode) needs no bucket.
__global__ __launch_bounds__(kScanThreads) void k_pack_group(DevLayout L, WsLayout W, void* blob, void* ws,
                                                            int level) {
  const int h = blockIdx.x;
  void* hb = head_base(blob, L, h);
  char* wh = static_cast<char*>(ws) + (int64_t)h * W.head_bytes;
  const PackView v = pack_view(L, W, hb, wh, level);
  if (v.skip || v.n_own > kPackLdsOwners) return;
  __shared__ int32_t cnt[kPackLdsOwners], base[kPackLdsOwners];
  for (int o = threadIdx.x; o < v.n_own; o += kScanThreads) cnt[o] = 0;
  __syncthreads();
  int32_t* oloc = at<int32_t>(wh, W.off_oloc);
  int32_t* parent = at<int32_t>(hb, L.off_parent[level]);
  const int8_t* lev = at<int8_t>(hb, L.off_lev);
  const int32_t* rank = v.root ? nullptr : at<int32_t>(wh, W.off_rank[level + 1]);
  float* s1w = at<float>(wh, W.off_s1);
  // U points per thread at a time, their loads in flight together
  constexpr int U = 8;
  for (int i0 = threadIdx.x; i0 < v.n_pts; i0 += kScanThreads * U) {
    int t[U], ow[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * kScanThreads;
      t[u] = i < v.n_pts ? (v.pts ? v.pts[i] : i) : -1;
    }
    if (!v.root) {
      int8_t lv[U];
      int par[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        lv[u] = t[u] >= 0 ? lev[t[u]] : 0;
        par[u] = t[u] >= 0 ? parent[t[u]] : 0;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool own = t[u] >= 0 && lv[u] >= level + 1;   // an owner is its own parent
        if (own) {
          parent[t[u]] = t[u];
          s1w[t[u]] = INFINITY;                              // the owner leads its own run
        }
        ow[u] = own ? t[u] : par[u];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) ow[u] = t[u] >= 0 ? rank[ow[u]] : 0;
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) ow[u] = 0;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (t[u] < 0) continue;
      oloc[i0 + u * kScanThreads] = ow[u];
      atomicAdd(&cnt[ow[u]], 1);
    }
  }
  __syncthreads();
  write_owner_table(L, W, hb, wh, v, level, cnt, base);
  __syncthreads();
  if (v.root) return;   // the virtual root's slots are its tokens in order (k_pack_place_root)
  for (int o = threadIdx.x; o < v.n_own; o += kScanThreads) cnt[o] = 0;   // bucket fill counters
  __syncthreads();
  int4* brec = at<int4>(wh, W.off_brec);
  const float* s1 = at<float>(wh, W.off_s1);
  for (int i0 = threadIdx.x; i0 < v.n_pts; i0 += kScanThreads * U) {
    int t[U], o[U];
    float key[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * kScanThreads;
      t[u] = i < v.n_pts ? (v.pts ? v.pts[i] : i) : -1;
      o[u] = i < v.n_pts ? oloc[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) key[u] = t[u] >= 0 ? s1[t[u]] : 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (t[u] < 0) continue;
      const int pos = base[o[u]] + atomicAdd(&cnt[o[u]], 1);
      brec[pos] = make_int4(__float_as_int(key[u]), t[u], o[u], 0);   // one 16-byte store per point
    }
  }
}

__global__ void k_pack_count(DevLayout L, WsLayout W, void* blob, void* ws, int level) {
  const int h = blockIdx.y;
  void* hb = head_base(blob, L, h);
  char* wh = static_cast<char*>(ws) + (int64_t)h * W.head_bytes;
  const PackView v = pack_view(L, W, hb, wh, level);
  if (v.skip) return;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= v.n_pts) return;
  int t;
  const int o = point_owner(L, W, hb, wh, v, level, i, t);
  at<int32_t>(wh, W.off_oloc)[i] = o;
  atomicAdd(at<int32_t>(wh, W.off_cnt) + o, 1);
}

__global__ void k_pack_scatter(DevLayout L, WsLayout W, void* blob, void* ws, int level) {
  const int h = blockIdx.y;
  void* hb = head_base(blob, L, h);
  char* wh = static_cast<char*>(ws) + (int64_t)h * W.head_bytes;
  const PackView v = pack_view(L, W, hb, wh, level);
  if (v.skip || v.root) return;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= v.n_pts) return;
  const int t = v.pts ? v.pts[i] : i;
  const int o = at<int32_t>(wh, W.off_oloc)[i];
  const int pos = at<int32_t>(wh, W.off_cbase)[o] + atomicAdd(at<int32_t>(wh, W.off_fill) + o, 1);
  at<int4>(wh, W.off_brec)[pos] = make_int4(__float_as_int(at<float>(wh, W.off_s1)[t]), t, o, 0);
}

// Final slot of every bucketed point: its rank in its owner's bucket by
// (score desc, token asc). A block takes 256 consecutive bucket positions;
// the buckets they fall in form one contiguous window of the bucket array,
// which the block stages in LDS when it fits (else each point scans its
// bucket in global memory). The owner's pages are consecutive, so rank r is
// slot r counted from its first page.
constexpr int kRankWin = 2048;   // LDS window (entries of 8 bytes)
__global__ __launch_bounds__(256) void k_pack_rank(DevLayout L, WsLayout W, void* blob, void* ws, int level) {
  const int h = blockIdx.y;
  void* hb = head_base(blob, L, h);
  char* wh = static_cast<char*>(ws) + (int64_t)h * W.head_bytes;
  const PackView v = pack_view(L, W, hb, wh, level);
  if (v.skip || v.root) return;
  const int p0 = blockIdx.x * 256;
  if (p0 >= v.n_pts) return;
  const int pos = p0 + (int)threadIdx.x;
  const bool live = pos < v.n_pts;
  const int4* brec = at<int4>(wh, W.off_brec);
  const int4 me = live ? brec[pos] : make_int4(0, 0, 0, 0);
  const int b = live ? at<int32_t>(wh, W.off_cbase)[me.z] : 0;
  const int c = live ? at<int32_t>(wh, W.off_cnt)[me.z] : 0;
  __shared__ int lohi[2];
  __shared__ int2 win[kRankWin];
  if (threadIdx.x == 0) lohi[0] = b;
  if (pos == min(p0 + 255, v.n_pts - 1)) lohi[1] = b + c;
  __syncthreads();
  const int lo = lohi[0], hi = lohi[1];
  const bool staged = hi - lo <= kRankWin;
  if (staged)
    for (int k = threadIdx.x; k < hi - lo; k += 256) {
      const int4 x = brec[lo + k];
      win[k] = make_int2(x.x, x.y);
    }
  __syncthreads();
  if (!live) return;
  const float key = __int_as_float(me.x);
  int r = 0;
  if (staged) {
    for (int j = b - lo; j < b - lo + c; ++j) {
      const int2 x = win[j];
      r += (__int_as_float(x.x) > key) || (__int_as_float(x.x) == key && x.y < me.y);
    }
  } else {
    for (int j = b; j < b + c; ++j) {
      const int4 x = brec[j];
      r += (__int_as_float(x.x) > key) || (__int_as_float(x.x) == key && x.y < me.y);
    }
  }
  at<int32_t>(hb, L.off_pg_tok[level])[(int64_t)at<int32_t>(wh, W.off_pbase)[me.z] * ICE_PAGE_CAP + r] = me.y;
}

// The virtual root's bucket holds every token in token order: token t takes
// slot t of the root's pages.
__global__ void k_pack_place_root(DevLayout L, WsLayout W, void* blob, void* ws, int level) {
  const int h = blockIdx.y;
  void* hb = head_base(blob, L, h);
  char* wh = static_cast<char*>(ws) + (int64_t)h * W.head_bytes;
  const PackView v = pack_view(L, W, hb, wh, level);
  if (v.skip || !v.root) return;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= v.n_pts) return;
  const int t = v.pts ? v.pts[i] : i;
  at<int32_t>(hb, L.off_pg_tok[level])[(int64_t)at<int32_t>(wh, W.off_pbase)[0] * ICE_PAGE_CAP + t] = t;
}

// Rows of the page table into its key (and, at level 0, value) pool; empty
// slots are zero. Upper tables also keep each point's lift coordinate.
template <int D, class T>
__global__ __launch_bounds__(256) void k_copy_pages(DevLayout L, const T* K, int64_t hstride, void* blob,
                                                    int level) {
  using G = RowGeo<D, T>;
  constexpr int UNR = 4;                 // rows per thread with their loads in flight together
  const int h = blockIdx.y;
  void* hb = head_base(blob, L, h);
  const Hdr* hdr = at<Hdr>(hb, L.off_hdr);
  const bool root = hdr->top_level == 0;
  if (root ? level != 0 : level >= hdr->top_level) return;
  const int n_pages = hdr->n_pages[level];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int32_t* pg_tok = at<int32_t>(hb, L.off_pg_tok[level]);
  T* pk = at<T>(hb, L.off_pgK[level]);
  float* pe = level == 0 ? nullptr : at<float>(hb, L.off_pgE[level]);
  const float* e = at<float>(hb, L.off_e);
  const T* Kh = K + (int64_t)h * hstride;
  const int nrows = n_pages * ICE_PAGE_CAP;
  const int64_t so = (lane % G::LPR) * 16;
  const int step = gridDim.x * 4 * G::RPP;
  for (int r0 = (blockIdx.x * 4 + wave) * G::RPP + lane / G::LPR; r0 < nrows; r0 += step * UNR) {
    int tok[UNR];
    V4 kv[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int r = r0 + u * step;
      tok[u] = r < nrows ? pg_tok[r] : -1;
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      kv[u] = V4{0, 0, 0, 0};
      if (tok[u] >= 0) kv[u] = *reinterpret_cast<const V4*>(reinterpret_cast<const char*>(Kh + (int64_t)tok[u] * D) + so);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int r = r0 + u * step;
      if (r >= nrows) continue;
      *reinterpret_cast<V4*>(reinterpret_cast<char*>(pk + (int64_t)r * D) + so) = kv[u];
      if (pe && (lane % G::LPR) == 0) pe[r] = tok[u] >= 0 ? e[tok[u]] : 0.0f;
    }
  }
}

// Level-0 V pages in the layout attention reads: [page][slot group g][dim][4
// slots], g = slot / 4, so each group of 4 slots is one contiguous run (the
// groups past a page's count are never read) and the 4 values of one
// dimension sit together. One wave per page; empty slots are zero.
template <int D, class T>
__global__ __launch_bounds__(256) void k_copy_vt(DevLayout L, const T* V, int64_t hstride, void* blob) {
  // One wave per page: its 16 rows arrive as 16-byte pieces (all of a lane's
  // loads in flight together) into an LDS copy of the page, from which each
  // lane assembles 16-byte pieces of the transposed layout.
  constexpr int RB = D * (int)sizeof(T);        // row bytes
  constexpr int PPR = RB / 16;                  // 16-byte pieces per row
  constexpr int NPL = ICE_PAGE_CAP * PPR / ICE_WAVE;   // pieces per lane
  constexpr int EPC = 16 / (int)sizeof(T);      // elements per piece
  __shared__ __attribute__((aligned(16))) char lds[4][ICE_PAGE_CAP * RB];
  const int h = blockIdx.y;
  void* hb = head_base(blob, L, h);
  const Hdr* hdr = at<Hdr>(hb, L.off_hdr);
  const int n_pages = hdr->n_pages[0];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int32_t* pg_tok = at<int32_t>(hb, L.off_pg_tok[0]);
  T* pv = reinterpret_cast<T*>(v_pages(L, hb, h));
  const char* Vh = reinterpret_cast<const char*>(V + (int64_t)h * hstride);
  char* buf = lds[wave];
  const T* bt = reinterpret_cast<const T*>(buf);
  // the block's waves take consecutive pages in step, so the barriers are uniform
  for (int pg0 = blockIdx.x * 4; pg0 < n_pages; pg0 += gridDim.x * 4) {
    const int pg = pg0 + wave;
    const bool live = pg < n_pages;
    V4 x[NPL];
#pragma unroll
    for (int u = 0; u < NPL; ++u) {
      const int q = lane + ICE_WAVE * u;
      const int tok = live ? pg_tok[(int64_t)pg * ICE_PAGE_CAP + q / PPR] : -1;
      x[u] = V4{0, 0, 0, 0};
      if (tok >= 0) x[u] = *reinterpret_cast<const V4*>(Vh + (int64_t)tok * RB + (q % PPR) * 16);
    }
#pragma unroll
    for (int u = 0; u < NPL; ++u) {
      const int q = lane + ICE_WAVE * u;
      *reinterpret_cast<V4*>(buf + (q / PPR) * RB + (q % PPR) * 16) = x[u];
    }
    __syncthreads();
    if (live) {
      // output element E = (g * D + d) * 4 + i holds slot 4 g + i, dimension d
#pragma unroll
      for (int u = 0; u < NPL; ++u) {
        const int o = lane + ICE_WAVE * u;
        alignas(16) T out[EPC];
#pragma unroll
        for (int k = 0; k < EPC; ++k) {
          const int E = o * EPC + k;
          const int i = E % 4, d = (E / 4) % D, g = E / (4 * D);
          out[k] = bt[(4 * g + i) * D + d];
        }
        *reinterpret_cast<V4*>(pv + (int64_t)pg * ICE_PAGE_CAP * D + (int64_t)o * EPC) =
            *reinterpret_cast<const V4*>(out);
      }
    }
    __syncthreads();
  }
}

template <int D, class T>
__global__ __launch_bounds__(256) void k_copy_top(DevLayout L, const T* K, int64_t hstride, void* blob) {
  using G = RowGeo<D, T>;
  const int h = blockIdx.y;
  void* hb = head_base(blob, L, h);
  const Hdr* hdr = at<Hdr>(hb, L.off_hdr);
  const int n_top = hdr->n_top;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int32_t* top = at<int32_t>(hb, L.off_top_tok);
  T* tk = at<T>(hb, L.off_top_K);
  float* te = at<float>(hb, L.off_top_E);
  const float* e = at<float>(hb, L.off_e);
  const T* Kh = K + (int64_t)h * hstride;
  for (int r0 = (blockIdx.x * 4 + wave) * G::RPP; r0 < n_top; r0 += gridDim.x * 4 * G::RPP) {
    const int r = r0 + lane / G::LPR;
    if (r >= n_top) continue;
    const int tok = top[r];
    const int64_t so = (lane % G::LPR) * 16;
    *reinterpret_cast<V4*>(reinterpret_cast<char*>(tk + (int64_t)r * D) + so) =
        *reinterpret_cast<const V4*>(reinterpret_cast<const char*>(Kh + (int64_t)tok * D) + so);
    if ((lane % G::LPR) == 0) te[r] = e[tok];
  }
}

inline unsigned blocks_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per < 1 ? 1 : (n + per - 1) / per); }

template <int D, class T>
hipError_t build_typed(const DevLayout& L, const WsLayout& W, void* blob, const void* Kv, const void* Vv,
                       int n, int64_t hstride, void* ws, bool keep, hipStream_t s, const PdciArgs* pd,
                       hipEvent_t* ev, BuildPart part) {
  const T* K = static_cast<const T*>(Kv);
  const T* V = static_cast<const T*>(Vv);
  const unsigned H = (unsigned)L.H;
  hipError_t err;
  const bool do_lift = part == BuildPart::kAll || part == BuildPart::kLift;
  const bool do_parent0 = part == BuildPart::kAll || part == BuildPart::kParent0;
  const bool do_rest = part == BuildPart::kAll || part == BuildPart::kRest;
  // phase boundaries (ICE_BUILD_PHASES + 1 events when timed)
  auto mark = [&](int i) -> hipError_t { return ev ? hipEventRecord(ev[i], s) : hipSuccess; };
  if ((err = mark(0))) return err;
#define ICE_CHECK()                                  \
  do {                                               \
    if ((err = hipGetLastError()) != hipSuccess) return err; \
  } while (0)
  // fresh header, parent links and owner heads; `keep` (a rebuild) keeps
  // the header's resident count and dense flag
  if (do_lift) {
    FillSet f;
    if (!keep) {
      f.add(L.off_hdr, sizeof(Hdr) / 4, 0);
    } else {
      f.add(L.off_hdr, offsetof(Hdr, n_resident) / 4, 0);
      f.add(L.off_hdr + offsetof(Hdr, M2), (sizeof(Hdr) - offsetof(Hdr, M2)) / 4, 0);
    }
    for (int l = 0; l < L.ntab; ++l) {
      f.add(L.off_parent[l], L.cap, -1);
      f.add(L.off_first[l], L.cap + 1, -1);
      f.add(L.off_tail[l], L.cap + 1, -1);
      f.add(L.off_orun[l], L.cap + 1, 0);
      f.add(L.off_ocnt[l], L.cap + 1, 0);
    }
    k_fill_set<<<dim3(blocks_for(L.cap + 1, 256 * 4), (unsigned)H, (unsigned)f.count), 256, 0, s>>>(blob, L.head_bytes,
                                                                                                   f);
    ICE_CHECK();
    if (n > 0) {
      k_norm_level<D, T><<<dim3(blocks_for(n, kNormTokens), H), kNormTokens, 0, s>>>(L, W, blob, K, hstride, n, ws,
                                                                                     true);
      ICE_CHECK();
    }
    k_lift_scan<<<H, kScanThreads, 0, s>>>(L, W, blob, ws, n);
    ICE_CHECK();
    if (n > 0) {
      k_lift_scatter<<<dim3(blocks_for(n, kNormTokens), H), kNormTokens, 0, s>>>(L, W, blob, ws, n);
      ICE_CHECK();
    }
  }
  if ((err = mark(1))) return err;
  const int last = L.L >= 2 ? L.L - 2 : 0;
  for (int level = 0; level <= last; ++level) {
    const int npts = L.ncap[level];
    if (level == 0 ? !do_parent0 : !do_rest) {
      // this part leaves the parent search of the level to another
    } else if (L.L >= 2 && n > 0) {
      if (pd) {
        if ((err = mark(2 + 4 * level))) return err;
        if ((err = launch_parent_pdci(L, W, *pd, blob, Kv, hstride, ws, level, s))) return err;
      } else {
        k_gather_opA<D, T><<<dim3(blocks_for((int64_t)L.ncap[level + 1] * W.kp, 256 * 8), H), 256, 0, s>>>(
            L, W, blob, K, hstride, ws, level);
        ICE_CHECK();
        if ((err = mark(2 + 4 * level))) return err;
        if ((err = launch_parent_gemm(L, W, blob, Kv, hstride, ws, level, s))) return err;
      }
    } else if ((err = mark(2 + 4 * level))) {
      return err;
    }
    if ((err = mark(3 + 4 * level))) return err;
    if (!do_rest) continue;
    const int nown = (L.L >= 2 ? L.ncap[level + 1] : 0) + 1;
    if (nown <= kPackLdsOwners) {
      // every head's owners fit one block's LDS: count, scan and bucket in one kernel
      k_pack_group<<<H, kScanThreads, 0, s>>>(L, W, blob, ws, level);
      ICE_CHECK();
    } else {
      if ((err = launch_fill_heads(ws, W.head_bytes, L.H, W.off_cnt, nown, 0, s))) return err;
      if (n > 0) {
        k_pack_count<<<dim3(blocks_for(npts, 256), H), 256, 0, s>>>(L, W, blob, ws, level);
        ICE_CHECK();
      }
      k_pack_scan<<<H, kScanThreads, 0, s>>>(L, W, blob, ws, level);
      ICE_CHECK();
      if (n > 0) {
        k_pack_scatter<<<dim3(blocks_for(npts, 256), H), 256, 0, s>>>(L, W, blob, ws, level);
        ICE_CHECK();
      }
    }
    if (n > 0) {
      if (L.L >= 2) {
        k_pack_rank<<<dim3(blocks_for(npts, 256), H), 256, 0, s>>>(L, W, blob, ws, level);
        ICE_CHECK();
      }
      if (level == 0) {
        k_pack_place_root<<<dim3(blocks_for(npts, 256), H), 256, 0, s>>>(L, W, blob, ws, level);
        ICE_CHECK();
      }
    }
    if ((err = mark(4 + 4 * level))) return err;
    if (n > 0) {
      using G = RowGeo<D, T>;
      k_copy_pages<D, T><<<dim3(blocks_for((int64_t)L.pcap[level] * ICE_PAGE_CAP, 4 * G::RPP * 8), H), 256, 0,
                           s>>>(L, K, hstride, blob, level);
      ICE_CHECK();
      if (level == 0) {
        k_copy_vt<D, T><<<dim3(blocks_for(L.pcap[0], 4 * 4), H), 256, 0, s>>>(L, V, hstride, blob);
        ICE_CHECK();
      }
    }
    if ((err = mark(5 + 4 * level))) return err;
  }
  for (int level = last + 1; level < ICE_MAX_LEVELS - 1; ++level)
    for (int i = 2; i < 6; ++i)
      if ((err = mark(i + 4 * level))) return err;
  if (do_rest && L.L >= 2 && n > 0) {
    using G = RowGeo<D, T>;
    k_copy_top<D, T><<<dim3(blocks_for(L.topcap, 4 * G::RPP * 4), H), 256, 0, s>>>(L, K, hstride, blob);
    ICE_CHECK();
  }
  if ((err = mark(ICE_BUILD_PHASES))) return err;
#undef ICE_CHECK
  return hipSuccess;
}

}  // namespace

hipError_t launch_fill_heads(void* base, int64_t head_bytes, int H, int64_t off, int64_t n, int32_t value,
                             hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_fill_heads<<<dim3(blocks_for(n, 256 * 4), (unsigned)H), 256, 0, s>>>(base, head_bytes, off, n, value);
  return hipGetLastError();
}

// Header of a head that takes another head's layout: the structure's counts
// from the source, no parent statistics (no parent was chosen), M^2 zero for
// the lift to fill, and its own resident count and dense flag when `keep`.
__global__ void k_reuse_header(DevLayout L, void* blob, const void* src, bool keep) {
  const int h = blockIdx.x;
  Hdr* d = at<Hdr>(head_base(blob, L, h), L.off_hdr);
  const Hdr* sh = at<Hdr>(head_base(src, L, h), L.off_hdr);
  if (threadIdx.x == 0) {
    const int nr = keep ? d->n_resident : 0, dn = keep ? d->dense : 0;
    Hdr x = *sh;
    x.clamps = x.splits = x.near_ties = x.overflow = x.sync_timeouts = 0;
    x.n_resident = nr;
    x.dense = dn;
    x.M2 = 0.0;
    *d = x;
  }
}

template <int D, class T>
hipError_t build_reuse_typed(const DevLayout& L, const WsLayout& W, void* blob, const void* src, const void* Kv,
                             const void* Vv, int n, int64_t hstride, void* ws, bool keep, hipStream_t s) {
  const T* K = static_cast<const T*>(Kv);
  const T* V = static_cast<const T*>(Vv);
  const unsigned H = (unsigned)L.H;
  hipError_t err;
  // the layout arrays, head by head (strided copies over the range)
  auto copy = [&](int64_t off, int64_t bytes) -> hipError_t {
    if (bytes <= 0) return hipSuccess;
    return hipMemcpy2DAsync(static_cast<char*>(blob) + off, (size_t)L.head_bytes, static_cast<const char*>(src) + off,
                            (size_t)L.head_bytes, (size_t)bytes, H, hipMemcpyDeviceToDevice, s);
  };
  const int64_t cap = L.cap;
  if ((err = copy(L.off_lev, cap))) return err;
  for (int l = 0; l < L.ntab; ++l) {
    const int64_t P = L.pcap[l];       // the resident pages stay the head's own
    if ((err = copy(L.off_parent[l], cap * 4))) return err;
    if ((err = copy(L.off_pg_tok[l], P * ICE_PAGE_CAP * 4))) return err;
    if ((err = copy(L.off_pg_cnt[l], P * 4))) return err;
    if ((err = copy(L.off_pg_next[l], P * 4))) return err;
    if ((err = copy(L.off_pg_owner[l], P * 4))) return err;
    if ((err = copy(L.off_first[l], (cap + 1) * 4))) return err;
    if ((err = copy(L.off_tail[l], (cap + 1) * 4))) return err;
    if ((err = copy(L.off_orun[l], (cap + 1) * 4))) return err;
    if ((err = copy(L.off_ocnt[l], (cap + 1) * 4))) return err;
  }
  if ((err = copy(L.off_top_tok, (int64_t)L.topcap * 4))) return err;
  k_reuse_header<<<H, 64, 0, s>>>(L, blob, src, keep);
  if ((err = hipGetLastError())) return err;
  // the head's own lift
  if (n > 0) {
    k_norm_level<D, T><<<dim3(blocks_for(n, kNormTokens), H), kNormTokens, 0, s>>>(L, W, blob, K, hstride, n, ws,
                                                                                   false);
    if ((err = hipGetLastError())) return err;
  }
  k_lift_scan<<<H, kScanThreads, 0, s>>>(L, W, blob, ws, n);
  if ((err = hipGetLastError())) return err;
  if (n > 0) {
    k_lift_scatter<<<dim3(blocks_for(n, kNormTokens), H), kNormTokens, 0, s>>>(L, W, blob, ws, n);
    if ((err = hipGetLastError())) return err;
  }
  if (n == 0) return hipSuccess;
  // its own rows into the pages
  using G = RowGeo<D, T>;
  const int last = L.L >= 2 ? L.L - 2 : 0;
  for (int level = 0; level <= last; ++level) {
    k_copy_pages<D, T><<<dim3(blocks_for((int64_t)L.pcap[level] * ICE_PAGE_CAP, 4 * G::RPP * 8), H), 256, 0, s>>>(
        L, K, hstride, blob, level);
    if ((err = hipGetLastError())) return err;
  }
  k_copy_vt<D, T><<<dim3(blocks_for(L.pcap[0], 4 * 4), H), 256, 0, s>>>(L, V, hstride, blob);
  if ((err = hipGetLastError())) return err;
  if (L.L >= 2) {
    k_copy_top<D, T><<<dim3(blocks_for(L.topcap, 4 * G::RPP * 4), H), 256, 0, s>>>(L, K, hstride, blob);
    if ((err = hipGetLastError())) return err;
  }
  return hipSuccess;
}

hipError_t launch_build_reuse(const DevLayout& L, const WsLayout& W, void* blob, const void* src, const void* K,
                              const void* V, int n_tokens, int64_t head_stride, void* ws, bool keep, hipStream_t s) {
  if (L.dtype == ICE_BF16) {
    if (L.d == 128) return build_reuse_typed<128, uint16_t>(L, W, blob, src, K, V, n_tokens, head_stride, ws, keep, s);
    return build_reuse_typed<64, uint16_t>(L, W, blob, src, K, V, n_tokens, head_stride, ws, keep, s);
  }
  if (L.d == 128) return build_reuse_typed<128, float>(L, W, blob, src, K, V, n_tokens, head_stride, ws, keep, s);
  return build_reuse_typed<64, float>(L, W, blob, src, K, V, n_tokens, head_stride, ws, keep, s);
}

hipError_t launch_build(const DevLayout& L, const WsLayout& W, void* blob, const void* K, const void* V,
                        int n_tokens, int64_t head_stride, void* ws, bool keep, hipStream_t s, const PdciArgs* pd,
                        hipEvent_t* ev, BuildPart part) {
  if (part != BuildPart::kAll && (pd || ev)) return hipErrorInvalidValue;
  if (L.dtype == ICE_BF16) {
    if (L.d == 128)
      return build_typed<128, uint16_t>(L, W, blob, K, V, n_tokens, head_stride, ws, keep, s, pd, ev, part);
    return build_typed<64, uint16_t>(L, W, blob, K, V, n_tokens, head_stride, ws, keep, s, pd, ev, part);
  }
  if (L.d == 128) return build_typed<128, float>(L, W, blob, K, V, n_tokens, head_stride, ws, keep, s, pd, ev, part);
  return build_typed<64, float>(L, W, blob, K, V, n_tokens, head_stride, ws, keep, s, pd, ev, part);
}

}  // namespace ice
