// Incremental insert of newly generated tokens.
//
// The aitangshan.cn IceCache article (section 3) inserts a new token without
// rebuilding: it draws its level with the same random promotion, then hangs
// it under the most similar parent at that level. The papernotes.org notes
// (key design 2) add that a node exceeding the page size splits off a new
// page. Here: the level is capped at the build's top level; below its level
// the token is its own parent; a parent search is a GEMV of the lifted key
// against the current points of the next level (ties to the lower token id);
// the token joins its owner's last page or, if that page is full, a newly
// split page that becomes the owner's last page. Placed tokens keep their
// slots, unless the index was created with ICE_SPLIT_RESORT: then a split
// also re-packs the owner's level-0 members over its pages in the build's
// order (distance to the owner, then token id), the new page last.
//
// One block per head; the new tokens of a call are inserted one after the
// other, so a token promoted by one insert is a candidate parent for the
// next. A single thread does the page bookkeeping, which keeps the layout
// deterministic.
#include "ice_launch.h"

#include <math.h>

namespace ice {
namespace {

struct Place {
  int32_t page[ICE_MAX_LEVELS];
  int32_t slot[ICE_MAX_LEVELS];
  int32_t top_slot;
};

// Appends token t to the last page of `owner` in table `tb` (a new owner
// opens its first page). Returns false if the table is full, which the page
// bound rules out while the token count stays within capacity.
__device__ bool place_token(const DevLayout& L, void* hb, Hdr* hdr, int tb, int owner, int t, int32_t& page,
                            int32_t& slot) {
  int32_t* pg_tok = at<int32_t>(hb, L.off_pg_tok[tb]);
  int32_t* pg_cnt = at<int32_t>(hb, L.off_pg_cnt[tb]);
  int32_t* pg_next = at<int32_t>(hb, L.off_pg_next[tb]);
  int32_t* pg_owner = at<int32_t>(hb, L.off_pg_owner[tb]);
  int32_t* first = at<int32_t>(hb, L.off_first[tb]);
  int32_t* tail = at<int32_t>(hb, L.off_tail[tb]);
  int32_t* orun = at<int32_t>(hb, L.off_orun[tb]);
  int32_t* ocnt = at<int32_t>(hb, L.off_ocnt[tb]);
  const int os = owner == ICE_ROOT ? L.cap : owner;
  const int tl = tail[os];
  if (tl >= 0 && pg_cnt[tl] < ICE_PAGE_CAP) {
    ocnt[os] += 1;
    page = tl;
    slot = pg_cnt[tl];
    pg_cnt[tl] = slot + 1;
    pg_tok[(int64_t)tl * ICE_PAGE_CAP + slot] = t;
    return true;
  }
  const int p = hdr->n_pages[tb];
  if (p >= L.pcap[tb]) return false;
  hdr->n_pages[tb] = p + 1;
  if (tl >= 0) {
    pg_next[tl] = p;
    if (tb == 0) hdr->splits += 1;   // a KV page split off; upper tables only chain storage blocks
    // the contiguous run grows while the new page directly follows it
    if (tl == first[os] + orun[os] - 1 && p == tl + 1) orun[os] += 1;
  } else {
    first[os] = p;
    orun[os] = 1;
  }
  ocnt[os] += 1;
  tail[os] = p;
  pg_owner[p] = owner;
  pg_next[p] = -1;
  pg_cnt[p] = 1;
  pg_tok[(int64_t)p * ICE_PAGE_CAP] = t;
  for (int s = 1; s < ICE_PAGE_CAP; ++s) pg_tok[(int64_t)p * ICE_PAGE_CAP + s] = -1;
  page = p;
  slot = 0;
  return true;
}

// The parent search's row dot products: 4 lanes per row, lane part p holding
// the row's 16-byte pieces p, p + 4, ... (one 64-byte segment per load across
// the row's lanes); bf16 rows use v_dot2 (exact products, fp32 sums).
template <int D, class T>
struct QuadRow {
  static constexpr int NL = D * (int)sizeof(T) / 64;   // 16-byte pieces per lane
  V4 q[NL];
  __device__ inline void load(const T* row, int part) {
#pragma unroll
    for (int i = 0; i < NL; ++i) q[i] = *reinterpret_cast<const V4*>(reinterpret_cast<const char*>(row) + 16 * (part + 4 * i));
  }
  __device__ inline void fetch(const T* row, int part, V4 (&out)[NL]) const {
#pragma unroll
    for (int i = 0; i < NL; ++i) out[i] = *reinterpret_cast<const V4*>(reinterpret_cast<const char*>(row) + 16 * (part + 4 * i));
  }
  // q . row over the row's 4 lanes (every one of them gets the sum)
  __device__ inline float dot(const V4 (&k)[NL]) const {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      if constexpr (sizeof(T) == 2) {
        typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, k[i].x), __builtin_bit_cast(bf2, q[i].x), s, false);
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, k[i].y), __builtin_bit_cast(bf2, q[i].y), s, false);
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, k[i].z), __builtin_bit_cast(bf2, q[i].z), s, false);
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, k[i].w), __builtin_bit_cast(bf2, q[i].w), s, false);
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

// (score desc, token asc) running best and runner-up
struct BestTok {
  float best = -INFINITY, second = -INFINITY;
  int tok = 0x7fffffff;
  __device__ inline void push(float s, int t) {
    if (s > best || (s == best && t < tok)) {
      second = best;
      best = s;
      tok = t;
    } else {
      second = fmaxf(second, s);
    }
  }
  __device__ inline void merge(float ob, float os, int ot) {
    if (ob > best || (ob == best && ot < tok)) {
      second = fmaxf(best, os);
      best = ob;
      tok = ot;
    } else {
      second = fmaxf(second, ob);
    }
  }
};

constexpr int kInsertWaves = 16;

// LDS of the re-sort split: the owner's chain, its members in chain order,
// their keys and destinations, and a staging area for the row moves.
struct ResplitLds {
  int32_t pages[ICE_RESPLIT_MAX / ICE_PAGE_CAP];
  int32_t tok[ICE_RESPLIT_MAX];
  int32_t dst[ICE_RESPLIT_MAX];
  double key[ICE_RESPLIT_MAX];
  int32_t opos, bad;
  alignas(16) char stage[32768];
};

// Position r of the owner's chain -> row of the page pool.
__device__ inline int64_t chain_row(const ResplitLds& R, int r) {
  return (int64_t)R.pages[r / ICE_PAGE_CAP] * ICE_PAGE_CAP + r % ICE_PAGE_CAP;
}

// Re-packs the n members of `owner` (chain pages already in R.pages, n <=
// ICE_RESPLIT_MAX, every page full but the last) in the order the build packs
// them: the owner first, then ascending lifted squared distance to the owner
// (fp64, from the stored rows and lift coordinates), ties by token id. Page
// ids, counts and chains stay; the page table's token ids and the K and V
// rows are permuted. Called by every thread of the block.
template <int D, class T, int NT>
__device__ void resplit_owner(const DevLayout& L, void* hb, int h, int owner, int n, ResplitLds& R) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int NW = NT / 64;
  constexpr int EPL = D / 64;              // row elements per lane
  int32_t* pg_tok = at<int32_t>(hb, L.off_pg_tok[0]);
  T* K = at<T>(hb, L.off_pgK[0]);
  T* V = reinterpret_cast<T*>(v_pages(L, hb, h));
  const float* eall = at<float>(hb, L.off_e);
  if (tid == 0) {
    R.opos = n;
    R.bad = 0;
  }
  __syncthreads();
  for (int i = tid; i < n; i += NT) {
    const int t = pg_tok[chain_row(R, i)];
    R.tok[i] = t;
    if (t == owner) atomicMin(&R.opos, i);
    if (t < 0 || t >= L.cap) atomicOr(&R.bad, 1);
  }
  __syncthreads();
  const int opos = R.opos;
  // the owner missing from its chain, or an empty slot among the members:
  // not a layout the inserts build, so the pages are left as they are
  if (opos >= n || R.bad) return;
  // squared distance to the owner: one wave per member, lanes over the dims
  float ko[EPL];
  const int64_t orow = chain_row(R, opos) * D;
#pragma unroll
  for (int j = 0; j < EPL; ++j) ko[j] = Elt<T>::load(K, orow + lane + 64 * j);
  const double eo = (double)eall[owner];
  for (int i = wave; i < n; i += NW) {
    const int64_t row = chain_row(R, i) * D;
    double acc = 0.0;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const double df = (double)Elt<T>::load(K, row + lane + 64 * j) - (double)ko[j];
      acc += df * df;
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) acc += __shfl_xor(acc, m, 64);
    if (lane == 0) {
      const double de = (double)eall[R.tok[i]] - eo;
      double dk = acc + de * de;
      if (!(dk >= 0.0)) dk = INFINITY;     // NaN rows sort last, so the order stays total
      R.key[i] = i == opos ? -1.0 : dk;    // the owner leads its run
    }
  }
  __syncthreads();
  // destination = rank under (key, token): a strict total order, so the
  // ranks are a permutation of 0..n-1
  for (int i = tid; i < n; i += NT) {
    const double ki = R.key[i];
    const int ti = R.tok[i];
    int rank = 0;
    for (int j = 0; j < n; ++j) {
      const double kj = R.key[j];
      rank += (kj < ki || (kj == ki && R.tok[j] < ti)) ? 1 : 0;
    }
    R.dst[i] = rank;
  }
  __syncthreads();
  for (int i = tid; i < n; i += NT) pg_tok[chain_row(R, R.dst[i])] = R.tok[i];
  // rows move through LDS, C dims of every member at a time
  T* stg = reinterpret_cast<T*>(R.stage);
  constexpr int E = (int)(sizeof(R.stage) / sizeof(T));
  int C = D;
  while (n * C > E) C >>= 1;
  for (int pass = 0; pass < 2; ++pass) {
    for (int c0 = 0; c0 < D; c0 += C) {
      for (int x = tid; x < n * C; x += NT) {
        const int i = x / C, c = x % C;
        const int64_t r = chain_row(R, i);
        const int64_t src = pass == 0 ? r * D + c0 + c
                                      : ((r / ICE_PAGE_CAP * 4 + r % ICE_PAGE_CAP / 4) * D + c0 + c) * 4 + r % 4;
        stg[R.dst[i] * C + c] = pass == 0 ? K[src] : V[src];
      }
      __syncthreads();
      for (int x = tid; x < n * C; x += NT) {
        const int i = x / C, c = x % C;
        const int64_t r = chain_row(R, i);
        const int64_t dst = pass == 0 ? r * D + c0 + c
                                      : ((r / ICE_PAGE_CAP * 4 + r % ICE_PAGE_CAP / 4) * D + c0 + c) * 4 + r % 4;
        (pass == 0 ? K : V)[dst] = stg[i * C + c];
      }
      __syncthreads();
    }
  }
}

template <int D, class T>
__global__ __launch_bounds__(kInsertWaves * 64) void k_insert(DevLayout L, void* blob, const T* knew, const T* vnew,
                                                              int n_new, int t0) {
  using QR = QuadRow<D, T>;
  constexpr int NW = kInsertWaves;
  const int h = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  void* hb = head_base(blob, L, h);
  Hdr* hdr = at<Hdr>(hb, L.off_hdr);
  const int Ltop = hdr->top_level;
  const double M2 = hdr->M2;
  int8_t* lev = at<int8_t>(hb, L.off_lev);
  float* eall = at<float>(hb, L.off_e);

  __shared__ double red_d[NW];
  __shared__ float red_s[NW], red_s2[NW];
  __shared__ int red_t[NW];
  __shared__ Place plc;
  __shared__ float e_sh;
  __shared__ int rs_owner, rs_n;
  __shared__ ResplitLds rs;

  for (int j = 0; j < n_new; ++j) {
    const int t = t0 + j;
    const T* krow = knew + ((int64_t)h * n_new + j) * D;
    const T* vrow = vnew + ((int64_t)h * n_new + j) * D;
    // |k|^2 in fp64 and the lift coordinate with the build's M^2
    double sq = 0.0;
    if (tid < D) {
      const float x = Elt<T>::load(krow, tid);
      sq = (double)x * (double)x;
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) sq += __shfl_xor(sq, m, 64);
    if (lane == 0) red_d[wave] = sq;
    __syncthreads();
    double n2 = 0.0;
    for (int w = 0; w < NW; ++w) n2 += red_d[w];
    const float et = (float)sqrt(fmax(0.0, M2 - n2));
    const int lam = min(Ltop, draw_level(L.seed, L.h0 + h, t, L.L, L.plog2));

    // parent at level lam among the current points of level lam+1: 16 rows
    // per wave pass, U passes' loads in flight, then a (score desc, token
    // asc) reduction over the lanes, the waves and the block
    if (lam < Ltop) {
      const int tb = lam + 1;
      const bool from_top = tb == Ltop;
      const int nrows = from_top ? hdr->n_top : hdr->n_pages[tb] * ICE_PAGE_CAP;
      const int32_t* toks = from_top ? at<int32_t>(hb, L.off_top_tok) : at<int32_t>(hb, L.off_pg_tok[tb]);
      const T* rows = from_top ? at<T>(hb, L.off_top_K) : at<T>(hb, L.off_pgK[tb]);
      const float* es = from_top ? at<float>(hb, L.off_top_E) : at<float>(hb, L.off_pgE[tb]);
      const int part = lane & 3;
      QR qr;
      qr.load(krow, part);
      BestTok bt;
      // passes in flight per wave (within 128 VGPRs)
      constexpr int U = QR::NL >= 8 ? 1 : 2;
      constexpr int STEP = U * NW * 16;
      // token ids run one iteration ahead of the rows, so that the empty
      // slots of partly filled pages (token -1) are never read
      auto tok_at = [&](int r) { return r < nrows ? toks[r] : -1; };
      int tokn[U];
#pragma unroll
      for (int u = 0; u < U; ++u) tokn[u] = tok_at(wave * 16 + u * NW * 16 + (lane >> 2));
      for (int r0 = wave * 16; r0 < nrows; r0 += STEP) {
        int tok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          tok[u] = tokn[u];
          tokn[u] = tok_at(r0 + STEP + u * NW * 16 + (lane >> 2));
        }
        V4 buf[U][QR::NL] = {};
        float ev[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int r = r0 + u * NW * 16 + (lane >> 2);
          // an empty slot's lanes load nothing and score 0, never pushed (a
          // row's 4 lanes agree, so the quad sum stays within the row)
          ev[u] = 0.0f;
          if (tok[u] >= 0) {
            ev[u] = es[r];
            qr.fetch(rows + (int64_t)r * D, part, buf[u]);
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float sc = fmaf(et, ev[u], qr.dot(buf[u]));
          if (tok[u] >= 0) bt.push(sc, tok[u]);
        }
      }
#pragma unroll
      for (int m = 1; m < 64; m <<= 1)
        bt.merge(__shfl_xor(bt.best, m, 64), __shfl_xor(bt.second, m, 64), __shfl_xor(bt.tok, m, 64));
      if (lane == 0) {
        red_s[wave] = bt.best;
        red_s2[wave] = bt.second;
        red_t[wave] = bt.tok;
      }
    }
    __syncthreads();
    if (tid == 0) {
      int p = -1;
      if (lam < Ltop) {
        BestTok bt;
        for (int w = 0; w < NW; ++w) bt.merge(red_s[w], red_s2[w], red_t[w]);
        const float best = bt.best, second = bt.second;
        p = bt.tok;
        if (p < 0 || p >= t || lev[p] < lam + 1) {
          // only when every score was NaN (non-finite input): take any point
          // of the next level instead of indexing out of range
          const int tb = lam + 1;
          if (tb == Ltop) {
            p = at<int32_t>(hb, L.off_top_tok)[0];
          } else {
            const int32_t* toks = at<int32_t>(hb, L.off_pg_tok[tb]);
            p = toks[0];
          }
        }
        const float m2f = (float)M2;
        if (second > -INFINITY && (best - second) < 1e-4f * (m2f - second)) hdr->near_ties += 1;
      }
      if (n2 > M2) hdr->clamps += 1;
      for (int l = 0; l < ICE_MAX_LEVELS; ++l) plc.page[l] = plc.slot[l] = -1;
      plc.top_slot = -1;
      bool ok = true;
      // level 0 (the KV page pool)
      const int owner0 = Ltop == 0 ? ICE_ROOT : (lam >= 1 ? t : p);
      ok &= place_token(L, hb, hdr, 0, owner0, t, plc.page[0], plc.slot[0]);
      // upper tables: t owns a new child list below its level, joins p's at it
      for (int l = 1; l < Ltop; ++l) {
        if (lam > l) ok &= place_token(L, hb, hdr, l, t, t, plc.page[l], plc.slot[l]);
        else if (lam == l) ok &= place_token(L, hb, hdr, l, p, t, plc.page[l], plc.slot[l]);
      }
      if (Ltop >= 1 && lam == Ltop) {
        // the top list is sized for every promoted position; the host rejects
        // inserts that could outgrow it, and a full list is flagged, not written past
        if (hdr->n_top < L.topcap) {
          plc.top_slot = hdr->n_top;
          at<int32_t>(hb, L.off_top_tok)[hdr->n_top] = t;
          hdr->n_top += 1;
        } else {
          ok = false;
        }
      }
      for (int l = 0; l < Ltop; ++l) {
        int32_t* par = at<int32_t>(hb, L.off_parent[l]);
        if (l < lam) par[t] = t;
        else if (l == lam) par[t] = p;
      }
      lev[t] = (int8_t)lam;
      eall[t] = et;
      if (!ok) hdr->overflow = 1;   // page table overflow (ruled out by the capacity bound)
      e_sh = et;
      // re-sort split: a token owner whose chain just grew a page (the new
      // token took slot 0 of a page that is not its first)
      rs_n = 0;
      rs_owner = owner0;
      if (L.resort && owner0 != ICE_ROOT && plc.page[0] >= 0 && plc.slot[0] == 0) {
        const int32_t* first0 = at<int32_t>(hb, L.off_first[0]);
        const int32_t* orun0 = at<int32_t>(hb, L.off_orun[0]);
        const int32_t* next0 = at<int32_t>(hb, L.off_pg_next[0]);
        const int n_mem = at<int32_t>(hb, L.off_ocnt[0])[owner0];
        const int n_pg = (n_mem + ICE_PAGE_CAP - 1) / ICE_PAGE_CAP;
        if (first0[owner0] != plc.page[0] && n_mem <= ICE_RESPLIT_MAX) {
          // the chain: the contiguous run from first[], then the links
          const int run = max(1, min(orun0[owner0], n_pg));
          int pg = first0[owner0];
          int k = 0;
          for (; k < run; ++k) rs.pages[k] = pg + k;
          pg = next0[pg + run - 1];
          for (; k < n_pg && pg >= 0; ++k, pg = next0[pg]) rs.pages[k] = pg;
          if (k == n_pg && rs.pages[n_pg - 1] == plc.page[0]) rs_n = n_mem;
        }
      }
    }
    __syncthreads();
    // a page created by this insert gets zero rows besides the new token, so
    // every row of every page holds finite values
    for (int l = 0; l < Ltop || l == 0; ++l) {
      if (plc.page[l] < 0 || plc.slot[l] != 0) continue;
      const int64_t base = (int64_t)plc.page[l] * ICE_PAGE_CAP;
      for (int i = tid + D; i < ICE_PAGE_CAP * D; i += NW * 64) {
        at<T>(hb, L.off_pgK[l])[base * D + i] = T(0);
        if (l != 0 && i % D == 0) at<float>(hb, L.off_pgE[l])[base + i / D] = 0.0f;
      }
      // V pages ([slot group][dim][4 slots]): every element but slot 0's
      if (l == 0)
        for (int i = tid; i < ICE_PAGE_CAP * D; i += NW * 64)
          if (i % 4 != 0 || i >= 4 * D) reinterpret_cast<T*>(v_pages(L, hb, h))[base * D + i] = T(0);
    }
    // rows into the pools
    for (int i = tid; i < D; i += NW * 64) {
      const T kv = krow[i];
      if (plc.page[0] >= 0) {
        const int64_t row = (int64_t)plc.page[0] * ICE_PAGE_CAP + plc.slot[0];
        at<T>(hb, L.off_pgK[0])[row * D + i] = kv;
        const int sl = plc.slot[0];
        reinterpret_cast<T*>(v_pages(L, hb, h))[(((int64_t)plc.page[0] * 4 + sl / 4) * D + i) * 4 + sl % 4] = vrow[i];
      }
      for (int l = 1; l < Ltop; ++l) {
        if (plc.page[l] < 0) continue;
        const int64_t row = (int64_t)plc.page[l] * ICE_PAGE_CAP + plc.slot[l];
        at<T>(hb, L.off_pgK[l])[row * D + i] = kv;
        if (i == 0) at<float>(hb, L.off_pgE[l])[row] = e_sh;
      }
      if (plc.top_slot >= 0) {
        at<T>(hb, L.off_top_K)[(int64_t)plc.top_slot * D + i] = kv;
        if (i == 0) at<float>(hb, L.off_top_E)[plc.top_slot] = e_sh;
      }
    }
    __threadfence_block();
    __syncthreads();
    if (rs_n > 0) {
      resplit_owner<D, T, NW * 64>(L, hb, h, rs_owner, rs_n, rs);
      __threadfence_block();
      __syncthreads();
    }
  }
  if (tid == 0) hdr->n_tokens = t0 + n_new;
}

}  // namespace

hipError_t launch_insert(const DevLayout& L, void* blob, const void* k_new, const void* v_new, int n_new, int t0,
                         hipStream_t s) {
  if (n_new <= 0) return hipSuccess;
  const dim3 grid((unsigned)L.H);
  if (L.dtype == ICE_BF16) {
    const uint16_t* k = static_cast<const uint16_t*>(k_new);
    const uint16_t* v = static_cast<const uint16_t*>(v_new);
    if (L.d == 128) k_insert<128, uint16_t><<<grid, kInsertWaves * 64, 0, s>>>(L, blob, k, v, n_new, t0);
    else k_insert<64, uint16_t><<<grid, kInsertWaves * 64, 0, s>>>(L, blob, k, v, n_new, t0);
  } else {
    const float* k = static_cast<const float*>(k_new);
    const float* v = static_cast<const float*>(v_new);
    if (L.d == 128) k_insert<128, float><<<grid, kInsertWaves * 64, 0, s>>>(L, blob, k, v, n_new, t0);
    else k_insert<64, float><<<grid, kInsertWaves * 64, 0, s>>>(L, blob, k, v, n_new, t0);
  }
  return hipGetLastError();
}

}  // namespace ice
