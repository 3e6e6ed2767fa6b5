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
// split page that becomes the owner's last page. Resident tokens never move.
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

template <int D, class T>
__global__ __launch_bounds__(256) void k_insert(DevLayout L, void* blob, const T* knew, const T* vnew, int n_new,
                                                int t0) {
  using G = RowGeo<D, T>;
  const int h = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  void* hb = head_base(blob, L, h);
  Hdr* hdr = at<Hdr>(hb, L.off_hdr);
  const int Ltop = hdr->top_level;
  const double M2 = hdr->M2;
  int8_t* lev = at<int8_t>(hb, L.off_lev);
  float* eall = at<float>(hb, L.off_e);

  __shared__ __attribute__((aligned(16))) float kf[D];
  __shared__ double red_d[4];
  __shared__ float red_s[4], red_s2[4];
  __shared__ int red_t[4];
  __shared__ Place plc;
  __shared__ float e_sh;

  for (int j = 0; j < n_new; ++j) {
    const int t = t0 + j;
    const T* krow = knew + ((int64_t)h * n_new + j) * D;
    const T* vrow = vnew + ((int64_t)h * n_new + j) * D;
    // |k|^2 in fp64 and the lift coordinate with the build's M^2
    double sq = 0.0;
    if (tid < D) {
      const float x = Elt<T>::load(krow, tid);
      kf[tid] = x;
      sq = (double)x * (double)x;
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) sq += __shfl_xor(sq, m, 64);
    if (lane == 0) red_d[wave] = sq;
    __syncthreads();
    const double n2 = red_d[0] + red_d[1] + red_d[2] + red_d[3];
    const float et = (float)sqrt(fmax(0.0, M2 - n2));
    const int lam = min(Ltop, draw_level(L.seed, h, t, L.L, L.plog2));

    // parent at level lam among the current points of level lam+1
    float best = -INFINITY, second = -INFINITY;
    int btok = 0x7fffffff;
    if (lam < Ltop) {
      const int tb = lam + 1;
      const bool from_top = tb == Ltop;
      const int nrows = from_top ? hdr->n_top : hdr->n_pages[tb] * ICE_PAGE_CAP;
      const int32_t* toks = from_top ? at<int32_t>(hb, L.off_top_tok) : at<int32_t>(hb, L.off_pg_tok[tb]);
      const T* rows = from_top ? at<T>(hb, L.off_top_K) : at<T>(hb, L.off_pgK[tb]);
      const float* es = from_top ? at<float>(hb, L.off_top_E) : at<float>(hb, L.off_pgE[tb]);
      float q[G::EPL];
#pragma unroll
      for (int i = 0; i < G::EPL; ++i) q[i] = kf[(lane % G::LPR) * G::EPL + i];
      for (int r0 = wave * G::RPP; r0 < nrows; r0 += 4 * G::RPP) {
        const int r = r0 + lane / G::LPR;
        const int tok = r < nrows ? toks[r] : -1;
        float s = 0.0f;
        if (tok >= 0) {
          const V4 v = *reinterpret_cast<const V4*>(reinterpret_cast<const char*>(rows + (int64_t)r * D) +
                                                    (lane % G::LPR) * 16);
          float f[G::EPL];
          Elt<T>::unpack(v, f);
#pragma unroll
          for (int i = 0; i < G::EPL; ++i) s = fmaf(q[i], f[i], s);
        }
        s = group_sum<G::LPR>(s);
        if (tok >= 0) {
          s = fmaf(et, es[r], s);
          if (s > best || (s == best && tok < btok)) {
            second = best;
            best = s;
            btok = tok;
          } else {
            second = fmaxf(second, s);
          }
        }
      }
      // reduce (score desc, token asc) over the wave, then the block
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        const float ob = __shfl_xor(best, m, 64), os = __shfl_xor(second, m, 64);
        const int ot = __shfl_xor(btok, m, 64);
        if (ob > best || (ob == best && ot < btok)) {
          second = fmaxf(best, os);
          best = ob;
          btok = ot;
        } else {
          second = fmaxf(second, ob);
        }
      }
      if (lane == 0) {
        red_s[wave] = best;
        red_s2[wave] = second;
        red_t[wave] = btok;
      }
    }
    __syncthreads();
    if (tid == 0) {
      int p = -1;
      if (lam < Ltop) {
        best = red_s[0];
        second = red_s2[0];
        btok = red_t[0];
        for (int w = 1; w < 4; ++w) {
          if (red_s[w] > best || (red_s[w] == best && red_t[w] < btok)) {
            second = fmaxf(best, red_s2[w]);
            best = red_s[w];
            btok = red_t[w];
          } else {
            second = fmaxf(second, red_s[w]);
          }
        }
        p = btok;
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
        plc.top_slot = hdr->n_top;
        at<int32_t>(hb, L.off_top_tok)[hdr->n_top] = t;
        hdr->n_top += 1;
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
    }
    __syncthreads();
    // a page created by this insert gets zero rows besides the new token, so
    // every row of every page holds finite values
    for (int l = 0; l < Ltop || l == 0; ++l) {
      if (plc.page[l] < 0 || plc.slot[l] != 0) continue;
      const int64_t base = (int64_t)plc.page[l] * ICE_PAGE_CAP;
      for (int i = tid + D; i < ICE_PAGE_CAP * D; i += 256) {
        at<T>(hb, L.off_pgK[l])[base * D + i] = T(0);
        if (l != 0 && i % D == 0) at<float>(hb, L.off_pgE[l])[base + i / D] = 0.0f;
      }
      // V pages ([slot group][dim][4 slots]): every element but slot 0's
      if (l == 0)
        for (int i = tid; i < ICE_PAGE_CAP * D; i += 256)
          if (i % 4 != 0 || i >= 4 * D) reinterpret_cast<T*>(v_pages(L, hb, h))[base * D + i] = T(0);
    }
    // rows into the pools
    for (int i = tid; i < D; i += 256) {
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
    if (L.d == 128) k_insert<128, uint16_t><<<grid, 256, 0, s>>>(L, blob, k, v, n_new, t0);
    else k_insert<64, uint16_t><<<grid, 256, 0, s>>>(L, blob, k, v, n_new, t0);
  } else {
    const float* k = static_cast<const float*>(k_new);
    const float* v = static_cast<const float*>(v_new);
    if (L.d == 128) k_insert<128, float><<<grid, 256, 0, s>>>(L, blob, k, v, n_new, t0);
    else k_insert<64, float><<<grid, 256, 0, s>>>(L, blob, k, v, n_new, t0);
  }
  return hipGetLastError();
}

}  // namespace ice
