// Sparse attention of one head on the matrix cores (bf16), shared by the
// attention kernel and the fused decode kernel.
//
// The papernotes.org IceCache notes (key design 1) give the weight of token j
// for query i as s_ij exp(q_i.k_j/sqrt d) / sum_j' s_ij' exp(q_i.k_j'/sqrt d),
// with s the selection mask: a softmax over the tokens of the selected pages
// only; every query head of a GQA group attends the group's page union (key
// design 3).
//
// Per page the work is two small dense products for the whole group, run as
// 16x16 MFMA tiles with all G <= 16 query heads in one tile:
// S^T (16 tokens x 16 queries) = K (16 x d) . Q^T (d x 16) with
// v_mfma_f32_16x16x32_bf16: lane l holds, for the d-chunk c of 32,
//   A = K[token l%16][32c + 8(l/16) .. +7]   (16 contiguous bytes of a row)
//   B = Q[query l%16][32c + 8(l/16) .. +7]
// and receives S^T[token 4(l/16)+j][query l%16], j < 4. So each lane holds 4
// tokens of one query: the softmax of a query is a max/sum over the lane's 4
// values and its 3 partner lanes l^16, l^32, l^48; and the weights are
// already laid out as the B operand of
// O^T (16 dims x 16 queries) += V^T (16 dims x 16 tokens) . P^T (16 tokens x
// 16 queries) with v_mfma_f32_16x16x16_bf16: A = V[tokens 4(l/16) .. +3][dim
// 16c + l%16] (one 8-byte piece of the V page), B = P[query l%16][tokens
// 4(l/16) .. +3], result O[query l%16][dim 16c + 4(l/16) + j]: every lane's
// accumulators belong to its own query, so the online-softmax rescale (running
// base m and sum l per query) needs no lane exchange; the base only moves when
// a page's max exceeds it by more than kSlack, so rescales are rare. P goes in as a bf16 pair
// hi + lo (p = hi + lo to 16 bits), two MFMAs per tile, so the weights keep
// fp32-level accuracy. Logits are kept in base 2 (scaled by scale * log2 e).
//
// The waves of the block take the union pages round-robin and keep the next
// page's loads in flight while the current page is used; their (m, l, o)
// partials are merged in LDS. Page pools: K pages are [page][slot][d]; V pages
// are [page][slot group g = slot/4][d][4 slots]. Loads are unconditional:
// rows and slot groups past a page's count re-read its last valid ones
// (already in cache, no extra memory traffic), and those tokens get weight 0.
#pragma once

#include "ice_common.h"

namespace ice {
namespace mfma_attend {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSlack = 8.0f;        // log2 headroom of the running softmax base

template <int D>
struct MGeo {
  static constexpr int KC = D / 32;   // 32-dim chunks of S
  static constexpr int VC = D / 16;   // 16-dim tiles of O
  static constexpr int ROWB = D * 2;
};

template <int D>
struct MPage {
  V4 k[MGeo<D>::KC];
  uint2 v[MGeo<D>::VC];     // used when V is prefetched with K
};

// 32-bit byte offsets from the head's pools (a head's pool is far below 4 GiB)
template <int D>
__device__ inline void mload_k(const char* pgK, int pg, int cnt, int lane, MPage<D>& r) {
  using M = MGeo<D>;
  const uint32_t page = (uint32_t)pg * (ICE_PAGE_CAP * M::ROWB);
  const int last = cnt > 0 ? cnt - 1 : 0;
  const uint32_t koff = page + (uint32_t)min(lane & 15, last) * M::ROWB + (lane >> 4) * 16;
#pragma unroll
  for (int c = 0; c < M::KC; ++c) r.k[c] = *reinterpret_cast<const V4*>(pgK + (koff + 64 * c));
}
template <int D>
__device__ inline void mload_v(const char* pgV, int pg, int cnt, int lane, uint2 (&v)[MGeo<D>::VC]) {
  using M = MGeo<D>;
  const uint32_t page = (uint32_t)pg * (ICE_PAGE_CAP * M::ROWB);
  const int last = cnt > 0 ? cnt - 1 : 0;
  const int g = min(lane >> 4, last >> 2);
  const uint32_t voff = page + (uint32_t)(g * D + (lane & 15)) * 8;
#pragma unroll
  for (int c = 0; c < M::VC; ++c) v[c] = *reinterpret_cast<const uint2*>(pgV + (voff + 128 * c));
}

__device__ inline uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// LDS floats of attend_head: the Q^T operand (16 queries x D bf16) and the
// partials of `nw` waves for G query heads
__host__ __device__ inline int part_floats(int nw, int G, int D) {
  return 8 * D + 2 * nw * ICE_MAX_GROUP + nw * G * D;
}

// One wave's running softmax state over the pages it has attended: base m
// and sum l of its lane's query, and O^T accumulators.
template <int D>
struct WaveAcc {
  float m, l;
  float4v acc[MGeo<D>::VC];
  __device__ inline void init() {
    m = -INFINITY;
    l = 0.0f;
#pragma unroll
    for (int c = 0; c < MGeo<D>::VC; ++c) acc[c] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
  }
};

// The Q^T operand in LDS (read once per page), queries past G zero: every
// thread of the block takes part; the caller synchronises before use.
template <int D>
__device__ inline void stage_q(const uint16_t* Qh, int G, float* part) {
  using M = MGeo<D>;
  V4* q_lds = reinterpret_cast<V4*>(part);          // [KC][4 parts][16 queries]: lane l reads entry c*64 + l
  for (int t = threadIdx.x; t < M::KC * 16 * 4; t += blockDim.x) {
    const int c = t / 64, part4 = (t >> 4) & 3, q = t & 15;     // entry c*64 + lane of lane (q, part4)
    const V4 x = *reinterpret_cast<const V4*>(reinterpret_cast<const char*>(Qh + (int64_t)min(q, G - 1) * D) +
                                               64 * c + 16 * part4);
    q_lds[t] = q < G ? x : V4{0, 0, 0, 0};
  }
}

// One page into a wave's running softmax state (m, l, acc): the scores of
// its first `cnt` tokens for every query (S^T = K Q^T), their weights
// against the running base, and O^T += V^T P^T. k: the lane's K pieces, v:
// its V pieces (mload_k / mload_v); q_lds: the staged Q^T; c2: the scale in
// base 2. cnt = 0 leaves the state unchanged.
template <int D>
__device__ inline void page_update(const V4 (&k)[MGeo<D>::KC], const uint2 (&v)[MGeo<D>::VC], int cnt, float c2,
                                   const V4* q_lds, int lane, float& m, float& l, float4v (&acc)[MGeo<D>::VC]) {
  using M = MGeo<D>;
  const int qt = lane >> 4;     // 4-token group of the lane (its query is lane % 16)
  float4v s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int c = 0; c < M::KC; ++c) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf16x8, k[c]), __builtin_bit_cast(bf16x8, q_lds[c * 64 + lane]), s, 0, 0, 0);
  float x[4];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[j] = 4 * qt + j < cnt ? s[j] * c2 : -INFINITY;
    mx = fmaxf(mx, x[j]);
  }
  mx = fmaxf(mx, xor_lane_f<16>(mx));
  mx = fmaxf(mx, xor_lane_f<32>(mx));
  // The running base m moves only when a page's max exceeds it by more
  // than kSlack (weights stay below 2^kSlack, harmless in fp32), so the
  // accumulators are rescaled on few pages only.
  const bool move = mx > m + kSlack;
  const float mn = move ? mx : m;
  const float corr = move ? (m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - mn)) : 1.0f;
  const bool any_move = __ballot(move) != 0;   // uniform over the wave
  float p[4], rs = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    p[j] = x[j] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x[j] - mn);
    rs += p[j];
  }
  rs += xor_lane_f<16>(rs);
  rs += xor_lane_f<32>(rs);
  l = l * corr + rs;
  m = mn;
  // P = hi + lo in bf16 (round to nearest even), as the B operand (query
  // qn, tokens 4qt .. 4qt+3)
  short4v phi, plo;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const __bf16 hi = (__bf16)p[j];
    phi[j] = __builtin_bit_cast(short, hi);
    plo[j] = __builtin_bit_cast(short, (__bf16)(p[j] - (float)hi));
  }
  if (any_move)
#pragma unroll
    for (int c = 0; c < M::VC; ++c) acc[c] *= corr;
#pragma unroll
  for (int c = 0; c < M::VC; ++c) {
    const short4v va = __builtin_bit_cast(short4v, v[c]);
    acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, phi, acc[c], 0, 0, 0);
    acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, plo, acc[c], 0, 0, 0);
  }
}

// One wave attends entries wi, wi + ws, ... of the head's page source (the
// union or, for a dense head, every page; then the resident pages; union ids
// outside the head's page table are skipped) for the head's G query heads,
// into `st`. part holds the staged Q^T. With staged V (host-pool mode, which
// has neither dense heads nor resident pages) the V page of entry i is
// staging entry i.
template <int D, bool PREFETCH_V>
__device__ void attend_pages(const DevLayout& L, const void* hb, int h, int G, const PageSrc& src, int wi, int ws,
                             float c2, const float* part, WaveAcc<D>& st) {
  using M = MGeo<D>;
  const V4* q_lds = reinterpret_cast<const V4*>(part);
  const int lane = threadIdx.x & 63;
  const char* pgK = at<char>(hb, L.off_pgK[0]);
  const bool staged = L.vstage != nullptr;
  const char* pgV = staged ? L.vstage + (int64_t)h * L.vstage_pages * (ICE_PAGE_CAP * M::ROWB) : v_pages(L, hb, h);
  const int32_t* pg_cnt = at<int32_t>(hb, L.off_pg_cnt[0]);
  float m = st.m, l = st.l;
  float4v acc[M::VC];
#pragma unroll
  for (int c = 0; c < M::VC; ++c) acc[c] = st.acc[c];
  (void)G;

  const int nu = src.count();
  const int npw = nu > wi ? (nu - wi + ws - 1) / ws : 0;
  for (int k0 = 0; k0 < npw; k0 += 64) {
    int my_pg = -1, my_cnt = 0;
    if (k0 + lane < npw) {
      my_pg = src.at(wi + ws * (k0 + lane));
      if (my_pg >= 0) my_cnt = pg_cnt[my_pg];
    }
    const int nk = min(64, npw - k0);
    // Two page buffers with fixed roles in each half of an unrolled pair of
    // steps: page k is used from one while page k+1 loads into the other. The
    // steps are straight-line code (page ids are picked with clamped indices
    // and selects, a missing page is masked rather than skipped) so the
    // compiler's wait counts stay exact and the next page stays in flight.
    MPage<D> bufA, bufB;
    auto issue = [&](int k, MPage<D>& b) {
      const int kc = min(k, nk - 1);
      const int pg = __shfl(my_pg, kc, 64), cnt = __shfl(my_cnt, kc, 64);
      const bool ok = k < nk && pg >= 0;
      mload_k<D>(pgK, ok ? pg : 0, ok ? cnt : 0, lane, b);
      if constexpr (PREFETCH_V) mload_v<D>(pgV, ok ? (staged ? wi + ws * (k0 + kc) : pg) : 0, ok ? cnt : 0, lane, b.v);
    };
    issue(0, bufA);
    auto step = [&](int k, MPage<D>& cur, MPage<D>& nxt) {
      const int kc = min(k, nk - 1);
      const int pg_k = __shfl(my_pg, kc, 64), cnt_k = __shfl(my_cnt, kc, 64);
      const int cnt = k < nk && pg_k >= 0 ? cnt_k : 0;      // 0: nothing to attend
      uint2 vcur[M::VC];
      if constexpr (!PREFETCH_V) mload_v<D>(pgV, cnt > 0 ? (staged ? wi + ws * (k0 + kc) : pg_k) : 0, cnt, lane, vcur);
      issue(k + 1, nxt);
      if constexpr (PREFETCH_V) page_update<D>(cur.k, cur.v, cnt, c2, q_lds, lane, m, l, acc);
      else page_update<D>(cur.k, vcur, cnt, c2, q_lds, lane, m, l, acc);
    };
    for (int k = 0; k < nk; k += 2) {
      step(k, bufA, bufB);
      step(k + 1, bufB, bufA);
    }
  }
  st.m = m;
  st.l = l;
#pragma unroll
  for (int c = 0; c < M::VC; ++c) st.acc[c] = acc[c];
}

// A wave's partials (m, l and o of query qn; every lane group holds m and l,
// lane group qt holds dims 16c + 4qt + j) into slot wv (< nw) of the LDS
// partials.
template <int D>
__device__ inline void write_partial(const WaveAcc<D>& st, int wv, int G, float* part, int nw) {
  using M = MGeo<D>;
  float* part_m = part + 8 * D;
  float* part_l = part_m + nw * ICE_MAX_GROUP;
  float* part_o = part_l + nw * ICE_MAX_GROUP;     // [nw][G][D]
  const int lane = threadIdx.x & 63;
  const int qn = lane & 15, qt = lane >> 4;
  if (qt == 0 && qn < G) {
    part_m[wv * ICE_MAX_GROUP + qn] = st.m;
    part_l[wv * ICE_MAX_GROUP + qn] = st.l;
  }
  if (qn < G)
#pragma unroll
    for (int c = 0; c < M::VC; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) part_o[(wv * G + qn) * D + 16 * c + 4 * qt + j] = st.acc[c][j];
}

// Merges the partials in slots 0 .. nused-1 of an area laid out for nw slots
// (nused = nw: every wave's; after a block barrier that follows every
// write_partial) in one pass, in slot order: every output element's thread
// forms its query's common base, total weight and the slots' normalised
// factors itself (the reads of one query's m and l are LDS broadcasts across
// a wave).
template <int D>
__device__ inline void merge_partials(int G, const float* part, int nw, float* Oh, float* lseh, int nused = -1) {
  const float* part_m = part + 8 * D;
  const float* part_l = part_m + nw * ICE_MAX_GROUP;
  const float* part_o = part_l + nw * ICE_MAX_GROUP;
  const int ns = nused < 0 ? nw : nused;
  for (int t = threadIdx.x; t < G * D; t += blockDim.x) {
    const int q = t / D, dd = t % D;
    float Mx = -INFINITY;
    for (int w = 0; w < ns; ++w) Mx = fmaxf(Mx, part_m[w * ICE_MAX_GROUP + q]);
    float Ls = 0.0f, a = 0.0f;
    for (int w = 0; w < ns; ++w) {
      const float mw = part_m[w * ICE_MAX_GROUP + q];
      const float f = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - Mx);
      Ls = fmaf(part_l[w * ICE_MAX_GROUP + q], f, Ls);
      a = fmaf(part_o[(w * G + q) * D + dd], f, a);
    }
    Oh[(int64_t)q * D + dd] = Ls > 0.0f ? a / Ls : 0.0f;
    if (lseh && dd == 0) lseh[q] = Ls > 0.0f ? (Mx + __log2f(Ls)) * kLn2 : -INFINITY;
  }
}

// Attention of head h for its G query heads over the nu page ids u[0..nu)
// (or every page, for a dense head) and the head's resident pages, by the
// whole block: wave w takes entries w, w + nw, ... Qh: the head's
// [G][D] queries; Oh: [G][D] outputs; lseh nullable. part: LDS of
// part_floats(nw, G, D) floats; nw: waves of the block (all of them call).
template <int D, bool PREFETCH_V>
__device__ void attend_head(const DevLayout& L, const void* hb, const uint16_t* Qh, int G, const int32_t* u, int nu,
                            float scale, float* Oh, float* lseh, float* part, int nw) {
  const int wv = threadIdx.x >> 6;
  stage_q<D>(Qh, G, part);
  __syncthreads();
  WaveAcc<D> st;
  st.init();
  attend_pages<D, PREFETCH_V>(L, hb, blockIdx.x, G, page_src(L, hb, u, nu), wv, nw, scale * kLog2e, part, st);
  write_partial<D>(st, wv, G, part, nw);
  __syncthreads();
  merge_partials<D>(G, part, nw, Oh, lseh);
}

}  // namespace mfma_attend
}  // namespace ice
