// Sparse attention over the selected pages.
//
// The papernotes.org IceCache notes (key design 1) give the weight of token j
// for query i as s_ij exp(q_i.k_j/sqrt d) / sum_j' s_ij' exp(q_i.k_j'/sqrt d),
// with s the selection mask: a softmax over the tokens of the selected pages
// only. Every query head of a GQA group attends the group's page union (key
// design 3).
//
// Per page the work is two small dense products for the whole group:
// S = K Q^T (16 tokens x G queries over d) and O += P V (G queries x d over
// 16 tokens), with an online softmax (running max m and sum l per query) in
// between. bf16 runs both products on the matrix cores (16x16 MFMA tiles, all
// G <= 16 query heads in one tile); fp32 runs them on the vector ALUs. Both
// kernels take one block per head, deal the union pages to the waves
// round-robin, keep the next page's loads in flight while the current page is
// used, and merge the waves' (m, l, o) partials in LDS. Logits are kept in
// base 2 (scaled by scale * log2 e).
//
// Page pools: K pages are [page][slot][d]; V pages are [page][slot group g =
// slot/4][d][4 slots], so a lane reads 4 consecutive slots of one dimension as
// one contiguous piece. Loads are unconditional: rows and slot groups past a
// page's count re-read its last valid ones (already in cache, no extra memory
// traffic), and those tokens get weight 0.
#include "ice_launch.h"

namespace ice {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ============================================================================
// bf16: matrix cores
// ============================================================================
// S^T (16 tokens x 16 queries) = K (16 x d) . Q^T (d x 16) with
// v_mfma_f32_16x16x32_bf16: lane l holds, for the d-chunk c of 32,
//   A = K[token l%16][32c + 8(l/16) .. +7]   (16 contiguous bytes of a row)
//   B = Q[query l%16][32c + 8(l/16) .. +7]
// and receives S^T[token 4(l/16)+j][query l%16], j < 4. So each lane holds 4
// tokens of one query: the softmax of a query is a max/sum over the lane's 4
// values and its 3 partner lanes l^16, l^32, l^48; and the weights are
// already laid out as the A operand of
// O (16 queries x 16 dims) += P (16 x 16 tokens) . V (16 tokens x 16 dims)
// with v_mfma_f32_16x16x16_bf16: A = P[query l%16][tokens 4(l/16) .. +3],
// B = V[tokens 4(l/16) .. +3][dim 16c + l%16] (one 8-byte piece of the V
// page), result O[query 4(l/16)+j][dim 16c + l%16]. P goes in as a bf16 pair
// hi + lo (p = hi + lo to 16 bits), two MFMAs per tile, so the weights keep
// fp32-level accuracy.

constexpr int kMW = 8;                // waves per block

template <int D>
struct MGeo {
  static constexpr int KC = D / 32;   // 32-dim chunks of S
  static constexpr int VC = D / 16;   // 16-dim tiles of O
  static constexpr int ROWB = D * 2;
};

template <int D>
struct MPage {
  V4 k[MGeo<D>::KC];
  uint2 v[MGeo<D>::VC];
};

// 32-bit byte offsets from the head's pools (a head's pool is far below 4 GiB)
template <int D>
__device__ inline void mload(const char* pgK, const char* pgV, int pg, int cnt, int lane, MPage<D>& r) {
  using M = MGeo<D>;
  const uint32_t page = (uint32_t)pg * (ICE_PAGE_CAP * M::ROWB);
  const int last = cnt > 0 ? cnt - 1 : 0;
  const uint32_t koff = page + (uint32_t)min(lane & 15, last) * M::ROWB + (lane >> 4) * 16;
#pragma unroll
  for (int c = 0; c < M::KC; ++c) r.k[c] = *reinterpret_cast<const V4*>(pgK + (koff + 64 * c));
  const int g = min(lane >> 4, last >> 2);
  const uint32_t voff = page + (uint32_t)(g * D + (lane & 15)) * 8;
#pragma unroll
  for (int c = 0; c < M::VC; ++c) r.v[c] = *reinterpret_cast<const uint2*>(pgV + (voff + 128 * c));
}

__device__ inline uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <int D>
__global__ __launch_bounds__(kMW * 64) void k_attend_mfma(DevLayout L, const void* blob, const uint16_t* Q,
                                                          const int32_t* uni, const int32_t* n_uni, int uni_stride,
                                                          float scale, float* O, float* lse) {
  using M = MGeo<D>;
  __shared__ float part_m[kMW][ICE_MAX_GROUP], part_l[kMW][ICE_MAX_GROUP];
  __shared__ float part_o[kMW][ICE_MAX_GROUP][D];
  __shared__ __attribute__((aligned(16))) float corr_lds[kMW][16];
  const int h = blockIdx.x;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int G = L.G;
  const int qn = lane & 15, qt = lane >> 4;     // query (B column, S^T column) and 4-token group
  const void* hb = head_base(blob, L, h);
  const char* pgK = at<char>(hb, L.off_pgK[0]);
  const char* pgV = at<char>(hb, L.off_pgV);
  const int32_t* pg_cnt = at<int32_t>(hb, L.off_pg_cnt[0]);
  const int n_pages = at<Hdr>(hb, L.off_hdr)->n_pages[0];
  const int nu = min(n_uni[h], uni_stride);
  const int32_t* u = uni + (int64_t)h * uni_stride;
  const float c2 = scale * kLog2e;

  // Q^T operand: query qn's 16-byte pieces; queries past G are zero
  bf16x8 qb[M::KC];
  {
    const char* qrow = reinterpret_cast<const char*>(Q + ((int64_t)h * G + min(qn, G - 1)) * D) + qt * 16;
#pragma unroll
    for (int c = 0; c < M::KC; ++c) {
      V4 x = *reinterpret_cast<const V4*>(qrow + 64 * c);
      if (qn >= G) x = V4{0, 0, 0, 0};
      qb[c] = __builtin_bit_cast(bf16x8, x);
    }
  }
  float m = -INFINITY, l = 0.0f;
  float4v acc[M::VC];
#pragma unroll
  for (int c = 0; c < M::VC; ++c) acc[c] = float4v{0.0f, 0.0f, 0.0f, 0.0f};

  const int npw = nu > wv ? (nu - wv + kMW - 1) / kMW : 0;
  for (int k0 = 0; k0 < npw; k0 += 64) {
    int my_pg = -1, my_cnt = 0;
    if (k0 + lane < npw) {
      my_pg = u[wv + kMW * (k0 + lane)];
      if (my_pg < 0 || my_pg >= n_pages) my_pg = -1;
      else my_cnt = pg_cnt[my_pg];
    }
    const int nk = min(64, npw - k0);
    MPage<D> bufA, bufB;
    {
      const int p0 = __shfl(my_pg, 0, 64);
      mload<D>(pgK, pgV, p0 >= 0 ? p0 : 0, __shfl(my_cnt, 0, 64), lane, bufA);
    }
    // page k from `cur` while page k+1 loads into `nxt` (unconditionally, so
    // the wait counts stay exact; past the last page it re-reads page 0)
    auto step = [&](int k, MPage<D>& cur, MPage<D>& nxt) {
      const int pg = __shfl(my_pg, k, 64);
      const int cnt = __shfl(my_cnt, k, 64);
      const int pgn = k + 1 < nk ? __shfl(my_pg, k + 1, 64) : -1;
      const int cntn = k + 1 < nk ? __shfl(my_cnt, k + 1, 64) : 0;
      mload<D>(pgK, pgV, pgn >= 0 ? pgn : 0, cntn, lane, nxt);
      if (pg < 0) return;
      float4v s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < M::KC; ++c) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8, cur.k[c]), qb[c], s, 0, 0, 0);
      float x[4];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[j] = 4 * qt + j < cnt ? s[j] * c2 : -INFINITY;
        mx = fmaxf(mx, x[j]);
      }
      mx = fmaxf(mx, xor_lane_f<16>(mx));
      mx = fmaxf(mx, xor_lane_f<32>(mx));
      const float mn = fmaxf(m, mx);           // finite: every page has a valid token
      const float corr = exp2f(m - mn);
      float p[4], rs = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[j] = exp2f(x[j] - mn);
        rs += p[j];
      }
      rs += xor_lane_f<16>(rs);
      rs += xor_lane_f<32>(rs);
      l = l * corr + rs;
      m = mn;
      // P = hi + lo in bf16, as the A operand (query qn, tokens 4qt .. 4qt+3)
      short4v phi, plo;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t hi = bf16_rne(p[j]);
        phi[j] = (short)hi;
        plo[j] = (short)bf16_rne(p[j] - __uint_as_float(hi << 16));
      }
      // the rescale factor of query 4qt + j for the accumulator rows
      if (qt == 0) corr_lds[wv][qn] = corr;
      wave_sync();
      const float4v cq = *reinterpret_cast<const float4v*>(&corr_lds[wv][4 * qt]);
      wave_sync();
#pragma unroll
      for (int c = 0; c < M::VC; ++c) {
        acc[c] *= cq;
        const short4v vb = __builtin_bit_cast(short4v, cur.v[c]);
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, vb, acc[c], 0, 0, 0);
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, vb, acc[c], 0, 0, 0);
      }
    };
    for (int k = 0; k < nk; k += 2) {
      step(k, bufA, bufB);
      if (k + 1 < nk) step(k + 1, bufB, bufA);
    }
  }
  // wave partials: m and l of query qn (every lane group holds them), the
  // accumulator rows 4qt + j
  if (qt == 0 && qn < G) {
    part_m[wv][qn] = m;
    part_l[wv][qn] = l;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = 4 * qt + j;
    if (q < G)
#pragma unroll
      for (int c = 0; c < M::VC; ++c) part_o[wv][q][16 * c + qn] = acc[c][j];
  }
  __syncthreads();
  for (int t = threadIdx.x; t < G * D; t += blockDim.x) {
    const int q = t / D, dd = t % D;
    float Mx = -INFINITY;
    for (int w = 0; w < kMW; ++w) Mx = fmaxf(Mx, part_m[w][q]);
    float Ls = 0.0f, a = 0.0f;
    if (Mx > -INFINITY) {
      for (int w = 0; w < kMW; ++w) {
        if (part_m[w][q] == -INFINITY) continue;
        const float wt = exp2f(part_m[w][q] - Mx);
        Ls = fmaf(part_l[w][q], wt, Ls);
        a = fmaf(part_o[w][q][dd], wt, a);
      }
    }
    O[((int64_t)h * G + q) * D + dd] = Ls > 0.0f ? a / Ls : 0.0f;
    if (lse && dd == 0) lse[(int64_t)h * G + q] = Ls > 0.0f ? (Mx + log2f(Ls)) * kLn2 : -INFINITY;
  }
}

// ============================================================================
// fp32: vector ALUs
// ============================================================================
// 8 waves; wave w takes union pages w, w+8, ...; up to 4 query heads per pass
// over the pages. K is read with 4 lanes per row (lane part p holds the row's
// 16-byte pieces p, p+4, ...); V with each lane owning 2 dimensions of every
// slot (of half the slots when d = 64), so o needs no replication across
// lanes and the weights reach the lanes as LDS broadcasts.

constexpr int kAttWaves = 8;
constexpr int kQPerPass = 4;

template <int D>
struct FGeo {
  static constexpr int ROWB = D * 4;
  static constexpr int NLK = ROWB / 64;        // 16-byte K pieces per lane
  static constexpr int VL = D / 2;             // lanes per V slot: 2 dims each
  static constexpr int RS = 64 / VL;           // slot halves (1 for d = 128, 2 for d = 64)
  static constexpr int NG = 4 / RS;            // slot groups per lane
};

template <int D>
struct FPage {
  V4 k[FGeo<D>::NLK];
  V4 v[FGeo<D>::NG][2];                        // per slot group: dim 2dp (4 slots), dim 2dp+1 (4 slots)
};

template <int D>
__device__ inline void fload_k(const char* pgK, int pg, int cnt, int lane, FPage<D>& r) {
  using A = FGeo<D>;
  const uint32_t page = (uint32_t)pg * (ICE_PAGE_CAP * A::ROWB);
  const int last = cnt > 0 ? cnt - 1 : 0;
  const uint32_t koff = page + (uint32_t)min(lane >> 2, last) * A::ROWB + (lane & 3) * 16;
#pragma unroll
  for (int i = 0; i < A::NLK; ++i) r.k[i] = *reinterpret_cast<const V4*>(pgK + (koff + 64 * i));
}
template <int D>
__device__ inline void fload_v(const char* pgV, int pg, int cnt, int lane, FPage<D>& r) {
  using A = FGeo<D>;
  const uint32_t page = (uint32_t)pg * (ICE_PAGE_CAP * A::ROWB);
  const int lastg = cnt > 0 ? (cnt - 1) >> 2 : 0;
  const int dp = lane % A::VL, rg = lane / A::VL;
#pragma unroll
  for (int gi = 0; gi < A::NG; ++gi) {
    const int g = min(rg * A::NG + gi, lastg);
    const uint32_t voff = page + (uint32_t)(g * D + 2 * dp) * 16;
    r.v[gi][0] = *reinterpret_cast<const V4*>(pgV + voff);
    r.v[gi][1] = *reinterpret_cast<const V4*>(pgV + voff + 16);
  }
}

// q.k over this lane's pieces (q[4 * i]: the query's piece i for this lane's
// part), summed over the row's 4 lanes
template <int D>
__device__ inline float qk_dot_f32(const V4* q, const V4* k) {
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < FGeo<D>::NLK; ++i) {
    const V4 qi = q[4 * i];
    s = fmaf(__uint_as_float(k[i].x), __uint_as_float(qi.x), s);
    s = fmaf(__uint_as_float(k[i].y), __uint_as_float(qi.y), s);
    s = fmaf(__uint_as_float(k[i].z), __uint_as_float(qi.z), s);
    s = fmaf(__uint_as_float(k[i].w), __uint_as_float(qi.w), s);
  }
  s += xor_lane_f<1>(s);
  s += xor_lane_f<2>(s);
  return s;
}

// sum / max over the 16 rows of a page (lanes 4r + part)
__device__ inline float rows_sum(float s) {
  s += xor_lane_f<4>(s);
  s += xor_lane_f<8>(s);
  s += xor_lane_f<16>(s);
  s += xor_lane_f<32>(s);
  return s;
}
__device__ inline float rows_max(float s) {
  s = fmaxf(s, xor_lane_f<4>(s));
  s = fmaxf(s, xor_lane_f<8>(s));
  s = fmaxf(s, xor_lane_f<16>(s));
  s = fmaxf(s, xor_lane_f<32>(s));
  return s;
}

template <int D>
__global__ __launch_bounds__(kAttWaves * 64) void k_attend_f32(DevLayout L, const void* blob, const float* Q,
                                                               const int32_t* uni, const int32_t* n_uni,
                                                               int uni_stride, float scale, float* O, float* lse) {
  using A = FGeo<D>;
  __shared__ float part_m[kAttWaves][kQPerPass], part_l[kAttWaves][kQPerPass];
  __shared__ float part_o[kAttWaves][kQPerPass][D];
  __shared__ V4 q_lds[kQPerPass][A::NLK][4];              // [query][piece i][lane part]
  __shared__ __attribute__((aligned(16))) float p_lds[kAttWaves][kQPerPass][16];   // page weights per wave
  const int h = blockIdx.x;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int G = L.G;
  const void* hb = head_base(blob, L, h);
  const char* pgK = at<char>(hb, L.off_pgK[0]);
  const char* pgV = at<char>(hb, L.off_pgV);
  const int32_t* pg_cnt = at<int32_t>(hb, L.off_pg_cnt[0]);
  const int n_pages = at<Hdr>(hb, L.off_hdr)->n_pages[0];
  const int nu = min(n_uni[h], uni_stride);
  const int32_t* u = uni + (int64_t)h * uni_stride;
  const float c2 = scale * kLog2e;
  const int krow = lane >> 2;
  const int rg = lane / A::VL;
  const int npw = nu > wv ? (nu - wv + kAttWaves - 1) / kAttWaves : 0;

  for (int g0 = 0; g0 < G; g0 += kQPerPass) {
    const int ng = min(kQPerPass, G - g0);
    if (threadIdx.x < kQPerPass * A::NLK * 4) {
      const int g = threadIdx.x / (A::NLK * 4), i = (threadIdx.x >> 2) % A::NLK, part = threadIdx.x & 3;
      const char* qrow = reinterpret_cast<const char*>(Q + ((int64_t)h * G + g0 + (g < ng ? g : 0)) * D);
      q_lds[g][i][part] = *reinterpret_cast<const V4*>(qrow + part * 16 + 64 * i);
    }
    __syncthreads();
    float m[kQPerPass], l[kQPerPass], o[kQPerPass][2];
#pragma unroll
    for (int g = 0; g < kQPerPass; ++g) {
      m[g] = -INFINITY;
      l[g] = 0.0f;
      o[g][0] = o[g][1] = 0.0f;
    }
    for (int k0 = 0; k0 < npw; k0 += 64) {
      int my_pg = -1, my_cnt = 0;
      if (k0 + lane < npw) {
        my_pg = u[wv + kAttWaves * (k0 + lane)];
        if (my_pg < 0 || my_pg >= n_pages) my_pg = -1;
        else my_cnt = pg_cnt[my_pg];
      }
      const int nk = min(64, npw - k0);
      FPage<D> bufA, bufB;
      {
        const int p0 = __shfl(my_pg, 0, 64), c0 = __shfl(my_cnt, 0, 64);
        fload_k<D>(pgK, p0 >= 0 ? p0 : 0, c0, lane, bufA);
        fload_v<D>(pgV, p0 >= 0 ? p0 : 0, c0, lane, bufA);
      }
      // page k from `cur`; page k+1's K loads before the scores, its V after
      auto step = [&](int k, FPage<D>& cur, FPage<D>& nxt) {
        const int pg = __shfl(my_pg, k, 64);
        const int cnt = __shfl(my_cnt, k, 64);
        const int pgn = k + 1 < nk ? __shfl(my_pg, k + 1, 64) : -1;
        const int cntn = k + 1 < nk ? __shfl(my_cnt, k + 1, 64) : 0;
        fload_k<D>(pgK, pgn >= 0 ? pgn : 0, cntn, lane, nxt);
        float corr[kQPerPass];
        if (pg >= 0) {
          const bool valid = krow < cnt;
#pragma unroll
          for (int g = 0; g < kQPerPass; ++g) {
            const float s = valid ? qk_dot_f32<D>(&q_lds[g][0][lane & 3], cur.k) * c2 : -INFINITY;
            const float mn = fmaxf(m[g], rows_max(s));
            corr[g] = exp2f(m[g] - mn);
            const float p = valid ? exp2f(s - mn) : 0.0f;
            l[g] = l[g] * corr[g] + rows_sum(p);
            m[g] = mn;
            if ((lane & 3) == 0) p_lds[wv][g][krow] = p;
          }
        }
        wave_sync();
        fload_v<D>(pgV, pgn >= 0 ? pgn : 0, cntn, lane, nxt);
        if (pg >= 0) {
#pragma unroll
          for (int g = 0; g < kQPerPass; ++g) {
            o[g][0] *= corr[g];
            o[g][1] *= corr[g];
          }
#pragma unroll
          for (int gi = 0; gi < A::NG; ++gi) {
            const float* va = reinterpret_cast<const float*>(&cur.v[gi][0]);
            const float* vb = reinterpret_cast<const float*>(&cur.v[gi][1]);
#pragma unroll
            for (int g = 0; g < kQPerPass; ++g) {
              const float4 pw = *reinterpret_cast<const float4*>(&p_lds[wv][g][4 * (rg * A::NG + gi)]);
              o[g][0] = fmaf(pw.x, va[0], o[g][0]);
              o[g][0] = fmaf(pw.y, va[1], o[g][0]);
              o[g][0] = fmaf(pw.z, va[2], o[g][0]);
              o[g][0] = fmaf(pw.w, va[3], o[g][0]);
              o[g][1] = fmaf(pw.x, vb[0], o[g][1]);
              o[g][1] = fmaf(pw.y, vb[1], o[g][1]);
              o[g][1] = fmaf(pw.z, vb[2], o[g][1]);
              o[g][1] = fmaf(pw.w, vb[3], o[g][1]);
            }
          }
        }
        wave_sync();
      };
      for (int k = 0; k < nk; k += 2) {
        step(k, bufA, bufB);
        if (k + 1 < nk) step(k + 1, bufB, bufA);
      }
    }
    // d = 64: the two slot halves hold partial outputs of the same dims
    const int dp = lane % A::VL;
#pragma unroll
    for (int g = 0; g < kQPerPass; ++g) {
      if constexpr (A::RS == 2) {
        o[g][0] += xor_lane_f<32>(o[g][0]);
        o[g][1] += xor_lane_f<32>(o[g][1]);
      }
      if (lane == 0) {
        part_m[wv][g] = m[g];
        part_l[wv][g] = l[g];
      }
      if (rg == 0) {
        part_o[wv][g][2 * dp] = o[g][0];
        part_o[wv][g][2 * dp + 1] = o[g][1];
      }
    }
    __syncthreads();
    for (int t = threadIdx.x; t < ng * D; t += blockDim.x) {
      const int g = t / D, dd = t % D;
      float M = -INFINITY;
      for (int w = 0; w < kAttWaves; ++w) M = fmaxf(M, part_m[w][g]);
      float Ls = 0.0f, acc = 0.0f;
      if (M > -INFINITY) {
        for (int w = 0; w < kAttWaves; ++w) {
          if (part_m[w][g] == -INFINITY) continue;
          const float wt = exp2f(part_m[w][g] - M);
          Ls = fmaf(part_l[w][g], wt, Ls);
          acc = fmaf(part_o[w][g][dd], wt, acc);
        }
      }
      O[((int64_t)h * G + g0 + g) * D + dd] = Ls > 0.0f ? acc / Ls : 0.0f;
      if (lse && dd == 0) lse[(int64_t)h * G + g0 + g] = Ls > 0.0f ? (M + log2f(Ls)) * kLn2 : -INFINITY;
    }
    __syncthreads();
  }
}

}  // namespace

int attend_splits(int) { return 0; }

hipError_t launch_attend(const DevLayout& L, const void* blob, const void* Q, const int32_t* uni,
                         const int32_t* n_uni, int uni_stride, float scale, float* O, float* lse, void*,
                         hipStream_t s) {
  const dim3 grid((unsigned)L.H);
  if (L.dtype == ICE_BF16) {
    const uint16_t* q = static_cast<const uint16_t*>(Q);
    if (L.d == 128) k_attend_mfma<128><<<grid, kMW * 64, 0, s>>>(L, blob, q, uni, n_uni, uni_stride, scale, O, lse);
    else k_attend_mfma<64><<<grid, kMW * 64, 0, s>>>(L, blob, q, uni, n_uni, uni_stride, scale, O, lse);
  } else {
    const float* q = static_cast<const float*>(Q);
    if (L.d == 128) k_attend_f32<128><<<grid, kAttWaves * 64, 0, s>>>(L, blob, q, uni, n_uni, uni_stride, scale, O, lse);
    else k_attend_f32<64><<<grid, kAttWaves * 64, 0, s>>>(L, blob, q, uni, n_uni, uni_stride, scale, O, lse);
  }
  return hipGetLastError();
}

}  // namespace ice
