// Sparse attention over the selected pages: the ice_attend kernels.
//
// The papernotes.org IceCache notes (key design 1) give the weight of token j
// for query i as s_ij exp(q_i.k_j/sqrt d) / sum_j' s_ij' exp(q_i.k_j'/sqrt d),
// with s the selection mask: a softmax over the tokens of the selected pages
// only. Every query head of a GQA group attends the group's page union (key
// design 3). Per page that is S = K Q^T (16 tokens x G queries over d) and
// O += P V, with an online softmax (running max m and sum l per query) in
// between. bf16 runs both products on the matrix cores (attend_mfma.h, one
// block of 8 waves per head); fp32 runs them on the vector ALUs (below).
#include "ice_launch.h"
#include "attend_mfma.h"

#include <algorithm>

namespace ice {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ============================================================================
// bf16: matrix cores (attend_mfma.h)
// ============================================================================
constexpr int kMW = 8;                // waves per block

template <int D>
__global__ __launch_bounds__(kMW * 64) void k_attend_mfma(DevLayout L, const void* blob, const uint16_t* Q,
                                                          const int32_t* uni, const int32_t* n_uni, int uni_stride,
                                                          float scale, float* O, float* lse) {
  extern __shared__ float part[];
  const int h = blockIdx.x, G = L.G;
  mfma_attend::attend_head<D, true>(L, head_base(blob, L, h), Q + (int64_t)h * G * D, G, uni + (int64_t)h * uni_stride,
                              min(n_uni[h], uni_stride), scale, O + (int64_t)h * G * D, lse ? lse + (int64_t)h * G : nullptr,
                              part, kMW);
}

// ============================================================================
// fp32: vector ALUs
// ============================================================================
// One block of 8 waves per head; wave w takes union pages w, w+8, ... and
// keeps the next page's loads in flight while it uses the current one; the
// waves' (m, l, o) partials are merged in LDS. Up to 4 query heads per pass
// over the pages. K is read with 4 lanes per row (lane part p holds the row's
// 16-byte pieces p, p+4, ...); V with each lane owning 2 dimensions of every
// slot (of half the slots when d = 64), so o needs no replication across
// lanes and the weights reach the lanes as LDS broadcasts. Page pools: K
// pages are [page][slot][d]; V pages are [page][slot group g = slot/4][d][4
// slots]. Loads are unconditional: rows and slot groups past a page's count
// re-read its last valid ones (no extra memory traffic) and get weight 0.

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
  // with staged V the page of union entry u is entry u of the head's staging area
  const bool staged = L.vstage != nullptr;
  const char* pgV = staged ? L.vstage + (int64_t)h * L.vstage_pages * (ICE_PAGE_CAP * D * 4) : v_pages(L, hb, h);
  const int32_t* pg_cnt = at<int32_t>(hb, L.off_pg_cnt[0]);
  // the union (or every page of a dense head), then the resident pages
  const PageSrc src = page_src(L, hb, uni + (int64_t)h * uni_stride, min(n_uni[h], uni_stride));
  const int nu = src.count();
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
        my_pg = src.at(wv + kAttWaves * (k0 + lane));
        if (my_pg >= 0) my_cnt = pg_cnt[my_pg];
      }
      const int nk = min(64, npw - k0);
      FPage<D> bufA, bufB;
      {
        const int p0 = __shfl(my_pg, 0, 64), c0 = __shfl(my_cnt, 0, 64);
        fload_k<D>(pgK, p0 >= 0 ? p0 : 0, c0, lane, bufA);
        fload_v<D>(pgV, p0 >= 0 ? (staged ? wv + kAttWaves * k0 : p0) : 0, c0, lane, bufA);
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
        fload_v<D>(pgV, pgn >= 0 ? (staged ? wv + kAttWaves * (k0 + k + 1) : pgn) : 0, cntn, lane, nxt);
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

// Host-pool mode, the bulk load of a step: copies the level-0 V pages of head
// h's union from the pinned host pool into entries 0..n_uni-1 of the head's
// staging area, in union order (16-byte pieces, kGatherUnroll loads in flight
// per thread, the link's latency hidden by the blocks of all heads). An id
// outside the head's page table stages a zero page.
constexpr int kGatherUnroll = 4;

__global__ __launch_bounds__(256) void k_gather_v(DevLayout L, const void* blob, const int32_t* uni,
                                                   const int32_t* n_uni, int uni_stride) {
  const int h = blockIdx.x;
  const void* hb = head_base(blob, L, h);
  const int64_t pb = (int64_t)ICE_PAGE_CAP * L.d * L.elt;
  const char* src = v_pages(L, hb, h);
  char* dst = const_cast<char*>(L.vstage) + (int64_t)h * L.vstage_pages * pb;
  const int n_pages = at<Hdr>(hb, L.off_hdr)->n_pages[0];
  const int nu = min(n_uni[h], uni_stride);
  const int32_t* u = uni + (int64_t)h * uni_stride;
  const int per = (int)(pb / 16);
  const int total = nu * per;
  const int step = gridDim.y * blockDim.x * kGatherUnroll;
  for (int i0 = blockIdx.y * blockDim.x * kGatherUnroll + threadIdx.x; i0 < total; i0 += step) {
    V4 v[kGatherUnroll];
#pragma unroll
    for (int j = 0; j < kGatherUnroll; ++j) {
      const int i = i0 + j * blockDim.x;
      v[j] = V4{0, 0, 0, 0};
      if (i < total) {
        const int pg = u[i / per];
        if (pg >= 0 && pg < n_pages) v[j] = *reinterpret_cast<const V4*>(src + (int64_t)pg * pb + (int64_t)(i % per) * 16);
      }
    }
#pragma unroll
    for (int j = 0; j < kGatherUnroll; ++j) {
      const int i = i0 + j * blockDim.x;
      if (i < total) *reinterpret_cast<V4*>(dst + (int64_t)i * 16) = v[j];
    }
  }
}

}  // namespace

hipError_t launch_gather_v(const DevLayout& L, const void* blob, const int32_t* uni, const int32_t* n_uni,
                           int uni_stride, hipStream_t s) {
  if (!L.vpool || !L.vstage) return hipErrorInvalidValue;
  // blocks per head: enough to cover the largest union in one pass
  const int64_t pieces = (int64_t)uni_stride * ICE_PAGE_CAP * L.d * L.elt / 16;
  const unsigned per_head = (unsigned)std::max<int64_t>(1, (pieces + 256 * kGatherUnroll - 1) / (256 * kGatherUnroll));
  k_gather_v<<<dim3((unsigned)L.H, per_head), 256, 0, s>>>(L, blob, uni, n_uni, uni_stride);
  return hipGetLastError();
}

hipError_t launch_attend(const DevLayout& L, const void* blob, const void* Q, const int32_t* uni,
                         const int32_t* n_uni, int uni_stride, float scale, float* O, float* lse, void*,
                         hipStream_t s) {
  const dim3 grid((unsigned)L.H);
  if (L.dtype == ICE_BF16) {
    const uint16_t* q = static_cast<const uint16_t*>(Q);
    const size_t part = (size_t)mfma_attend::part_floats(kMW, L.G, L.d) * sizeof(float);
    if (L.d == 128) k_attend_mfma<128><<<grid, kMW * 64, part, s>>>(L, blob, q, uni, n_uni, uni_stride, scale, O, lse);
    else k_attend_mfma<64><<<grid, kMW * 64, part, s>>>(L, blob, q, uni, n_uni, uni_stride, scale, O, lse);
  } else {
    const float* q = static_cast<const float*>(Q);
    if (L.d == 128) k_attend_f32<128><<<grid, kAttWaves * 64, 0, s>>>(L, blob, q, uni, n_uni, uni_stride, scale, O, lse);
    else k_attend_f32<64><<<grid, kAttWaves * 64, 0, s>>>(L, blob, q, uni, n_uni, uni_stride, scale, O, lse);
  }
  return hipGetLastError();
}

namespace {

// Resident pages: the caller's n tokens of each head (row-major K and V)
// into pages pcap[0] .. pcap[0] + res_pages - 1 of the page pool, K as
// [slot][d] and V as [slot group][d][4 slots] like every KV page, zeros past
// n; then the pages' row counts and the header's resident count. One wave
// per resident page.
template <int D, class T>
__global__ __launch_bounds__(64) void k_set_resident(DevLayout L, void* blob, const T* K, const T* V, int n,
                                                     int64_t hstride) {
  const int p = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  void* hb = head_base(blob, L, h);
  const int pg = L.pcap[0] + p;
  T* pk = at<T>(hb, L.off_pgK[0]) + (int64_t)pg * ICE_PAGE_CAP * D;
  T* pv = reinterpret_cast<T*>(v_pages(L, hb, h)) + (int64_t)pg * ICE_PAGE_CAP * D;
  const T* Kh = K + (int64_t)h * hstride;
  const T* Vh = V + (int64_t)h * hstride;
  for (int i = lane; i < ICE_PAGE_CAP * D; i += 64) {
    const int sl = i / D, c = i % D, t = ICE_PAGE_CAP * p + sl;
    const bool in = t < n;
    pk[i] = in ? Kh[(int64_t)t * D + c] : T(0);
    pv[((sl / 4) * D + c) * 4 + sl % 4] = in ? Vh[(int64_t)t * D + c] : T(0);
  }
  if (lane == 0) {
    at<int32_t>(hb, L.off_pg_cnt[0])[pg] = max(0, min(ICE_PAGE_CAP, n - ICE_PAGE_CAP * p));
    if (p == 0) at<Hdr>(hb, L.off_hdr)->n_resident = n;
  }
}

}  // namespace

hipError_t launch_set_resident(const DevLayout& L, void* blob, const void* K, const void* V, int n, int64_t hstride,
                               hipStream_t s) {
  const dim3 grid((unsigned)L.res_pages, (unsigned)L.H);
  if (L.dtype == ICE_BF16) {
    const uint16_t* k = static_cast<const uint16_t*>(K);
    const uint16_t* v = static_cast<const uint16_t*>(V);
    if (L.d == 128) k_set_resident<128, uint16_t><<<grid, 64, 0, s>>>(L, blob, k, v, n, hstride);
    else k_set_resident<64, uint16_t><<<grid, 64, 0, s>>>(L, blob, k, v, n, hstride);
  } else {
    const float* k = static_cast<const float*>(K);
    const float* v = static_cast<const float*>(V);
    if (L.d == 128) k_set_resident<128, float><<<grid, 64, 0, s>>>(L, blob, k, v, n, hstride);
    else k_set_resident<64, float><<<grid, 64, 0, s>>>(L, blob, k, v, n, hstride);
  }
  return hipGetLastError();
}

}  // namespace ice
