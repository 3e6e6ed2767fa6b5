// Sparse attention over the selected pages.
//
// The papernotes.org IceCache notes (key design 1) give the weight of token j
// for query i as s_ij exp(q_i.k_j/sqrt d) / sum_j' s_ij' exp(q_i.k_j'/sqrt d),
// with s the selection mask: a softmax over the tokens of the selected pages
// only. Every query head of a GQA group attends the group's page union (key
// design 3).
//
// One block of 8 waves per head; wave w takes union pages w, w+8, ... and
// keeps an online softmax (running max m, sum l, output o) for up to 4 query
// heads at a time. Per page (16 rows) the wave reads K with 4 lanes per row
// (16-byte pieces p, p+4, ... for lane part p; bf16 dot2 for q.k) and V with 16 lanes per row (each
// lane 4 rows x D/16 dims), so both are plain coalesced 16-byte loads; the
// next page's loads are issued before the current page is used. Logits are
// kept in base 2 (scaled by scale * log2 e). The 8 wave partials of a head
// are merged in LDS. Loads are unconditional (so the next page's loads stay
// in flight): the lanes of rows past a page's count re-read its last valid
// row, which costs no extra memory traffic, and those rows are masked.
#include "ice_launch.h"

namespace ice {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kAttWaves = 8;
constexpr int kQPerPass = 4;        // query heads per pass over the pages
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D, class T>
struct AttGeo {
  static constexpr int ROWB = D * (int)sizeof(T);
  static constexpr int NLK = ROWB / 64;        // 16-byte K loads per lane (quarter row)
  static constexpr int VB = ROWB / 16;         // V bytes per lane per row (16 lanes per row)
  static constexpr int DV = D / 16;            // output dims per lane
  static constexpr int EPK = 16 / (int)sizeof(T);
};

// V bytes -> floats
template <class T, int DV>
__device__ inline void unpack_v(const char* src, float* out) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(src);
#pragma unroll
    for (int i = 0; i < DV / 2; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    const float* f = reinterpret_cast<const float*>(src);
#pragma unroll
    for (int i = 0; i < DV; ++i) out[i] = f[i];
  }
}

template <int D, class T>
struct PageRegs {
  using A = AttGeo<D, T>;
  V4 k[A::NLK];
  uint32_t v[4][A::VB / 4];
  int cnt;
};

template <int D, class T>
__device__ inline void load_page(const T* pgK, const T* pgV, int pg, int cnt, int lane, PageRegs<D, T>& r) {
  using A = AttGeo<D, T>;
  const int64_t base = (int64_t)pg * ICE_PAGE_CAP;
  // rows past the page's count are masked later; they read the last valid row
  // (already in cache) instead of the empty slots
  const int last = cnt > 0 ? cnt - 1 : 0;
  // lane part p holds the 16-byte pieces p, p + 4, ...: the 4 lanes of a row
  // read one contiguous 64-byte segment per load
  const char* krow = reinterpret_cast<const char*>(pgK + (base + min(lane >> 2, last)) * D) + (lane & 3) * 16;
#pragma unroll
  for (int i = 0; i < A::NLK; ++i) r.k[i] = *reinterpret_cast<const V4*>(krow + 64 * i);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const char* vrow = reinterpret_cast<const char*>(pgV + (base + min((lane >> 4) + 4 * i, last)) * D) + (lane & 15) * A::VB;
    if constexpr (A::VB >= 16) {
#pragma unroll
      for (int c = 0; c < A::VB / 16; ++c) {
        const V4 x = *reinterpret_cast<const V4*>(vrow + 16 * c);
        r.v[i][4 * c] = x.x;
        r.v[i][4 * c + 1] = x.y;
        r.v[i][4 * c + 2] = x.z;
        r.v[i][4 * c + 3] = x.w;
      }
    } else {
      const uint2 x = *reinterpret_cast<const uint2*>(vrow);
      r.v[i][0] = x.x;
      r.v[i][1] = x.y;
    }
  }
}

template <int D, class T>
__device__ inline float qk_dot(const V4* q, const V4* k) {
  using A = AttGeo<D, T>;
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < A::NLK; ++i) {
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

template <int D, class T>
__global__ __launch_bounds__(kAttWaves * 64) void k_attend(DevLayout L, const void* blob, const T* Q,
                                                           const int32_t* uni, const int32_t* n_uni,
                                                           int uni_stride, float scale, float* O, float* lse) {
  using A = AttGeo<D, T>;
  __shared__ float part_m[kAttWaves][kQPerPass], part_l[kAttWaves][kQPerPass];
  __shared__ float part_o[kAttWaves][kQPerPass][D];
  const int h = blockIdx.x;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int G = L.G;
  const void* hb = head_base(blob, L, h);
  const T* pgK = at<T>(hb, L.off_pgK[0]);
  const T* pgV = at<T>(hb, L.off_pgV);
  const int32_t* pg_cnt = at<int32_t>(hb, L.off_pg_cnt[0]);
  const int n_pages = at<Hdr>(hb, L.off_hdr)->n_pages[0];
  const int nu = min(n_uni[h], uni_stride);
  const int32_t* u = uni + (int64_t)h * uni_stride;
  const float c2 = scale * kLog2e;
  const int krow = lane >> 2;

  for (int g0 = 0; g0 < G; g0 += kQPerPass) {
    const int ng = min(kQPerPass, G - g0);
    V4 q[kQPerPass][A::NLK];
#pragma unroll
    for (int g = 0; g < kQPerPass; ++g) {
      const char* qrow = reinterpret_cast<const char*>(Q + ((int64_t)h * G + g0 + (g < ng ? g : 0)) * D) +
                         (lane & 3) * 16;
#pragma unroll
      for (int i = 0; i < A::NLK; ++i) q[g][i] = *reinterpret_cast<const V4*>(qrow + 64 * i);
    }
    float m[kQPerPass], l[kQPerPass], o[kQPerPass][A::DV];
#pragma unroll
    for (int g = 0; g < kQPerPass; ++g) {
      m[g] = -INFINITY;
      l[g] = 0.0f;
#pragma unroll
      for (int c = 0; c < A::DV; ++c) o[g][c] = 0.0f;
    }
    // pages wv, wv+8, ...: their ids and valid counts are fetched up front, one
    // per lane (ids outside the page table are skipped)
    const int npw = nu > wv ? (nu - wv + kAttWaves - 1) / kAttWaves : 0;
    for (int k0 = 0; k0 < npw; k0 += 64) {
      int my_pg = -1, my_cnt = 0;
      if (k0 + lane < npw) {
        my_pg = u[wv + kAttWaves * (k0 + lane)];
        if (my_pg < 0 || my_pg >= n_pages) my_pg = -1;
        else my_cnt = pg_cnt[my_pg];
      }
      const int nk = min(64, npw - k0);
      // loads are unconditional (a skipped id reads page 0 and is masked) so
      // the next page's loads stay in flight while the current one is used
      int pg = __shfl(my_pg, 0, 64);
      PageRegs<D, T> cur, nxt;
      load_page<D, T>(pgK, pgV, pg >= 0 ? pg : 0, __shfl(my_cnt, 0, 64), lane, cur);
      for (int k = 0; k < nk; ++k) {
        const int pgn = k + 1 < nk ? __shfl(my_pg, k + 1, 64) : -1;
        load_page<D, T>(pgK, pgV, pgn >= 0 ? pgn : 0, k + 1 < nk ? __shfl(my_cnt, k + 1, 64) : 0, lane, nxt);
        const int cnt = __shfl(my_cnt, k, 64);
        if (pg >= 0) {
          const bool valid = krow < cnt;
          float p[kQPerPass];
#pragma unroll
          for (int g = 0; g < kQPerPass; ++g) {
            const float s = valid ? qk_dot<D, T>(q[g], cur.k) * c2 : -INFINITY;
            const float mn = fmaxf(m[g], rows_max(s));
            const float corr = exp2f(m[g] - mn);
            p[g] = valid ? exp2f(s - mn) : 0.0f;
            l[g] = l[g] * corr + rows_sum(p[g]);
            m[g] = mn;
#pragma unroll
            for (int c = 0; c < A::DV; ++c) o[g][c] *= corr;
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float v[A::DV];
            unpack_v<T, A::DV>(reinterpret_cast<const char*>(cur.v[r]), v);
            const int src = 4 * ((lane >> 4) + 4 * r);   // a lane holding row (lane/16 + 4r)'s weight
#pragma unroll
            for (int g = 0; g < kQPerPass; ++g) {
              const float pr = __shfl(p[g], src, 64);
#pragma unroll
              for (int c = 0; c < A::DV; ++c) o[g][c] = fmaf(pr, v[c], o[g][c]);
            }
          }
        }
        cur = nxt;
        pg = pgn;
      }
    }
    // the four row groups of the wave hold partial outputs of the same dims
#pragma unroll
    for (int g = 0; g < kQPerPass; ++g) {
#pragma unroll
      for (int c = 0; c < A::DV; ++c) {
        o[g][c] += xor_lane_f<16>(o[g][c]);
        o[g][c] += xor_lane_f<32>(o[g][c]);
      }
      if (lane == 0) {
        part_m[wv][g] = m[g];
        part_l[wv][g] = l[g];
      }
      if (lane < 16)
#pragma unroll
        for (int c = 0; c < A::DV; ++c) part_o[wv][g][lane * A::DV + c] = o[g][c];
    }
    __syncthreads();
    // merge the wave partials: thread -> (query, dim)
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
  const dim3 grid((unsigned)L.H), block(kAttWaves * 64);
  if (L.dtype == ICE_BF16) {
    const uint16_t* q = static_cast<const uint16_t*>(Q);
    if (L.d == 128) k_attend<128, uint16_t><<<grid, block, 0, s>>>(L, blob, q, uni, n_uni, uni_stride, scale, O, lse);
    else k_attend<64, uint16_t><<<grid, block, 0, s>>>(L, blob, q, uni, n_uni, uni_stride, scale, O, lse);
  } else {
    const float* q = static_cast<const float*>(Q);
    if (L.d == 128) k_attend<128, float><<<grid, block, 0, s>>>(L, blob, q, uni, n_uni, uni_stride, scale, O, lse);
    else k_attend<64, float><<<grid, block, 0, s>>>(L, blob, q, uni, n_uni, uni_stride, scale, O, lse);
  }
  return hipGetLastError();
}

}  // namespace ice
