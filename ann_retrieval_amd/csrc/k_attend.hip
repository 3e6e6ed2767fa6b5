// Sparse attention over the selected pages.
//
// The papernotes.org IceCache notes (key design 1) give the weight of token j
// for query i as s_ij exp(q_i.k_j/sqrt d) / sum_j' s_ij' exp(q_i.k_j'/sqrt d),
// with s the selection mask: a softmax over the tokens of the selected pages
// only. Every query head of a GQA group attends the group's page union (key
// design 3).
//
// k_attend_part: one block per (split of the union, head). The block stages
// 4 pages (64 rows of K and V) at a time in LDS with 16-byte coalesced loads
// and keeps an online softmax per query head (one wave per query head). Logits
// are kept in base-2 units (q pre-scaled by scale * log2 e) so the exponent is
// one exp2. k_attend_combine merges the per-split (m, l, o) partials.
#include "ice_launch.h"

namespace ice {
namespace {

constexpr int kPagesPerSplit = 8;
constexpr int kBatchPages = 4;
constexpr int kRows = kBatchPages * ICE_PAGE_CAP;   // 64 rows per LDS batch
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMaxQPerWave = ICE_MAX_GROUP / 4;

template <int D, class T>
__global__ __launch_bounds__(256) void k_attend_part(DevLayout L, const void* blob, const T* Q,
                                                     const int32_t* uni, const int32_t* n_uni, int uni_stride,
                                                     float scale, float* part) {
  constexpr int ROWB = D * (int)sizeof(T);
  constexpr int LDSB = ROWB + 16;     // padded row stride: rows start on different banks
  constexpr int DPL = D / 64;         // output dims per lane
  __shared__ __attribute__((aligned(16))) char Kt[kRows * LDSB];
  __shared__ __attribute__((aligned(16))) char Vt[kRows * LDSB];
  __shared__ __attribute__((aligned(16))) float qs[ICE_MAX_GROUP * D];
  __shared__ float ps[4][kRows];
  __shared__ int32_t rowcnt[kBatchPages];
  __shared__ int32_t rowpg[kBatchPages];

  const int h = blockIdx.y, split = blockIdx.x, nsplit = gridDim.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = L.G;
  const void* hb = head_base(blob, L, h);
  const T* pgK = at<T>(hb, L.off_pgK[0]);
  const T* pgV = at<T>(hb, L.off_pgV);
  const int32_t* pg_cnt = at<int32_t>(hb, L.off_pg_cnt[0]);
  const int n_pages = at<Hdr>(hb, L.off_hdr)->n_pages[0];
  const int nu = min(n_uni[h], uni_stride);
  const int pbeg = split * kPagesPerSplit;
  const int pend = min(nu, pbeg + kPagesPerSplit);

  for (int i = threadIdx.x; i < G * D; i += 256)
    qs[i] = Elt<T>::load(Q, (int64_t)h * G * D + i) * (scale * kLog2e);

  float m[kMaxQPerWave], l[kMaxQPerWave], o[kMaxQPerWave][DPL];
#pragma unroll
  for (int j = 0; j < kMaxQPerWave; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.0f;
#pragma unroll
    for (int c = 0; c < DPL; ++c) o[j][c] = 0.0f;
  }

  for (int pb = pbeg; pb < pend; pb += kBatchPages) {
    const int npg = min(kBatchPages, pend - pb);
    __syncthreads();
    if (threadIdx.x < kBatchPages) {
      int pg = threadIdx.x < npg ? uni[(int64_t)h * uni_stride + pb + threadIdx.x] : -1;
      if (pg >= n_pages) pg = -1;   // ids outside the page table are ignored
      rowpg[threadIdx.x] = pg;
      rowcnt[threadIdx.x] = pg >= 0 ? pg_cnt[pg] : 0;
    }
    __syncthreads();
    constexpr int CPR = ROWB / 16;    // 16-byte chunks per row
    for (int c = threadIdx.x; c < kRows * CPR; c += 256) {
      const int r = c / CPR, q = c % CPR;
      const int pg = rowpg[r / ICE_PAGE_CAP];
      V4 kx = {0, 0, 0, 0}, vx = {0, 0, 0, 0};
      if (pg >= 0 && (r % ICE_PAGE_CAP) < rowcnt[r / ICE_PAGE_CAP]) {
        const int64_t row = (int64_t)pg * ICE_PAGE_CAP + (r % ICE_PAGE_CAP);
        kx = *reinterpret_cast<const V4*>(reinterpret_cast<const char*>(pgK + row * D) + q * 16);
        vx = *reinterpret_cast<const V4*>(reinterpret_cast<const char*>(pgV + row * D) + q * 16);
      }
      *reinterpret_cast<V4*>(Kt + r * LDSB + q * 16) = kx;
      *reinterpret_cast<V4*>(Vt + r * LDSB + q * 16) = vx;
    }
    __syncthreads();
    const bool valid = rowpg[lane / ICE_PAGE_CAP] >= 0 && (lane % ICE_PAGE_CAP) < rowcnt[lane / ICE_PAGE_CAP];
#pragma unroll
    for (int j = 0; j < kMaxQPerWave; ++j) {
      const int g = wave + 4 * j;
      if (g >= G) break;
      // logit of row `lane` for query g
      float s = -INFINITY;
      if (valid) {
        float acc = 0.0f;
        const float* qg = qs + g * D;
#pragma unroll 4
        for (int c = 0; c < ROWB / 16; ++c) {
          const V4 kv = *reinterpret_cast<const V4*>(Kt + lane * LDSB + c * 16);
          float f[Elt<T>::per16];
          Elt<T>::unpack(kv, f);
#pragma unroll
          for (int i = 0; i < Elt<T>::per16; ++i) acc = fmaf(qg[c * Elt<T>::per16 + i], f[i], acc);
        }
        s = acc;
      }
      const float mt = wave_max(s);
      if (mt == -INFINITY) continue;
      const float mn = fmaxf(m[j], mt);
      const float corr = exp2f(m[j] - mn);
      const float p = valid ? exp2f(s - mn) : 0.0f;
      l[j] = l[j] * corr + wave_sum(p);
      m[j] = mn;
#pragma unroll
      for (int c = 0; c < DPL; ++c) o[j][c] *= corr;
      ps[wave][lane] = p;
      wave_sync();
      for (int r = 0; r < kRows; ++r) {
        const float pr = ps[wave][r];
#pragma unroll
        for (int c = 0; c < DPL; ++c) {
          const int dim = lane * DPL + c;
          const float vv = sizeof(T) == 4 ? *reinterpret_cast<const float*>(Vt + r * LDSB + dim * 4)
                                          : bf16_to_f32(*reinterpret_cast<const uint16_t*>(Vt + r * LDSB + dim * 2));
          o[j][c] = fmaf(pr, vv, o[j][c]);
        }
      }
      wave_sync();
    }
  }
  // partials [h][split][g] = (m, l, o[D])
#pragma unroll
  for (int j = 0; j < kMaxQPerWave; ++j) {
    const int g = wave + 4 * j;
    if (g >= G) break;
    float* dst = part + (((int64_t)h * nsplit + split) * G + g) * (D + 2);
    if (lane == 0) {
      dst[0] = m[j];
      dst[1] = l[j];
    }
#pragma unroll
    for (int c = 0; c < DPL; ++c) dst[2 + lane * DPL + c] = o[j][c];
  }
}

template <int D>
__global__ void k_attend_combine(int G, int nsplit, const float* part, float* O, float* lse) {
  constexpr int DPL = D / 64;
  const int h = blockIdx.x;
  const int g = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (g >= G) return;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part[(((int64_t)h * nsplit + s) * G + g) * (D + 2)]);
  float Ls = 0.0f, o[DPL];
#pragma unroll
  for (int c = 0; c < DPL; ++c) o[c] = 0.0f;
  if (M > -INFINITY) {
    for (int s = 0; s < nsplit; ++s) {
      const float* p = part + (((int64_t)h * nsplit + s) * G + g) * (D + 2);
      if (p[0] == -INFINITY) continue;
      const float w = exp2f(p[0] - M);
      Ls = fmaf(p[1], w, Ls);
#pragma unroll
      for (int c = 0; c < DPL; ++c) o[c] = fmaf(p[2 + lane * DPL + c], w, o[c]);
    }
  }
  float* out = O + ((int64_t)h * G + g) * D;
  const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
#pragma unroll
  for (int c = 0; c < DPL; ++c) out[lane * DPL + c] = o[c] * inv;
  if (lse && lane == 0) lse[(int64_t)h * G + g] = Ls > 0.0f ? (M + log2f(Ls)) * kLn2 : -INFINITY;
}

}  // namespace

int attend_splits(int uni_stride) {
  const int n = (uni_stride + kPagesPerSplit - 1) / kPagesPerSplit;
  return n < 1 ? 1 : n;
}

hipError_t launch_attend(const DevLayout& L, const void* blob, const void* Q, const int32_t* uni,
                         const int32_t* n_uni, int uni_stride, float scale, float* O, float* lse, void* ws,
                         hipStream_t s) {
  const int nsplit = attend_splits(uni_stride);
  float* part = static_cast<float*>(ws);
  const dim3 grid((unsigned)nsplit, (unsigned)L.H);
  if (L.dtype == ICE_BF16) {
    const uint16_t* q = static_cast<const uint16_t*>(Q);
    if (L.d == 128) k_attend_part<128, uint16_t><<<grid, 256, 0, s>>>(L, blob, q, uni, n_uni, uni_stride, scale, part);
    else k_attend_part<64, uint16_t><<<grid, 256, 0, s>>>(L, blob, q, uni, n_uni, uni_stride, scale, part);
  } else {
    const float* q = static_cast<const float*>(Q);
    if (L.d == 128) k_attend_part<128, float><<<grid, 256, 0, s>>>(L, blob, q, uni, n_uni, uni_stride, scale, part);
    else k_attend_part<64, float><<<grid, 256, 0, s>>>(L, blob, q, uni, n_uni, uni_stride, scale, part);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (L.d == 128) k_attend_combine<128><<<(unsigned)L.H, 64 * L.G, 0, s>>>(L.G, nsplit, part, O, lse);
  else k_attend_combine<64><<<(unsigned)L.H, 64 * L.G, 0, s>>>(L.G, nsplit, part, O, lse);
  return hipGetLastError();
}

}  // namespace ice
