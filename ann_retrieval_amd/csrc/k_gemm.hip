// Nearest parent of every level-l point among the level-(l+1) points: a
// distance GEMM on the matrix cores fused with a running argmax.
//
// The aitangshan.cn IceCache article (section 3) gives every point the most
// similar point one level up as its parent, after a lift that turns inner
// product into Euclidean distance. For lifted keys x = [k, e] with |x| = M,
// |x_i - x_j|^2 = 2M^2 - 2 s_ij with s_ij = k_i.k_j + e_i e_j, so the nearest
// parent is the argmax of s over the candidates; ties go to the lower token
// id (the candidates are in ascending token order).
//
// Layout (bf16, gfx950 v_mfma_f32_32x32x16_bf16): candidate parents are the
// MFMA rows (A operand, streamed through double-buffered LDS in stages of 64
// rows, each stage's global loads issued before the previous stage's MFMAs),
// children the columns (B operand, kept in registers for the whole sweep: two
// 32-child fragments per wave, whose MFMA chains interleave). Each lane then
// owns one child column per fragment and 16 parent rows of every 32-row
// block, so the argmax runs inside the lane's accumulators (a v_max3 fold per
// 32-row block, and a copy of the block's scores when it holds a new best)
// with one cross-lane step at the end. The
// e_i e_j term rides in one extra k-step: e is split into three bf16 parts
// and six of the products are laid out as extra columns (the dropped terms
// are below 2^-24 relative).
#include "ice_launch.h"

namespace ice {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kChildBf16 = 256;  // children per block: 4 waves x 64 (bf16), 4 waves x 32 (fp32)
constexpr int kChildF32 = 128;
constexpr uint16_t kBf16One = 0x3F80;

struct GemmView {
  int h;
  bool skip;
  int n_child, n_cand;
  const int32_t* exact;
  const int32_t* pts;
  char* wh;
  Hdr* hdr;
};

// Block (child block cb, head h) of the parent search from the 1-D launch
// index. Consecutive launch indices go to the 8 XCDs in turn; the mapping
// hands each XCD a contiguous range of (head, child block) pairs, so the
// blocks that share a head's candidate operand share one L2. nbx: child
// blocks per head; the last total % 8 indices keep their own position.
struct GemmBlock {
  int cb, h;
};
__device__ inline GemmBlock gemm_block(int nbx, int H) {
  const int b = blockIdx.x, total = nbx * H, q = total / 8;
  const int logical = b < 8 * q ? (b % 8) * q + b / 8 : b;
  return GemmBlock{logical % nbx, logical / nbx};
}

__device__ inline GemmView gemm_view(const DevLayout& L, const WsLayout& W, void* blob, void* ws, int level, int h) {
  GemmView v;
  void* hb = head_base(blob, L, h);
  v.hdr = at<Hdr>(hb, L.off_hdr);
  v.wh = static_cast<char*>(ws) + (int64_t)h * W.head_bytes;
  v.skip = level >= v.hdr->top_level;
  const int32_t* cnts = at<int32_t>(v.wh, W.off_cnts);
  v.n_child = cnts[ICE_MAX_LEVELS + level];
  v.n_cand = cnts[level + 1];
  v.exact = at<int32_t>(v.wh, W.off_exact[level]);
  v.pts = at<int32_t>(v.wh, W.off_pts[level + 1]);
  v.h = h;
  return v;
}

// Running best / runner-up over the lane's rows. Rows arrive in increasing
// order, so a strict comparison keeps the lowest index among equal scores.
struct ArgMax {
  float best = -INFINITY, second = -INFINITY;
  int idx = 0x7fffffff;
  __device__ inline void push(float s, int p) {
    if (s > best) {
      second = best;
      best = s;
      idx = p;
    } else {
      second = fmaxf(second, s);
    }
  }
  // Combine with the other half-wave holding the same child column.
  __device__ inline void merge_halves() {
    const float ob = __shfl_xor(best, 32, 64);
    const float os = __shfl_xor(second, 32, 64);
    const int oi = __shfl_xor(idx, 32, 64);
    if (ob > best || (ob == best && oi < idx)) {
      second = fmaxf(best, os);
      best = ob;
      idx = oi;
    } else {
      second = fmaxf(second, ob);
    }
  }
};

__device__ inline void write_parent(const DevLayout& L, const WsLayout& W, const GemmView& v, void* blob,
                                    int level, int ctok, const ArgMax& a) {
  const int h = v.h;
  void* hb = head_base(blob, L, h);
  // a.idx is unset only if every score was NaN (non-finite input): fall back
  // to the first candidate rather than index out of range
  const int pi = (a.idx >= 0 && a.idx < v.n_cand) ? a.idx : 0;
  at<int32_t>(hb, L.off_parent[level])[ctok] = v.pts[pi];
  at<float>(v.wh, W.off_s1)[ctok] = a.best;
  at<float>(v.wh, W.off_s2)[ctok] = a.second;
  // lifted distances D = 2(M^2 - s): near-tie when D2 - D1 < 1e-4 D2
  const float M2 = (float)v.hdr->M2;
  if (a.second > -INFINITY && (a.best - a.second) < 1e-4f * (M2 - a.second)) atomicAdd(&v.hdr->near_ties, 1);
}

// Running best / runner-up of one lane over its rows of one child column, by
// 32-row blocks (16 scores per lane and block). Per block: the block's max
// by a v_max3 chain; if it beats the running best (strict, so equal scores
// keep the earlier block, i.e. the lower rows), the block's 16 scores are
// kept and the block recorded; `second` tracks the best of every other
// block's max (v_med3 of the old best, itself and the block max). At the end
// the kept block gives the winning row (its first score equal to the best:
// rows increase with the accumulator index) and its own runner-up, so best,
// row and runner-up equal a score-by-score scan of the lane's rows.
struct LaneMax {
  float best = -INFINITY, second = -INFINITY;
  int blk = -1;
  float kept[16];
  __device__ inline void push_block(const float (&s)[16], int b) {
    float bm = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
    for (int j = 3; j < 15; j += 2) bm = fmaxf(fmaxf(bm, s[j]), s[j + 1]);
    bm = fmaxf(bm, s[15]);
    const bool gt = bm > best;
    second = __builtin_amdgcn_fmed3f(best, second, bm);
    best = gt ? bm : best;
    blk = gt ? b : blk;
    // selects, not a branch: the block's MFMAs and the previous block's
    // epilogue stay in one basic block, so the scheduler can interleave them
#pragma unroll
    for (int j = 0; j < 16; ++j) kept[j] = gt ? s[j] : kept[j];
  }
  // winning accumulator index j (first one equal to the best) and the
  // runner-up over all the lane's scores
  __device__ inline int finish(float& runner_up) const {
    int jb = 15;
#pragma unroll
    for (int j = 14; j >= 0; --j) jb = kept[j] == best ? j : jb;
    float r = second;
#pragma unroll
    for (int j = 0; j < 16; ++j) r = j == jb ? r : fmaxf(r, kept[j]);
    runner_up = r;
    return jb;
  }
};

// 16 bytes per lane from global memory into LDS without registers
// (global_load_lds_dwordx4): lane i writes bytes 16 i .. 16 i + 15 of the
// wave-uniform LDS address `lds_run` (through m0, which this kernel uses for
// nothing else). Written as inline assembly: the compiler then does not treat
// the copy as an LDS store that every later LDS read must wait for, which
// would wait for the stages still in flight; the kernel waits for its own
// stages (vmcnt, then a barrier) before reading them.
__device__ inline void load_to_lds16(const void* src, void* lds_run) {
  const uint32_t m = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_run;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(__builtin_amdgcn_readfirstlane((int)m)) : "memory", "m0");
}
// Waits until this wave's vector-memory loads are complete.
__device__ inline void wait_vm_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Waits until at most N of this wave's vector-memory loads are outstanding
// (they complete in issue order).
template <int N>
__device__ inline void wait_vm_loads_le() {
  if constexpr (N == 1) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
  else if constexpr (N == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
  else if constexpr (N == 3) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
  else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
}

template <int D>
__global__ __launch_bounds__(256, 2) void k_parent_bf16(DevLayout L, WsLayout W, void* blob, const uint16_t* K,
                                                     int64_t hstride, void* ws, int level, int nbx) {
  constexpr int KP = D + 16;            // operand row length (elements)
  constexpr int KS = KP / 16;           // k-steps of 16
  constexpr int ROWB = KP * 2;          // operand row bytes
  constexpr int LDSB = ROWB + 16;       // padded LDS row stride
  constexpr int TILE = kGemmTile;       // candidate rows per stage
  constexpr int NB = TILE / 32;         // 32-row MFMA blocks per stage (even)
  static_assert(NB % 2 == 0, "blocks alternate between two accumulator sets");
  constexpr int NF = 2;                 // 32-child fragments per wave
  __shared__ __attribute__((aligned(16))) char tile[3][TILE * LDSB];

  const GemmBlock gb = gemm_block(nbx, L.H);
  const GemmView v = gemm_view(L, W, blob, ws, level, gb.h);
  if (v.skip) return;
  const int c0 = gb.cb * kChildBf16;
  if (c0 >= v.n_child) return;
  const int h = gb.h;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const float* e = at<float>(head_base(blob, L, h), L.off_e);
  const uint16_t* Kh = K + (int64_t)h * hstride;
  const char* opA = reinterpret_cast<const char*>(at<uint16_t>(v.wh, W.off_opA));
  const int half = lane >> 5;

  // child operands: fragment f holds column lane%32 = child c0 + 64 wave + 32 f
  // + lane%32, k elements 8*(lane/32) .. +7 of each step
  int ctok[NF];
  bool cvalid[NF];
  bf16x8 bfr[NF][KS];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int ci = c0 + wave * 64 + f * 32 + (lane & 31);
    cvalid[f] = ci < v.n_child;
    ctok[f] = cvalid[f] ? v.exact[ci] : 0;
#pragma unroll
    for (int ks = 0; ks < KS - 1; ++ks) {
      V4 x = {0, 0, 0, 0};
      if (cvalid[f]) x = *reinterpret_cast<const V4*>(Kh + (int64_t)ctok[f] * D + ks * 16 + half * 8);
      bfr[f][ks] = __builtin_bit_cast(bf16x8, x);
    }
    V4 x = {0, 0, 0, 0};
    if (cvalid[f] && half == 0) {
      const float ev = e[ctok[f]];
      const uint16_t a0 = f32_to_bf16(ev);
      const float r1 = ev - bf16_to_f32(a0);
      const uint16_t a1 = f32_to_bf16(r1);
      const uint16_t a2 = f32_to_bf16(r1 - bf16_to_f32(a1));
      // child side of the six lift products: c0 c0 c1 c0 c2 c1
      x.x = (uint32_t)a0 | ((uint32_t)a0 << 16);
      x.y = (uint32_t)a1 | ((uint32_t)a0 << 16);
      x.z = (uint32_t)a2 | ((uint32_t)a1 << 16);
    }
    // column 15 of the step is 1: it carries the padding rows' sentinel
    if (half == 1) x.w = (uint32_t)kBf16One << 16;
    bfr[f][KS - 1] = __builtin_bit_cast(bf16x8, x);
  }

  // Candidate stages go from global memory straight into LDS
  // (global_load_lds_dwordx4: lane i of an instruction fills 16-byte slot i
  // of a 1 KiB run, no registers held) while the two stages before them are
  // used. A
  // stage is TILE rows of 18 slots each plus one pad slot (the padded row
  // stride LDSB), TILE * 19 slots in runs of 64, split over the 4 waves; a pad
  // slot loads its row's first 16 bytes, never read. The loads carry no
  // bounds checks: the operand has kGemmPadRows readable rows past the last
  // candidate, and those rows score far below any candidate (their sentinel
  // column), so the argmax needs no row mask.
  static_assert(2 * TILE <= kGemmPadRows, "stage loads past the candidates");
  static_assert(LDSB == ROWB + 16, "one pad slot per row");
  constexpr int SLOTS_ROW = LDSB / 16;               // 19
  constexpr int RUNS = TILE * SLOTS_ROW / 64;        // runs of 64 slots per stage
  static_assert(TILE * SLOTS_ROW % 64 == 0, "whole runs");
  constexpr int RPW = (RUNS + 3) / 4;                // runs per wave
  // wave w takes runs w, w + 4, ...; where that passes the last run, the
  // wave loads its previous run again (the same bytes to the same place), so
  // every wave issues RPW loads per stage and no load is conditional
  uint32_t goff[RPW];
  int lrun[RPW];
#pragma unroll
  for (int m = 0; m < RPW; ++m) {
    lrun[m] = wave + 4 * m < RUNS ? wave + 4 * m : wave + 4 * (m - 1);
    const int sl = lrun[m] * 64 + lane;
    const int r = min(sl / SLOTS_ROW, TILE - 1), q = sl % SLOTS_ROW;
    goff[m] = (uint32_t)(r * ROWB + (q < SLOTS_ROW - 1 ? q * 16 : 0));
  }
  auto load_stage = [&](int t, char* buf) {
    const char* base = opA + (int64_t)t * TILE * ROWB;
#pragma unroll
    for (int m = 0; m < RPW; ++m) load_to_lds16(base + goff[m], buf + lrun[m] * 1024);
  };
  // this wave's stage loads have landed (their LDS writes are done)
  auto loads_done = [&]() { wait_vm_loads(); };
  // the older of this wave's two stages in flight has landed: at most the
  // newer stage's RPW loads are outstanding (loads complete in issue order)
  static_assert(RPW >= 1 && RPW <= 5, "wait counts below");
  auto older_stage_done = [&]() { wait_vm_loads_le<RPW>(); };

  LaneMax am[NF];
  // A pieces of 32-row block rb of a stage buffer
  auto read_a = [&](const char* buf, int rb, V4 (&a)[KS]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      a[ks] = *reinterpret_cast<const V4*>(buf + (rb * 32 + (lane & 31)) * LDSB + ks * 32 + half * 16);
  };
  // MFMAs of one 32-row block from its A pieces
  auto mfma_regs = [&](const V4 (&a)[KS], f32x16 (&acc)[NF]) {
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[f] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int f = 0; f < NF; ++f)
        acc[f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[ks]), bfr[f][ks], acc[f], 0, 0, 0);
    }
  };
  // argmax of 32-row block `blk` (accumulator j of a lane is row 8 (j/4) +
  // 4 half + j%4 of the block)
  auto epilogue = [&](const f32x16 (&acc)[NF], int blk) {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      float sc[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) sc[j] = acc[f][j];
      am[f].push_block(sc, blk);
    }
  };
  // Software pipeline over 32-row blocks: a block's MFMAs are issued before
  // the previous block's argmax, so the matrix cores work while the vector
  // ALUs fold the previous scores. Three stage buffers: stage t (NB blocks)
  // sits in `cur`, stage t + 1 in `nxt`, stage t + 2 is on its way into the
  // third; once every wave is past stage t (one barrier), stage t + 3 is
  // loaded into `cur`, so each stage has two stages' time to land. The last
  // stage runs the same straight-line code: it multiplies a stage of padding
  // rows whose scores are dropped.
  // Block 1 of a stage is read from LDS into registers while block 0's MFMAs
  // run (a1), so its MFMAs start without waiting for LDS.
  static_assert(NB == 2, "two blocks per stage");
  const int n_tiles = (v.n_cand + TILE - 1) / TILE;
  f32x16 accA[NF], accB[NF];
  V4 a0[KS], a1[KS];
  load_stage(0, tile[0]);
  load_stage(min(1, n_tiles), tile[1]);
  older_stage_done();                              // stage 0 is in tile[0]
  __syncthreads();
  load_stage(min(2, n_tiles), tile[2]);
  read_a(tile[0], 0, a0);
  read_a(tile[0], 1, a1);
  mfma_regs(a0, accA);                             // block (0, 0)
  // blocks of a stage alternate between the accumulator sets A (block 0)
  // and B (block 1)
  auto stage = [&](int t, char* cur, char* nxt) {
    mfma_regs(a1, accB);                           // block (t, 1)
    epilogue(accA, NB * t);                        // block (t, 0)
    older_stage_done();                            // stage t + 1 is in nxt
    __syncthreads();
    load_stage(min(t + 3, n_tiles), cur);          // at most one stage past the candidates' last stage
    read_a(nxt, 0, a0);
    read_a(nxt, 1, a1);
    mfma_regs(a0, accA);                           // block (t + 1, 0)
    epilogue(accB, NB * t + 1);                    // block (t, 1)
  };
  // stages in threes, so each one's LDS buffers are fixed addresses
  for (int t = 0; t < n_tiles; t += 3) {
    stage(t, tile[0], tile[1]);
    if (t + 1 < n_tiles) stage(t + 1, tile[1], tile[2]);
    if (t + 2 < n_tiles) stage(t + 2, tile[2], tile[0]);
  }
  loads_done();   // no load may still write the LDS when the block ends
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    ArgMax a;
    float ru;
    const int j = am[f].finish(ru);
    a.best = am[f].best;
    a.second = ru;
    a.idx = am[f].blk >= 0 ? am[f].blk * 32 + 8 * (j >> 2) + (j & 3) + 4 * half : 0x7fffffff;
    a.merge_halves();
    if (lane < 32 && cvalid[f]) write_parent(L, W, v, blob, level, ctok[f], a);
  }
}

// fp32 inputs: v_mfma_f32_32x32x2f32, operand rows [key | e | 0 0 0].
template <int D>
__global__ __launch_bounds__(256) void k_parent_f32(DevLayout L, WsLayout W, void* blob, const float* K,
                                                    int64_t hstride, void* ws, int level, int nbx) {
  constexpr int KP = D + 4;
  constexpr int KS = (D + 2) / 2;       // k-steps of 2 over [key | e | 0]
  constexpr int LDSW = KP + 1;          // padded LDS row stride (floats)
  constexpr int TILE = 32;
  __shared__ float tile[TILE * LDSW];

  const GemmBlock gb = gemm_block(nbx, L.H);
  const GemmView v = gemm_view(L, W, blob, ws, level, gb.h);
  if (v.skip) return;
  const int c0 = gb.cb * kChildF32;
  if (c0 >= v.n_child) return;
  const int h = gb.h;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* e = at<float>(head_base(blob, L, h), L.off_e);
  const float* Kh = K + (int64_t)h * hstride;
  const float* opA = at<float>(v.wh, W.off_opA);

  const int ci = c0 + wave * 32 + (lane & 31);
  const bool cvalid = ci < v.n_child;
  const int ctok = cvalid ? v.exact[ci] : 0;
  const int half = lane >> 5;
  float bfr[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int col = 2 * ks + half;
    float x = 0.0f;
    if (cvalid) x = col < D ? Kh[(int64_t)ctok * D + col] : (col == D ? e[ctok] : 0.0f);
    bfr[ks] = x;
  }
  ArgMax am;
  for (int p0 = 0; p0 < v.n_cand; p0 += TILE) {
    __syncthreads();
    for (int c = threadIdx.x; c < TILE * KP; c += 256) {
      const int r = c / KP, q = c % KP;
      tile[r * LDSW + q] = p0 + r < v.n_cand ? opA[(int64_t)(p0 + r) * KP + q] : 0.0f;
    }
    __syncthreads();
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const float a = tile[(lane & 31) * LDSW + 2 * ks + half];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, bfr[ks], acc, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int p = p0 + 8 * (j >> 2) + 4 * half + (j & 3);
      if (p < v.n_cand) am.push(acc[j], p);
    }
  }
  am.merge_halves();
  if (lane < 32 && cvalid) write_parent(L, W, v, blob, level, ctok, am);
}

}  // namespace

hipError_t launch_parent_gemm(const DevLayout& L, const WsLayout& W, void* blob, const void* K,
                              int64_t head_stride, void* ws, int level, hipStream_t s) {
  const int n_child_max = L.ncap[level];
  const int per = L.dtype == ICE_BF16 ? kChildBf16 : kChildF32;
  const int nbx = (n_child_max + per - 1) / per;
  if (nbx == 0) return hipSuccess;
  const dim3 grid((unsigned)((int64_t)nbx * L.H));
  if (L.dtype == ICE_BF16) {
    const uint16_t* Kb = static_cast<const uint16_t*>(K);
    if (L.d == 128) k_parent_bf16<128><<<grid, 256, 0, s>>>(L, W, blob, Kb, head_stride, ws, level, nbx);
    else k_parent_bf16<64><<<grid, 256, 0, s>>>(L, W, blob, Kb, head_stride, ws, level, nbx);
  } else {
    const float* Kf = static_cast<const float*>(K);
    if (L.d == 128) k_parent_f32<128><<<grid, 256, 0, s>>>(L, W, blob, Kf, head_stride, ws, level, nbx);
    else k_parent_f32<64><<<grid, 256, 0, s>>>(L, W, blob, Kf, head_stride, ws, level, nbx);
  }
  return hipGetLastError();
}

}  // namespace ice
