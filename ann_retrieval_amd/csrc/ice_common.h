// Internal definitions shared by the HIP sources of the IceCache library:
// the device-blob and workspace layouts, the per-head header, and small
// device helpers (promotion hash, bf16 conversion, sortable keys, row loads).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ice.h"

#define ICE_WAVE 64
#define ICE_ROOT (-1)

namespace ice {

// Per-head header at the start of every head's region of the blob. Mirrors
// ice_head_stats field by field so ice_export can copy it out directly.
struct Hdr {
  int32_t n_tokens;
  int32_t top_level;
  int32_t n_top;
  int32_t n_pages[ICE_MAX_LEVELS];
  int32_t clamps;
  int32_t splits;
  int32_t near_ties;
  int32_t overflow;        // page table full (ruled out within capacity)
  int32_t sync_timeouts;
  int32_t n_resident;      // resident tokens attended beside the pages
  int32_t dense;           // nonzero: attention covers every indexed page
  double M2;
};
static_assert(sizeof(Hdr) == sizeof(ice_head_stats), "header mirrors ice_head_stats");

// Byte offsets of every array inside one head's region of the index blob.
// Page table l (0 <= l < ntab) groups the level-l points by their level-(l+1)
// owner in pages of 16; table 0 is the KV page pool. When no token is
// promoted (one level, or an empty top), table 0 has the single owner ROOT,
// which is stored at owner slot `cap`.
struct DevLayout {
  int32_t H, G, d, dtype, L, plog2, cap, ntab;
  int32_t h0;                    // absolute number of head 0 (a build of a head range)
  uint64_t seed;
  int32_t ncap[ICE_MAX_LEVELS];  // max over heads of #positions < cap with level >= l
  int32_t pcap[ICE_MAX_LEVELS];  // page capacity of table l
  int32_t res_pages;             // resident pages per head, after table 0's pcap[0] pages
  int32_t topcap;                // capacity of the top list
  int32_t elt;                   // bytes per element of K/V/Q
  int32_t resort;                // nonzero: inserts split by re-sorting (ICE_SPLIT_RESORT)
  int64_t head_bytes;            // stride between heads
  int64_t off_hdr, off_lev, off_e;
  int64_t off_parent[ICE_MAX_LEVELS];
  int64_t off_pg_tok[ICE_MAX_LEVELS], off_pg_cnt[ICE_MAX_LEVELS], off_pg_next[ICE_MAX_LEVELS];
  int64_t off_pg_owner[ICE_MAX_LEVELS], off_first[ICE_MAX_LEVELS], off_tail[ICE_MAX_LEVELS];
  // per owner slot: pages in the contiguous run that starts at first[], and
  // the owner's member count (its pages are all full except the last)
  int64_t off_orun[ICE_MAX_LEVELS], off_ocnt[ICE_MAX_LEVELS];
  int64_t off_pgK[ICE_MAX_LEVELS], off_pgE[ICE_MAX_LEVELS], off_pgV;
  int64_t off_top_tok, off_top_K, off_top_E;
  // Host-pool mode: level-0 V pages live outside the blob, in pinned host
  // memory mapped into the device address space (head h at vpool + h *
  // vpool_head_bytes, same page layout); off_pgV is then unused. Attention
  // reads V from vstage when it is set: the V page of union entry u of head h
  // at vstage + (h * vstage_pages + u) * page bytes.
  char* vpool;
  int64_t vpool_head_bytes;
  const char* vstage;
  int32_t vstage_pages;
};

// Level-0 V pages of head h (hb = its region of the blob).
__host__ __device__ inline char* v_pages(const DevLayout& L, void* hb, int h) {
  return L.vpool ? L.vpool + (int64_t)h * L.vpool_head_bytes : static_cast<char*>(hb) + L.off_pgV;
}
__host__ __device__ inline const char* v_pages(const DevLayout& L, const void* hb, int h) {
  return L.vpool ? L.vpool + (int64_t)h * L.vpool_head_bytes : static_cast<const char*>(hb) + L.off_pgV;
}

// Candidate rows per stage of the parent GEMM, and the operand rows readable
// past the last candidate: two stages.
constexpr int kGemmTile = 64;
constexpr int kGemmPadRows = 2 * kGemmTile;
// tokens per block of the lift: the per-block level counts are kept per
// kLiftBlock tokens
constexpr int kLiftBlock = 256;

// Build workspace, also laid out per head.
struct WsLayout {
  int32_t kp;                    // padded reduction length of the parent GEMM operand
  int64_t head_bytes;
  int64_t off_n2;                // f64 [cap]
  int64_t off_rank[ICE_MAX_LEVELS];   // i32 [cap], l >= 1: position of t in pts[l], -1 if absent
  int64_t off_pts[ICE_MAX_LEVELS];    // i32 [ncap[l]], l >= 1: points with level >= l, ascending
  int64_t off_exact[ICE_MAX_LEVELS];  // i32 [ncap[l]]: points with level == l, ascending
  int64_t off_cnts;              // i32 [2*ICE_MAX_LEVELS]: n_ge[l], n_eq[l]
  int64_t off_blkcnt;            // i32 [ceil(cap / kLiftBlock)][2*ICE_MAX_LEVELS]: a token block's n_ge, n_eq,
                                 // then (scanned) the counts before it
  int64_t off_opA;               // elt [ncap[1]][kp]: candidate-parent operand rows
  int64_t off_s1, off_s2;        // f32 [cap]: best / runner-up parent score per token
  int64_t off_oloc;              // i32 [cap]: owner slot of each point
  int64_t off_cnt, off_fill, off_cbase, off_pbase;  // i32 [ncap[1]+1]
  int64_t off_brec;              // bucketed points: (score bits, token, owner, 0) int4 [cap]
  int64_t build_bytes;           // H * head_bytes
  // P-DCI parent search (ice_build_pdci): a region after the per-head
  // build workspace holding, per head and simple index, ncap[1] keys by
  // candidate, the sorted keys, the sorted candidates and their positions
  int64_t pdci_bytes;
};

// P-DCI parameters and arrays of one build; element (h, k, c) of each array
// sits at (h * ICE_PDCI_MAX_KEYS + k) * stride + c.
struct PdciArgs {
  const float* dirs;             // [mk][d+1] directions, simple index k of composite j is row j*l + k
  int32_t m, l, mk, visits, cands;
  int32_t stride;                // ncap[1]
  double* keys;                  // keys by candidate
  double* skeys;                 // keys in ascending (key, candidate) order
  int32_t* sidx;                 // candidates in that order
  int32_t* posof;                // position of each candidate in that order
};

template <class T>
__host__ __device__ inline T* at(void* base, int64_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}
template <class T>
__host__ __device__ inline const T* at(const void* base, int64_t off) {
  return reinterpret_cast<const T*>(static_cast<const char*>(base) + off);
}

// The pages one head attends: the explicit ids u[0..nu) (the group's union;
// ids outside the head's page table are skipped as -1) or, for a dense head,
// every page [0, n_pages); then its resident pages, which follow the page
// pool's pcap[0] pages.
struct PageSrc {
  const int32_t* u;
  int nu, n_pages, dense, res_base, nr;
  __device__ inline int count() const { return (dense ? n_pages : nu) + nr; }
  __device__ inline int at(int i) const {
    const int n0 = dense ? n_pages : nu;
    if (i >= n0) return res_base + (i - n0);
    if (dense) return i;
    const int p = u[i];
    return p >= 0 && p < n_pages ? p : -1;
  }
};
__device__ inline PageSrc page_src(const DevLayout& L, const void* hb, const int32_t* u, int nu) {
  const Hdr* hdr = at<Hdr>(hb, L.off_hdr);
  PageSrc s;
  s.u = u;
  s.nu = nu;
  s.n_pages = hdr->n_pages[0];
  s.dense = hdr->dense;
  s.res_base = L.pcap[0];
  s.nr = (hdr->n_resident + 15) / 16;
  return s;
}


__host__ __device__ inline void* head_base(void* blob, const DevLayout& L, int h) {
  return static_cast<char*>(blob) + (int64_t)h * L.head_bytes;
}
__host__ __device__ inline const void* head_base(const void* blob, const DevLayout& L, int h) {
  return static_cast<const char*>(blob) + (int64_t)h * L.head_bytes;
}

// ---- promotion draw ------------------------------------------------------
// SplitMix64 (Steele, Lea & Flood, OOPSLA 2014): output i of the generator
// seeded with s is mix(s + (i+1) * golden_gamma). Head h uses the stream
// seeded with seed + h * 2^40 and token t takes output t; the level is the
// number of trailing zero bits divided by promote_log2, capped at L-1 (the
// article's section 3: a random part is promoted, and a smaller random part
// of that part again).
__host__ __device__ inline uint64_t splitmix64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__host__ __device__ inline int draw_level(uint64_t seed, int h, int t, int L, int plog2) {
  const uint64_t s = seed + ((uint64_t)h << 40);
  const uint64_t z = splitmix64_mix(s + (uint64_t)(t + 1) * 0x9E3779B97F4A7C15ull);
  const int c = z ? __builtin_ctzll(z) : 64;
  const int lv = c / plog2;
  return lv < L - 1 ? lv : L - 1;
}

// ---- element conversion ---------------------------------------------------
__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest even; inputs here are finite.
__device__ inline uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Sortable 64-bit key: larger score first, then smaller id. Never 0 for a
// finite score, so 0 marks an empty slot.
__device__ inline uint32_t ordered_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline uint64_t make_key(float score, int32_t id) {
  return ((uint64_t)ordered_bits(score) << 32) | (uint64_t)(~(uint32_t)id);
}
__device__ inline int32_t key_id(uint64_t k) { return (int32_t)(~(uint32_t)(k & 0xffffffffu)); }

// 16-byte vector load/store helpers.
struct alignas(16) V4 {
  uint32_t x, y, z, w;
};

template <class T>
struct Elt;
template <>
struct Elt<float> {
  static constexpr int per16 = 4;
  __device__ static inline void unpack(const V4& v, float* out) {
    out[0] = __uint_as_float(v.x);
    out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z);
    out[3] = __uint_as_float(v.w);
  }
  __device__ static inline float load(const void* p, int64_t i) { return static_cast<const float*>(p)[i]; }
};
template <>
struct Elt<uint16_t> {
  static constexpr int per16 = 8;
  __device__ static inline void unpack(const V4& v, float* out) {
    out[0] = __uint_as_float(v.x << 16);
    out[1] = __uint_as_float(v.x & 0xffff0000u);
    out[2] = __uint_as_float(v.y << 16);
    out[3] = __uint_as_float(v.y & 0xffff0000u);
    out[4] = __uint_as_float(v.z << 16);
    out[5] = __uint_as_float(v.z & 0xffff0000u);
    out[6] = __uint_as_float(v.w << 16);
    out[7] = __uint_as_float(v.w & 0xffff0000u);
  }
  __device__ static inline float load(const void* p, int64_t i) {
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  }
};

// Row geometry for a head dimension D of element type T: a row is split in
// 16-byte slices, LPR lanes per row, RPP rows per wave pass.
template <int D, class T>
struct RowGeo {
  static constexpr int bytes = D * (int)sizeof(T);
  static constexpr int LPR = bytes / 16;
  static constexpr int RPP = ICE_WAVE / LPR;
  static constexpr int EPL = 16 / (int)sizeof(T);
};

// Sum over groups of `width` consecutive lanes (width a power of two <= 64).
template <int width>
__device__ inline float group_sum(float v) {
#pragma unroll
  for (int m = 1; m < width; m <<= 1) v += __shfl_xor(v, m, ICE_WAVE);
  return v;
}
template <int width>
__device__ inline double group_sum_d(double v) {
#pragma unroll
  for (int m = 1; m < width; m <<= 1) v += __shfl_xor(v, m, ICE_WAVE);
  return v;
}

// Orders this lane's earlier LDS writes before later LDS reads of any lane
// of the same wave.
__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// ---- cross-lane exchange on the VALU (no LDS round trip) -----------------
// xor_lane<m>(x) returns x from lane ^ m. m = 1, 2: DPP quad permutes; m = 4:
// two DPP row shifts under bank masks (banks 0 and 2 of a row read lane + 4,
// banks 1 and 3 lane - 4; a bank is 4 lanes of a 16-lane row); m = 8:
// row_ror:8; m = 16, 32: the gfx950 permlane16 / permlane32 swaps. The DPP
// moves leave no lane unwritten, so they need no initial value. All lanes of
// the wave must be active.
template <int m>
__device__ inline int xor_lane(int x) {
  if constexpr (m == 1) {
    return __builtin_amdgcn_mov_dpp(x, 0xb1, 0xf, 0xf, false);     // quad_perm [1,0,3,2]
  } else if constexpr (m == 2) {
    return __builtin_amdgcn_mov_dpp(x, 0x4e, 0xf, 0xf, false);     // quad_perm [2,3,0,1]
  } else if constexpr (m == 4) {
    const int y = __builtin_amdgcn_update_dpp(x, x, 0x104, 0xf, 0x5, false);   // row_shl:4, banks 0, 2
    return __builtin_amdgcn_update_dpp(y, x, 0x114, 0xf, 0xa, false);          // row_shr:4, banks 1, 3
  } else if constexpr (m == 8) {
    return __builtin_amdgcn_mov_dpp(x, 0x128, 0xf, 0xf, false);    // row_ror:8
  } else if constexpr (m == 16) {
    // lanes with bit 4 set take the swapped-in lower row (a constant lane mask)
    const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return __builtin_amdgcn_inverse_ballot_w64(0xffff0000ffff0000ull) ? (int)p[0] : (int)p[1];
  } else {
    static_assert(m == 32, "xor distance");
    const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return __builtin_amdgcn_inverse_ballot_w64(0xffffffff00000000ull) ? (int)p[0] : (int)p[1];
  }
}
template <int m>
__device__ inline float xor_lane_f(float x) {
  return __int_as_float(xor_lane<m>(__float_as_int(x)));
}
template <int m>
__device__ inline uint64_t xor_lane_u64(uint64_t x) {
  const int lo = xor_lane<m>((int)(uint32_t)x), hi = xor_lane<m>((int)(uint32_t)(x >> 32));
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int m = 1; m < ICE_WAVE; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, ICE_WAVE));
  return v;
}
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < ICE_WAVE; m <<= 1) v += __shfl_xor(v, m, ICE_WAVE);
  return v;
}

}  // namespace ice
