// Host-side launchers of the HIP kernels, one group per source file.
#pragma once

#include "ice_common.h"

namespace ice {

// k_build.hip
// heads of `blob` take the layout of the same-numbered heads of `src` (both
// range starts) and place their own rows into it
hipError_t launch_build_reuse(const DevLayout& L, const WsLayout& W, void* blob, const void* src, const void* K,
                              const void* V, int n_tokens, int64_t head_stride, void* ws, bool keep, hipStream_t s);
// Parts of a build, in the order they must run for a range of heads: the lift
// (fills, norms, levels and level lists), the parent search of level 0, and
// the rest (level 0's pack and page copies, the upper levels, the top list).
// A pipelined build runs the parts of different head ranges on two streams.
enum class BuildPart { kAll, kLift, kParent0, kRest };
// keep: a rebuild, which keeps the headers' resident counts and dense flags
// pd: parents by P-DCI instead of the exact search (nullptr: exact)
// ev: nullable, ICE_BUILD_PHASES + 1 events recorded on s at the phase boundaries
// pd and ev need part == kAll
hipError_t launch_build(const DevLayout& L, const WsLayout& W, void* blob, const void* K, const void* V,
                        int n_tokens, int64_t head_stride, void* ws, bool keep, hipStream_t s,
                        const PdciArgs* pd = nullptr, hipEvent_t* ev = nullptr, BuildPart part = BuildPart::kAll);
// k_gemm.hip: nearest parent of every level-`level` point among the level-(level+1) points
hipError_t launch_parent_gemm(const DevLayout& L, const WsLayout& W, void* blob, const void* K,
                              int64_t head_stride, void* ws, int level, hipStream_t s);
// k_pdci.hip: parent of every level-`level` point by P-DCI among the level-(level+1) points
hipError_t launch_parent_pdci(const DevLayout& L, const WsLayout& W, const PdciArgs& P, void* blob, const void* K,
                              int64_t head_stride, void* ws, int level, hipStream_t s);
// k_insert.hip
hipError_t launch_insert(const DevLayout& L, void* blob, const void* k_new, const void* v_new, int n_new,
                         int t0, hipStream_t s);
// k_select.hip
hipError_t launch_select(const DevLayout& L, const void* blob, const void* Q, int budget, int beam,
                         int32_t* sel, int32_t* uni, int32_t* n_uni, int32_t* trace, hipStream_t s);
// true if select + attend run as one fused kernel (bf16, lists of at most 64)
bool decode_fused(const DevLayout& L, int budget, int beam);
hipError_t launch_decode(const DevLayout& L, const void* blob, const void* Q, int budget, int beam, int32_t* sel,
                         int32_t* uni, int32_t* n_uni, float scale, float* O, float* lse, hipStream_t s);
// k_attend.hip
hipError_t launch_attend(const DevLayout& L, const void* blob, const void* Q, const int32_t* uni,
                         const int32_t* n_uni, int uni_stride, float scale, float* O, float* lse, void* ws,
                         hipStream_t s);
// host-pool mode: the V pages of every head's union from the host pool into L.vstage
hipError_t launch_gather_v(const DevLayout& L, const void* blob, const int32_t* uni, const int32_t* n_uni,
                           int uni_stride, hipStream_t s);
// fills `n` int32 words at byte offset `off` of every head region
hipError_t launch_set_resident(const DevLayout& L, void* blob, const void* K, const void* V, int n, int64_t hstride,
                               hipStream_t s);
hipError_t launch_fill_heads(void* base, int64_t head_bytes, int H, int64_t off, int64_t n, int32_t value,
                             hipStream_t s);

}  // namespace ice
