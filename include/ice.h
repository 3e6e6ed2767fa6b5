/*
 * ice.h - C ABI of the IceCache hot path on MI355X (gfx950).
 *
 * What the calls compute follows the IceCache method pages:
 *   - papernotes.org, "IceCache: Memory-Efficient KV-cache Management for
 *     Long-Sequence LLMs", section "Overall framework": (1) index - at prefill
 *     (or when window tokens are offloaded) build one DCI tree per attention
 *     head that clusters tokens by key similarity, each node one physical
 *     page; (2) page selection - at decode every head picks its own top-k
 *     pages with an M-DCI nearest-neighbour search; (3) bulk loading + sparse
 *     attention over the picked pages.
 *   - aitangshan.cn IceCache article, section 3 (the DCI tree: key lift,
 *     random promotion, nearest parent one level up, same parent = same page,
 *     incremental insert without rebuild) and section 6 (TK/TQ transform, the
 *     union of pages over a GQA group).
 *
 * Model of the data. A "head" is one independent index: one (sequence,
 * layer, KV head). All heads of one index object share the parameters and
 * the token count. Keys, values and queries share one element type, fp32 or
 * bf16 (raw IEEE bfloat16 bits). Every device buffer is owned by the caller;
 * the library never allocates device memory. Every call that takes a
 * `stream` (a hipStream_t; NULL = the default stream) only enqueues work and
 * returns; results are ready when the stream reaches them. All argument and
 * capacity checks run on the host before anything is enqueued, so a call that
 * returns an error has changed nothing. Nothing throws across the ABI.
 * Calls on one index object must be issued from one host thread at a time
 * and must not overlap on the device (enqueue them on one stream).
 */
#ifndef ICE_H_
#define ICE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define ICE_OK            0
#define ICE_ERR_ARG      -1  /* null pointer, bad size, bad budget or beam      */
#define ICE_ERR_DTYPE    -2  /* unsupported element type / head dimension        */
#define ICE_ERR_STATE    -3  /* select / insert / attend before build            */
#define ICE_ERR_CAPACITY -4  /* tokens beyond `capacity`, workspace too small    */
#define ICE_ERR_HIP      -5  /* a HIP runtime call failed (message has details) */

/* ---- element types ----------------------------------------------------- */
#define ICE_F32  0
#define ICE_BF16 1

/* ---- limits ------------------------------------------------------------ */
#define ICE_PAGE_CAP   16   /* tokens per page (the article's section 2 example) */
#define ICE_MAX_LEVELS 4
#define ICE_MAX_GROUP  16   /* query heads per KV head                          */
#define ICE_MAX_BEAM   256  /* beam width and pages per query                    */
#define ICE_MAX_RESIDENT 4096 /* resident (sink + window) tokens per head         */

typedef struct ice_params {
  int32_t  n_heads;       /* H >= 1: independent indexes (sequence x layer x KV head)     */
  int32_t  group;         /* G in [1, ICE_MAX_GROUP]: query heads sharing one KV head      */
  int32_t  d;             /* head dimension: 64 or 128                                    */
  int32_t  dtype;         /* ICE_F32 or ICE_BF16, for K, V and Q                          */
  int32_t  page_cap;      /* must be ICE_PAGE_CAP                                         */
  int32_t  levels;        /* L in [1, ICE_MAX_LEVELS]: levels 0..L-1, bottom included      */
  int32_t  promote_log2;  /* promotion probability per level = 2^-promote_log2, in [1,16] */
  int32_t  capacity;      /* max tokens per head, build plus inserts, 1 .. 2^26          */
  uint32_t flags;         /* 0, ICE_HOST_POOL or ICE_SPLIT_RESORT                         */
  uint64_t seed;          /* seed of the promotion draws                                  */
  int32_t  resident;      /* resident tokens per head kept beside the index (sink and
                             recent window, see ice_set_resident), 0 .. ICE_MAX_RESIDENT;
                             0 with ICE_HOST_POOL                                          */
} ice_params;

/* Host-pool mode (the notes' overall framework, step 3, and the aitangshan.cn
 * article, sections 4 and 5: the KV cache is offloaded to CPU memory and the
 * selected pages are moved to the GPU in one bulk load per step). The
 * level-0 V pages live in a caller-allocated pinned host pool instead of the
 * device blob; keys, the index and the selection stay in device memory. Each
 * ice_attend / ice_decode first gathers the V pages of the union from the
 * pool into a staging area of the workspace (a GPU kernel reads them over the
 * host link) and attends from there. Results equal the device-pool mode's
 * bit for bit. */
#define ICE_HOST_POOL 1u

/* Re-sort split (the notes' key design 2 leaves open how an overflowing node
 * splits; this is the other reading, beside the default append split). When
 * an insert finds its level-0 owner's last page full, the new page is still
 * appended to the owner's chain, and then all the owner's members, the new
 * token included, are re-packed over the owner's pages in chain order as the
 * build packs them: the owner first, then ascending lifted squared distance
 * to the owner (fp64 from the stored rows), ties by token id. Page ids,
 * chains and counts are those of the append split; the tokens' pages and
 * slots, and their K and V rows, move. The virtual root (no promoted token)
 * and owners with more than ICE_RESPLIT_MAX members split by appending.
 * Needs the device V pool (ICE_ERR_ARG with ICE_HOST_POOL). */
#define ICE_SPLIT_RESORT 2u
#define ICE_RESPLIT_MAX 1024

typedef struct ice_index ice_index;   /* opaque host-side handle */

/* Device bytes of the index blob for these parameters. The sizes come from
 * the promotion draws of every position 0..capacity-1 of every head, so the
 * blob bounds every page table exactly; 0 on invalid parameters. */
size_t ice_index_bytes(const ice_params* p);

/* Device bytes of the workspace that ice_build, ice_insert, ice_select and
 * ice_attend need for queries up to `max_budget_tokens` (a multiple of
 * page_cap) per query head (in host-pool mode this includes the V staging
 * area, n_heads * group * max_budget_tokens / 16 pages). One workspace may be
 * shared by successive calls on one stream; it holds nothing between calls.
 * 0 on invalid arguments. */
size_t ice_workspace_bytes(const ice_params* p, int32_t max_budget_tokens);

/* Pinned host bytes of the V page pool in host-pool mode (0 without
 * ICE_HOST_POOL or on invalid parameters). */
size_t ice_host_pool_bytes(const ice_params* p);

/* Creates a host handle over a caller-allocated device blob of at least
 * ice_index_bytes(p) bytes (256-byte aligned). The blob stays owned by the
 * caller and must outlive the handle. */
int ice_create(const ice_params* p, void* index_dev, size_t index_bytes, ice_index** out);
void ice_destroy(ice_index* idx);

/* Host-pool mode: attaches the V page pool, at least ice_host_pool_bytes(p)
 * bytes of pinned host memory (hipHostMalloc, or a pinned torch tensor),
 * 256-byte aligned, that stays owned by the caller and must outlive the
 * handle. The device reads and writes it directly. Required before
 * ice_build; ICE_ERR_STATE without ICE_HOST_POOL, ICE_ERR_ARG if the memory
 * is not pinned host memory the device can reach. */
int ice_attach_host_pool(ice_index* idx, void* host_pool, size_t host_pool_bytes);

/* Index build at prefill (the framework's step 1; the article's section 3).
 * K, V: device, [H][n_tokens][d] with `head_stride` elements between heads
 * (>= n_tokens*d). For every head: lift keys to [k, sqrt(M^2-|k|^2)] with M^2
 * the head's largest squared key norm; draw every token's promotion level;
 * give every point of level l its nearest point of level l+1 as parent
 * (lifted Euclidean distance, ties to the lower token id); store the points
 * sharing a parent together, ordered by distance and cut into pages of 16;
 * copy K and V rows into the page pool. Replaces any earlier content.
 * 0 <= n_tokens <= capacity. ws: workspace of ice_workspace_bytes.
 * A build of 16 or more heads with 2 or more levels runs as a pipeline over
 * up to 4 ranges of heads on two streams: `stream` runs the ranges' level-0
 * parent searches and a second stream, made by the handle at its first such
 * build on the current device and destroyed with it, runs the other phases
 * of each range. Events order it after the work enqueued on `stream` before
 * the call and the work enqueued on `stream` after it after all of it, as a
 * one-stream call would be; the result is the one-stream build's, bit for
 * bit. Under stream capture, or on a device other than the one of the
 * handle's second stream, it runs on `stream` alone. Calls on one handle
 * come from one host thread at a time. */
int ice_build(ice_index* idx, const void* K, const void* V, int32_t n_tokens, int64_t head_stride,
              void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): ice_build
 * without a workspace argument. Its scratch is a fixed array of
 * ICE_NOALLOC_SCRATCH_BYTES in each device's global memory, part of the
 * loaded library and held until the process ends; the call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine). The device
 * is the current one; its array's address is looked up on the first call on
 * that device. ICE_ERR_CAPACITY (nothing enqueued) when the index's build
 * needs more scratch than that, i.e. ice_workspace_bytes' build part: enough
 * for one 32k-token layer of 8 KV heads (d = 128 bf16), not for all layers of
 * a model at once. Every call on one device shares that device's array, so
 * calls that overlap on one device (other streams, other indexes, other host
 * threads) race; enqueue them on one stream. The build leaves nothing in the
 * array that a later call relies on. It runs on `stream` alone (no second
 * stream). Otherwise as ice_build. */
#define ICE_NOALLOC_SCRATCH_BYTES 67108864  /* 64 MiB */
int ice_build_noalloc(ice_index* idx, const void* K, const void* V, int32_t n_tokens, int64_t head_stride,
                      void* stream);

/* ice_build, with the time of each build phase measured by events recorded
 * on `stream` between the phases' kernels; waits for `stream` to reach the
 * end of the build. phase_ms: host, ICE_BUILD_PHASES floats, in ms:
 *   ICE_PHASE_LIFT                    header reset, key norms, promotion
 *                                     levels, lift and level lists;
 *   ICE_PHASE_OPERAND + 4 l           candidate-parent operand of level l;
 *   ICE_PHASE_PARENT + 4 l            nearest-parent search of level l (the
 *                                     distance GEMM with its argmax);
 *   ICE_PHASE_PACK + 4 l              page pack of level l;
 *   ICE_PHASE_COPY + 4 l              page-pool copies of level l;
 *   ICE_PHASE_TOP                     top-list copy;
 * for l = 0 .. ICE_MAX_LEVELS - 2 (a phase with no kernel, such as the
 * parent search of a level that does not exist, reports the few
 * microseconds between two events).
 * It runs on `stream` alone (no pipeline), so the phases add up to the
 * one-stream build. Everything else is as in ice_build. */
#define ICE_BUILD_PHASES  14
#define ICE_PHASE_LIFT     0
#define ICE_PHASE_OPERAND  1
#define ICE_PHASE_PARENT   2
#define ICE_PHASE_PACK     3
#define ICE_PHASE_COPY     4
#define ICE_PHASE_TOP     13
int ice_build_timed(ice_index* idx, const void* K, const void* V, int32_t n_tokens, int64_t head_stride,
                    void* ws, size_t ws_bytes, void* stream, float* phase_ms);

/* ice_build with parents found by Prioritized DCI instead of the exact
 * search (the notes' key design 2: M-DCI sits on P-DCI; the article's
 * section 3 names it as the prior work; composite and simple indices as in
 * Li and Malik, ICML 2017). dirs: device fp32 [m*l][d+1] projection
 * directions over lifted keys [k, e], shared by every head and level; simple
 * index i of composite index j uses row j*l + i. Per child point and
 * composite index, the l simple indices are walked outward from the child's
 * key in their sorted order, always visiting the walker front with the
 * smallest |key - child key| (ties: simple index, then candidate); a
 * candidate is complete once all l have visited it; the walk ends after
 * `visits` visits (once it has a candidate) or `cands` complete candidates.
 * The complete candidates of all composite indices are ranked by lifted
 * inner product (ties to the lower token id). Keys are fp64 from the stored
 * rows and fp32 lift coordinate. 1 <= l <= ICE_PDCI_MAX_L, m >= 1,
 * m*l <= ICE_PDCI_MAX_KEYS, visits >= 1, cands >= 1. The workspace of
 * ice_workspace_bytes covers it. It runs on `stream` alone. Everything else
 * is as in ice_build. */
#define ICE_PDCI_MAX_KEYS 16
#define ICE_PDCI_MAX_L 4
int ice_build_pdci(ice_index* idx, const void* K, const void* V, int32_t n_tokens, int64_t head_stride,
                   const float* dirs, int32_t m, int32_t l, int32_t visits, int32_t cands, void* ws, size_t ws_bytes,
                   void* stream);

/* Build of heads h0 .. h0+n_heads-1 only, as ice_build does it for every
 * head (the aitangshan.cn article, section 4, and the notes' key design 4:
 * the index of one layer is built while the model works on the next). K, V:
 * device, the rows of those heads, [n_heads][n_tokens][d] at head_stride.
 * Every head of an index holds the same token count: once any head is built,
 * a build of fewer than all heads must pass that count (ICE_ERR_ARG
 * otherwise). Builds of disjoint head ranges may run at the same time on
 * different streams with one workspace, each head using its own part of it
 * (a range of 16 or more heads is pipelined as in ice_build; the handle's
 * one second stream then serves the ranges in turn).
 * Select, attend, decode and insert need every head built (ICE_ERR_STATE
 * before). A range rebuilt as a whole keeps its resident tokens and dense
 * flags; heads built for the first time start with neither. */
int ice_build_heads(ice_index* idx, const void* K, const void* V, int32_t n_tokens, int64_t head_stride,
                    int32_t h0, int32_t n_heads, void* ws, size_t ws_bytes, void* stream);

/* Index reuse across layers (the aitangshan.cn article, section 5: the
 * accelerated variant IceCache(reuse) shares the index between layers; the
 * notes' key design 4 stacks page reuse on the prefill pipeline). Heads h0 .. h0+n_heads-1 take the layout of the built heads
 * src_h0 .. src_h0+n_heads-1, head by head in order: levels, parents, which
 * tokens share a page and in what order, the top list. They place their own
 * K and V rows ([n_heads][n_tokens][d] at head_stride, device) into it and
 * lift their own keys (M and e). Their selection then scores their own keys
 * inside the shared structure. n_tokens must equal the source heads' count;
 * the ranges must not overlap. No parent search runs, so it costs copies
 * only. Later inserts into these heads follow their own promotion draws; an
 * insert that would give such a head more points at some level than its
 * tables were sized for (they are sized from each head's own draws over the
 * whole capacity) is refused with ICE_ERR_CAPACITY before anything is
 * enqueued. */
int ice_build_reuse(ice_index* idx, const void* K, const void* V, int32_t n_tokens, int64_t head_stride,
                    int32_t h0, int32_t n_heads, int32_t src_h0, void* ws, size_t ws_bytes, void* stream);

/* Incremental insert (the article's section 3: no rebuild; the notes' key
 * design 2: a node over the page size splits off a new page). k_new, v_new:
 * device, [H][n_new][d] contiguous, k_new 16-byte aligned (ICE_ERR_ARG
 * otherwise). Tokens are inserted one after another at
 * the next positions: each draws its level (capped at the build's top level),
 * takes the nearest point of the next level as parent, and is appended to
 * its owner's last page, or to a newly split page if that one is full.
 * Tokens already placed keep their page and slot, except under
 * ICE_SPLIT_RESORT (see there). ICE_ERR_CAPACITY if the count would exceed
 * capacity, or a head built by ice_build_reuse would outgrow its tables
 * (nothing is inserted). */
int ice_insert(ice_index* idx, const void* k_new, const void* v_new, int32_t n_new,
               void* ws, size_t ws_bytes, void* stream);

/* Page selection (the notes' key designs 2 and 3). Q: device [H][G][d].
 * Per query head: score the top level by q.k, keep the `beam` best; score the
 * children of the kept points one level down, keep `beam`; ...; at level 0
 * rank every page of the kept level-1 points by its best token score and keep
 * k = budget_tokens/16 pages (score descending, then page id ascending).
 *   sel   [H][G][k]   page ids in rank order, -1 padded (device)
 *   uni   [H][G*k]    union over the group, ascending, -1 padded (device)
 *   n_uni [H]         union sizes (device)
 *   trace [H][G][L][beam] nullable: kept point ids per cut, top level first
 *                     (cuts that do not exist are -1); for parity checks.
 * budget_tokens: positive multiple of 16, <= the workspace's max budget and
 * <= ICE_MAX_BEAM*16; beam in [1, ICE_MAX_BEAM]. */
int ice_select(const ice_index* idx, const void* Q, int32_t budget_tokens, int32_t beam,
               int32_t* sel, int32_t* uni, int32_t* n_uni, int32_t* trace,
               void* ws, size_t ws_bytes, void* stream);

/* Sparse attention over the selected pages (the notes' key design 1: the
 * weight of token j is s_j exp(q.k_j/sqrt d) normalised over the selected
 * tokens). For every (h, g): o = sum_j softmax_j(scale * q.k_j) v_j over the
 * valid tokens of pages uni[h][0..n_uni[h]). O: device [H][G][d] fp32;
 * lse: device [H][G] fp32 log-sum-exp of the scaled logits, nullable. A head
 * with no selected token gets o = 0, lse = -inf. uni_stride: ints between
 * heads in `uni` (>= the max n_uni), at most the workspace's budget times G
 * over 16. */
int ice_attend(const ice_index* idx, const void* Q, const int32_t* uni, const int32_t* n_uni,
               int32_t uni_stride, float scale, float* O, float* lse,
               void* ws, size_t ws_bytes, void* stream);

/* Resident tokens (the aitangshan.cn IceCache article, section 6: the first
 * "sink" tokens and the most recent window stay on the GPU, outside the
 * index; only the tokens in between are indexed and retrieved). K, V:
 * device, [H][n][d] at head_stride elements per head (>= n*d), the index's
 * dtype, 16-byte aligned; 0 <= n <= params.resident (ICE_ERR_ARG otherwise).
 * They are copied into per-head resident pages beside the page pool, and
 * every later ice_attend / ice_decode attends them together with the pages
 * it attends, in one softmax, until the next call replaces them (n = 0
 * clears them). The selection never sees them. A caller moving a token out
 * of the window inserts it (ice_insert) and passes the shorter window.
 * After ice_build (ICE_ERR_STATE before); later builds keep them. */
int ice_set_resident(ice_index* idx, const void* K, const void* V, int32_t n, int64_t head_stride, void* stream);

/* Dense heads (the notes' discussion of the method's limits: the first two
 * layers are left out of retrieval because their attention is not sparse).
 * dense: host, [H] bytes, nonzero = that head's attention covers every
 * indexed token (and its resident tokens) instead of the selected pages;
 * nullable = none. Selection still runs for such heads, and its output is
 * not used by their attention. ice_decode runs as separate select and attend
 * kernels while any head is dense. ICE_ERR_ARG with ICE_HOST_POOL. After
 * ice_build (ICE_ERR_STATE before); later builds keep them. Waits for
 * `stream`, then copies the flags synchronously. */
int ice_set_dense(ice_index* idx, const uint8_t* dense, void* stream);

/* One decode step of the hot path (the framework's steps 2 and 3 together):
 * ice_select (without trace) followed by ice_attend over its union, with
 * uni_stride = G * budget_tokens / 16. The outputs and argument rules are
 * those of the two calls; the results equal theirs up to the order of the
 * fp32 sums in the attention. For bf16 keys with beam and budget/16 at most
 * 64 it runs as one kernel per step (each head selects, then attends its own
 * union, with no pass through memory in between); otherwise it enqueues the
 * two calls' kernels. Either way two calls on the same index and queries
 * give the same bits: the one-kernel step hands fixed chunks of the union to
 * its waves as they become free and merges the chunks' partial sums in chunk
 * order. */
int ice_decode(const ice_index* idx, const void* Q, int32_t budget_tokens, int32_t beam,
               int32_t* sel, int32_t* uni, int32_t* n_uni, float scale, float* O, float* lse,
               void* ws, size_t ws_bytes, void* stream);

/* ---- inspection (synchronise the stream; for parity tests and stats) ---- */

/* Arrays of one head that ice_export copies to host memory. */
#define ICE_EXP_LEVEL      0   /* int8  [capacity]          level used by the index        */
#define ICE_EXP_LIFT       1   /* f32   [capacity]          extra lift coordinate e        */
#define ICE_EXP_PARENT     2   /* int32 [capacity] level `level`: parent token (-1 none)   */
#define ICE_EXP_PAGE_TOK   3   /* int32 [pages][16] level `level` page table, -1 = empty   */
#define ICE_EXP_PAGE_CNT   4   /* int32 [pages]                                            */
#define ICE_EXP_PAGE_NEXT  5   /* int32 [pages] next page of the same owner, -1 = last     */
#define ICE_EXP_PAGE_OWNER 6   /* int32 [pages] owner token, -1 = virtual root             */
#define ICE_EXP_OWNER_FIRST 7  /* int32 [capacity+1] first page per owner (+ root), -1     */
#define ICE_EXP_OWNER_TAIL 8   /* int32 [capacity+1] last page per owner (+ root), -1      */
#define ICE_EXP_TOP        9   /* int32 [top capacity] top-level points in order           */
#define ICE_EXP_PAGE_K     10  /* dtype [pages][16][d] page-pool keys (level 0) / copies   */
#define ICE_EXP_PAGE_V     11  /* dtype [pages][16][d] page-pool values (level 0 only; the
                                  device stores each 4-slot group dimension-major; in
                                  host-pool mode they are read from the host pool) */
#define ICE_EXP_HEADER     12  /* ice_head_stats                                           */
#define ICE_EXP_OWNER_RUN  13  /* int32 [capacity+1] pages of the owner's contiguous run   */
#define ICE_EXP_OWNER_COUNT 14 /* int32 [capacity+1] members of the owner                  */

typedef struct ice_head_stats {
  int32_t n_tokens;        /* tokens in the head                                  */
  int32_t top_level;       /* highest non-empty level at build (L_top)            */
  int32_t n_top;           /* points in the top list                              */
  int32_t n_pages[ICE_MAX_LEVELS]; /* pages per page table (level 0 = KV pages)    */
  int32_t clamps;          /* inserted keys longer than the build's M (lift = 0)   */
  int32_t splits;          /* KV pages split off by inserts (level-0 page table)   */
  int32_t near_ties;       /* parent choices whose two best lifted distances were
                              within 1e-4 relative, build and insert              */
  int32_t overflow;        /* 1 if a page table was full (ruled out by the sizes) */
  int32_t sync_timeouts;   /* selection-kernel barrier waits that hit their spin
                              limit (a bound that keeps kernels finite; 0 in
                              correct operation)                                 */
  int32_t n_resident;      /* resident tokens attended beside the pages          */
  int32_t dense;           /* nonzero: attention covers every indexed token      */
  double  M2;              /* largest squared key norm at build                   */
} ice_head_stats;

/* Bytes of one export array for this index (per head), 0 if not applicable. */
size_t ice_export_bytes(const ice_index* idx, int32_t what, int32_t level);
/* Copies array `what` of `head` (page tables: of `level`) into host memory
 * `dst` of at least ice_export_bytes bytes. Synchronises `stream` first. */
int ice_export(const ice_index* idx, int32_t head, int32_t what, int32_t level, void* dst,
               size_t dst_bytes, void* stream);

/* Number of tokens per head as tracked by the handle. */
int32_t ice_n_tokens(const ice_index* idx);

/* Message of the last error on this thread ("" if none). */
const char* ice_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* ICE_H_ */
