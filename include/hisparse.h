/* hisparse.h -- C ABI of a two-tier (host + GPU) KV cache for top-k sparse
 * attention decoding on AMD MI355X (gfx950).
 *
 * Sources (pages, cited by title and section):
 *   [P3] "HiSparse: Scaling Sparse-Attention Decoding with Hierarchical KV
 *        Cache Management" -- Abstract, AI Summary.
 *   [P2] "Hybrid HiSparse" (knowledge card) -- Timeline.
 *   [P1] "HiSparse" (knowledge card) -- Timeline.
 *
 * Model.  Every request keeps its full KV history in host memory and a small
 * fixed-size cache in GPU memory [P3 Abstract].  The library keeps one cache
 * per (request, layer) -- a "stream" -- made of C LRU slots and R resident
 * slots.  Each decode step hands it, per layer, the positions the sparse
 * indexer selected (whatever the indexer is [P3 Abstract]); the library
 * classifies each one as resident, hot (cached) or missing in one pass
 * [P2 Timeline], picks LRU victims, copies only the missing rows from host
 * memory [P1 Timeline; P3 Abstract] and emits the slot map that sparse MLA
 * attention reads.  Only placement changes, so attention over the slot map
 * equals attention over the full history [P3 Abstract].
 *
 * Readings taken where the pages are silent:
 *   - the LRU clock is a per-stream step counter, advanced once per resolve;
 *   - victims are the slots not referenced in this step, ordered by
 *     (last use ascending, slot ascending); the j-th miss in ascending
 *     selection index takes the j-th victim;
 *   - resident rows are the last R positions of the context, held in ring
 *     slot C + (p mod R), outside the LRU, tested before the cache lookup;
 *   - -1 in a selection is padding.
 *
 * Memory and ownership.  The caller owns the host history (pinned and
 * device-mapped, e.g. from hisparse_host_alloc), the device cache and the
 * device metadata buffer (sizes from hisparse_workspace_bytes; any device
 * allocator), and every sel / ctx_len / out_slot buffer.  The library owns
 * its handle, its events and a small per-layer prefetch buffer allocated in
 * hisparse_create.  Device layouts:
 *   cache:  [num_layers][num_requests][C + R][row_bytes] bytes; slot s of
 *           stream (b, l) starts at ((l*B + b)*(C+R) + s) * row_bytes.
 *   meta:   see hisparse_meta_layout.
 *
 * Errors.  Every function returns HISPARSE_OK (0) or a negative code;
 * hisparse_last_error() describes the most recent failure of the calling
 * thread.  Data errors found on the device (a selection outside [-1, ctx), a
 * context length outside [0, max_positions], a repeated position when
 * HISPARSE_DEBUG_VALIDATE is set) are reported through a sticky status word
 * (hisparse_get_status): that stream's state is left untouched and its
 * out_slot row is all -1.
 *
 * Asynchrony.  hisparse_resolve, hisparse_append_resolve, hisparse_prefetch,
 * hisparse_append, hisparse_load_window and hisparse_reset only enqueue work on the given
 * stream(s): they never synchronize, allocate or read device memory on the
 * host, so they can be captured into a HIP graph (prefetch forks and joins
 * by events, which capture as graph edges).  A handle is not thread-safe.
 */
#ifndef HISPARSE_H
#define HISPARSE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ------------------------------------------------------ */
#define HISPARSE_OK 0
#define HISPARSE_ERR_INVALID_ARG (-1) /* bad argument or configuration        */
#define HISPARSE_ERR_OOM (-2)         /* an allocation failed                 */
#define HISPARSE_ERR_HIP (-3)         /* a HIP runtime call failed            */
#define HISPARSE_ERR_STATE (-4)       /* call out of order (e.g. prefetch)    */
#define HISPARSE_ERR_UNSUPPORTED (-5) /* shape beyond the kernels' limits     */

/* ---- configuration flags (hisparse_config.flags) ----------------------- */
#define HISPARSE_NO_IO 0x1u /* metadata only: resolve never copies rows     */
#define HISPARSE_DEBUG_VALIDATE 0x2u /* also reject repeated positions      */
#define HISPARSE_SERIALIZE_PREFETCH 0x4u /* prefetch runs on the main stream */

/* ---- device status bits (hisparse_get_status) -------------------------- */
#define HISPARSE_STATUS_SEL_RANGE 0x1u /* a selection outside [-1, ctx)     */
#define HISPARSE_STATUS_SEL_DUP 0x2u   /* a repeated position (debug only)  */
#define HISPARSE_STATUS_CTX_RANGE 0x4u /* ctx_len outside [0, max_positions]*/
#define HISPARSE_STATUS_PREFETCH_MISMATCH 0x8u /* resolve's sel differs from
                                                  the prefetched one         */

/* ---- host-memory flags (hisparse_host_alloc) --------------------------- */
#define HISPARSE_HOST_COHERENT 0x0u    /* fine-grained, coherent (default)  */
#define HISPARSE_HOST_NONCOHERENT 0x1u /* coarse-grained, GPU may cache it  */

/* Shape of one cache instance.  All streams share it. */
typedef struct hisparse_config {
  int32_t num_requests;    /* B: request slots, 1..32768                     */
  int32_t num_layers;      /* layers, each with its own cache (>= 1)         */
  int64_t max_positions;   /* host rows per stream (tokens or pages), < 2^31 */
  int32_t row_bytes;       /* bytes per row, a positive multiple of 16       */
  int32_t cache_slots;     /* C: LRU slots per stream, top_k <= C <= 16384   */
  int32_t resident_window; /* R: resident ring slots per stream (>= 0)       */
  int32_t top_k;           /* k: selections per stream per call, 1..4096     */
  uint32_t flags;          /* HISPARSE_NO_IO | HISPARSE_DEBUG_VALIDATE | ... */
} hisparse_config;

/* Byte offsets inside the device metadata buffer.  Stream (b, l) owns the
 * block at stream_base + (l*B + b) * stream_stride; the other offsets are
 * relative to that block.  All arrays are int32 unless noted.
 *   status:     uint32 sticky status word of the handle (absolute offset)
 *   hdr:        int32[16]: [0] t (LRU clock), [1] status of the last call,
 *               [2..7] counters of the last call: n_pad, n_res, n_hit,
 *               n_miss, n_evict, bytes fetched; int64 running totals since
 *               the last reset: [8..9] misses, [10..11] evictions,
 *               [12..13] hits; [14..15] reserved
 *   pos2slot:   int32[max_positions]: LRU slot of position p, or -1
 *   slot2pos:   int32[C]: position held by LRU slot s, or -1
 *   last_use:   int32[C]: step at which slot s was last referenced
 *   lru_order:  int32[C]: LRU slots sorted by (last_use, slot)
 *   evict_log:  int32[2*k]: (slot, old position or -1) of the j-th miss of
 *               the last call
 *   miss_list:  int32[2*k]: (slot, position) rows fetched by the last call */
typedef struct hisparse_meta_layout {
  size_t total_bytes;
  size_t status;
  size_t stream_base;
  size_t stream_stride;
  size_t hdr;
  size_t pos2slot;
  size_t slot2pos;
  size_t last_use;
  size_t lru_order;
  size_t evict_log;
  size_t miss_list;
} hisparse_meta_layout;

/* Accumulated GPU time of the library's kernels while timing is enabled. */
typedef struct hisparse_timing {
  int64_t resolve_launches; /* resolve kernel launches timed               */
  int64_t fetch_launches;   /* fetch kernel launches timed                 */
  double resolve_ms;        /* summed event time of the resolve kernels    */
  double fetch_ms;          /* summed event time of the fetch kernels      */
} hisparse_timing;

typedef struct hisparse* hisparse_t;

/* Sizes of the caller-owned device buffers for `cfg`.  Host only; no GPU
 * needed.  [P3 Abstract: a small fixed-size GPU cache per request.]
 * cache_bytes = L*B*(C+R)*row_bytes; meta_bytes = hisparse_meta_layout's
 * total.  Either output pointer may be NULL.  Errors: INVALID_ARG. */
int hisparse_workspace_bytes(const hisparse_config* cfg, size_t* cache_bytes,
                             size_t* meta_bytes);

/* Offsets of every array in the metadata buffer (see above).  Host only. */
int hisparse_meta_layout_of(const hisparse_config* cfg, hisparse_meta_layout* out);

/* Allocate `bytes` of pinned, device-mapped host memory for a host history
 * (hipHostMalloc; HISPARSE_HOST_* flags) on a NUMA node.  [P3 Abstract: the
 * full history lives in host memory; every miss is read from it over the
 * host link, so it belongs on the node next to the GPU.]
 *   numa_node >= 0:        that node (the calling thread's memory policy is
 *                          bound to it for the allocation, then restored);
 *                          INVALID_ARG when the process may not use it;
 *   HISPARSE_NUMA_DEVICE:  the node closest to the current HIP device
 *                          (hipDeviceAttributeHostNumaId); when the device
 *                          reports none or the process may not use it, the
 *                          process's own policy applies;
 *   HISPARSE_NUMA_DEFAULT: the process's own policy.
 * hisparse_host_numa_node tells where the pages landed.  The caller frees
 * the memory with hisparse_host_free.  Errors: INVALID_ARG (bytes == 0, bad
 * flags, numa_node < -2 or >= 1024, node not usable), OOM, HIP. */
#define HISPARSE_NUMA_DEVICE (-1)
#define HISPARSE_NUMA_DEFAULT (-2)
int hisparse_host_alloc(size_t bytes, int numa_node, uint32_t flags, void** host_ptr);
int hisparse_host_free(void* host_ptr);

/* NUMA node of the host page holding `host_ptr` (get_mempolicy with
 * MPOL_F_NODE | MPOL_F_ADDR), e.g. to check where hisparse_host_alloc put a
 * history.  Pinned memory from the GPU driver is a device-file mapping the
 * kernel does not place-query: then *node is the host's only node when it
 * has one, else -1 (unknown).  Host only; no GPU needed.  Errors:
 * INVALID_ARG (NULL). */
int hisparse_host_numa_node(const void* host_ptr, int* node);

/* NUMA node closest to the current HIP device, or -1 when the device
 * reports none.  Errors: INVALID_ARG (NULL), HIP. */
int hisparse_device_numa_node(int* node);

/* Create a cache instance on the current HIP device.
 *   host_rows:   host pointers [num_layers * num_requests], entry l*B + b is
 *                the pinned host history of stream (b, l), max_positions *
 *                row_bytes bytes, caller-owned and alive until destroy;
 *   device_cache, device_meta: caller-owned device buffers of the sizes from
 *                hisparse_workspace_bytes (256-byte aligned).
 * Initializes the metadata (every slot empty, clocks 0) and synchronizes.
 * The resident slots are not loaded: call hisparse_load_window.
 * [P3 Abstract: full host history, fixed-size GPU cache per request.]
 * Errors: INVALID_ARG (bad shape, unpinned host memory, misaligned buffer),
 * UNSUPPORTED (C > 16384 or k > 4096), OOM, HIP. */
int hisparse_create(const hisparse_config* cfg, void* const* host_rows, void* device_cache,
                    void* device_meta, hisparse_t* out);

/* Release the handle's events and buffers after synchronizing its work.
 * Caller-owned memory is not touched.  NULL is accepted. */
int hisparse_destroy(hisparse_t h);

/* Resolve one layer's selections for every request, on `stream`.
 *   sel:      device int32 [B, k]; per row distinct positions in [0, ctx),
 *             -1 = padding;
 *   ctx_len:  device int32 [B]: context length (rows) of each request;
 *   layer:    0 <= layer < num_layers;
 *   out_slot: device int32 [B, k]: slot in [0, C+R) of stream (b, layer)
 *             holding sel[b, i] after the call, -1 for padding; must not
 *             overlap sel or ctx_len (INVALID_ARG).
 * One pass per stream does hit detection, LRU victim choice and the
 * metadata update; then (unless HISPARSE_NO_IO) the missing rows are copied
 * from the host history into their slots.  When `layer` was prefetched in
 * this step, the call only joins the prefetch and copies its slot map.
 * [P3 Abstract: per-layer resolution -- hit detection, LRU replacement,
 * host-to-device fetches -- inside the decode graph; P2 Timeline: resident,
 * hot and missing rows in a single pass, graph-capturable; P1 Timeline:
 * only the missing top-k rows are copied back.]
 * Errors: INVALID_ARG (NULL pointer, bad layer, overlapping buffers), HIP. */
int hisparse_resolve(hisparse_t h, hipStream_t stream, const int32_t* sel,
                     const int32_t* ctx_len, int32_t layer, int32_t* out_slot);

/* Resolve one layer for several query tokens per request at once (multi-
 * token prediction or speculative decoding), on `stream`.
 *   sel:      device int32 [B, queries, per_query]: each query's selections,
 *             -1 = padding; positions may repeat across and within queries;
 *   queries x per_query <= top_k;
 *   out_slot: device int32 [B, queries, per_query]: the slot holding each
 *             entry's position after the call, -1 for padding; must not
 *             overlap sel or ctx_len.
 * The queries of a step attend through the same cache, so the step resolves
 * the union of their selections once (one clock tick per stream): the union
 * is taken in first-occurrence order over the entries (query-major), every
 * missing position is fetched once, and every entry is served by its
 * position's slot.  The per-stream counters are those of the union padded
 * to queries x per_query entries (repeats count as padding).  A row with an
 * entry outside [-1, ctx) is rejected as by hisparse_resolve.
 * [P2 Timeline: multi-token prediction is listed among the features the
 * method works with; the union reading is this library's.]
 * Errors: INVALID_ARG (NULL pointer, bad layer, queries x per_query outside
 * [1, top_k]), STATE (the layer has a pending prefetch), UNSUPPORTED (the
 * deduplication table does not fit the device's LDS), HIP. */
int hisparse_resolve_multi(hisparse_t h, hipStream_t stream, const int32_t* sel,
                           int32_t queries, int32_t per_query, const int32_t* ctx_len,
                           int32_t layer, int32_t* out_slot);

/* Resolve `layer` early on `side_stream`, ordered after the work already
 * enqueued on `main_stream` (event fork), for models whose layers share one
 * selection.  The next hisparse_resolve of that layer on `main_stream` joins
 * it (event wait) and returns the same slot map; the state after prefetch +
 * resolve equals the state after the resolve alone.
 *   out_slot: NULL, or the buffer the joining resolve will pass, [B, k]: the
 *             prefetch writes the slot map there directly (on the side
 *             stream: no other work may read or write it until the join).
 * The resolve must pass the same selections.  When it passes the same sel
 * and out_slot pointers as the prefetch (and HISPARSE_DEBUG_VALIDATE is
 * off), the join is only an event wait: the selections' contents are taken
 * as unchanged.  Otherwise a join kernel copies the prefetched map into its
 * out_slot and compares the selections with the prefetched ones: a
 * difference sets HISPARSE_STATUS_PREFETCH_MISMATCH.
 * [P3 Abstract: exact layer-wise prefetching for models sharing selections
 * across layers; P3 AI Summary: per-layer prefetching hides part of the miss
 * penalty; P1 Timeline: not applicable to layers with independent
 * selections.]
 * Errors: INVALID_ARG (also out_slot overlapping sel or ctx_len), STATE (the
 * layer already has a pending prefetch), HIP. */
int hisparse_prefetch(hisparse_t h, hipStream_t main_stream, hipStream_t side_stream,
                      const int32_t* sel, const int32_t* ctx_len, int32_t layer,
                      int32_t* out_slot);

/* Copy the rows of positions [max(0, ctx-R), ctx) of every request from the
 * host history into their resident ring slots C + (p mod R) of `layer`
 * (layer = -1: every layer).  ctx_len: device int32 [B].  Used at admission.
 * [P2 Timeline: resident rows.]  Errors: INVALID_ARG, HIP. */
int hisparse_load_window(hisparse_t h, hipStream_t stream, int32_t layer,
                         const int32_t* ctx_len);

/* Append one new row per request to `layer`: rows is device memory
 * [B, row_bytes]; pos is device int32 [B], the new row's position (the old
 * context length; -1 skips that request).  The row is written to the host
 * history at `pos` and, when R > 0, to ring slot C + (pos mod R), which
 * drops position pos - R out of the resident window.  The next resolve must
 * pass ctx_len = pos + 1.  [P2 Timeline: requests keep decoding while their
 * context grows in host memory.]  Errors: INVALID_ARG, HIP. */
int hisparse_append(hisparse_t h, hipStream_t stream, int32_t layer, const void* rows,
                    const int32_t* pos);

/* hisparse_append followed by hisparse_resolve on the same layer, in one
 * launch: the decode step of a growing context, where each layer's new row
 * is appended and its selections resolved [P2 Timeline].  Arguments as for
 * the two calls (ctx_len = pos + 1 for every appending request); results
 * are identical to calling them in order on `stream`.  With a resident
 * window (R >= 1) the appended position is resident, so the resolution
 * neither looks it up nor fetches it and the row stores run inside the
 * resolve launch; without a window, or when `layer` has a pending prefetch,
 * the two calls are made as separate launches.  A pending prefetch has
 * resolved the layer already: with a window the append then runs before the
 * join; without a window the call is rejected (STATE), because that prefetch
 * may have fetched the appended position's host row before it was written --
 * append with hisparse_append before hisparse_prefetch instead.
 * Graph-capturable like hisparse_resolve.  Errors: INVALID_ARG, STATE (no
 * window and a pending prefetch on `layer`; nothing is launched), HIP. */
int hisparse_append_resolve(hisparse_t h, hipStream_t stream, int32_t layer, const void* rows,
                            const int32_t* pos, const int32_t* sel, const int32_t* ctx_len,
                            int32_t* out_slot);

/* hisparse_append followed by hisparse_resolve_multi on the same layer, in
 * one launch when a resident window holds the appended position (two in
 * order otherwise): the decode step of a growing context with several query
 * tokens per request.  Arguments as for the two calls.  Errors: as
 * hisparse_resolve_multi (checked before anything is launched), and
 * INVALID_ARG for rows or pos. */
int hisparse_append_resolve_multi(hisparse_t h, hipStream_t stream, int32_t layer,
                                  const void* rows, const int32_t* pos, const int32_t* sel,
                                  int32_t queries, int32_t per_query, const int32_t* ctx_len,
                                  int32_t* out_slot);

/* Return streams to the empty state (every slot free, clock 0).  layer and
 * request select one stream; -1 means all.  Used for admission and reuse of
 * a request slot.  Errors: INVALID_ARG, HIP. */
int hisparse_reset(hisparse_t h, hipStream_t stream, int32_t layer, int32_t request);

/* Read the sticky device status word (HISPARSE_STATUS_* bits); when `clear`
 * is non-zero, zero it afterwards.  Synchronizes the device: not capturable.
 * Errors: INVALID_ARG, HIP. */
int hisparse_get_status(hisparse_t h, uint32_t* status, int clear);

/* Enable (1) or disable (0) event timing of the resolve and fetch kernels of
 * eager (not captured) calls; enabling clears the totals. */
int hisparse_set_timing(hisparse_t h, int enable);

/* Synchronize and return the accumulated kernel times. */
int hisparse_get_timing(hisparse_t h, hisparse_timing* out);

/* Link probe: read `bytes` (a multiple of 16) of pinned host memory with a
 * zero-copy kernel of `workgroups` x 256 threads (16-byte loads) and write
 * them to device memory.  Measures the host-to-device read rate that the
 * miss fetch is bounded by.  Errors: INVALID_ARG, HIP. */
int hisparse_probe_host_read(hipStream_t stream, const void* host, void* device, size_t bytes,
                             int32_t workgroups);

/* ---- sparse MLA decode attention over the slot map ----------------------
 * The step the slot map exists for: attention of every request's query heads
 * over the rows its slot map points at, read from the HBM slot cache.  Only
 * placement changes, so the result equals attention over the same positions
 * of the full host history [P3 Abstract]; the method sits under sparse MLA
 * decoding [P2 Timeline; P1 Timeline].
 *
 * Rows are sparse-MLA latent rows: 576 bf16 = 512 latent values (keys and
 * values) + 64 rope values (keys only); a slot holds row_bytes / 1152 token
 * rows (16 for 16-token pages), all of which are attended.  For request b,
 * head h:  score_i = scale * q[b,h,:] . row_i[:576];  out[b,h,:] =
 * sum_i softmax(score)_i * row_i[:512];  lse[b,h] = log sum_i exp(score_i)
 * (-inf and out = 0 when every entry is padding).  fp32 accumulation; the
 * softmax weights enter the value product with ~24 significant bits.
 *
 * hisparse_mla_workspace_bytes: size of the caller-owned device workspace
 *   (per-split partial results) for num_heads, a multiple of 16.  Host only;
 *   the workspace needs no initialisation.
 * hisparse_sparse_mla_decode (async on `stream`, graph-capturable; two
 *   launches: the split attention, then the merge of the splits):
 *   q:        device bf16 [B, num_heads, 576], 16-byte aligned;
 *   out_slot: device int32 [B, k], as written by hisparse_resolve for `layer`;
 *   workspace: 256-byte aligned, hisparse_mla_workspace_bytes bytes;
 *   out:      device fp32 [B, num_heads, 512];  lse: device fp32 [B, num_heads].
 * Errors: INVALID_ARG (NULL, misaligned, bad layer or head count),
 * UNSUPPORTED (row_bytes not a multiple of 1152), HIP.  Launches sharing one
 * workspace must be ordered (same stream). */
int hisparse_mla_workspace_bytes(hisparse_t h, int32_t num_heads, size_t* bytes);
int hisparse_sparse_mla_decode(hisparse_t h, hipStream_t stream, int32_t layer, const void* q,
                               const int32_t* out_slot, int32_t num_heads, float scale,
                               void* workspace, float* out, float* lse);

/* The same attention for several query tokens per request (multi-token
 * prediction), over the slot map hisparse_resolve_multi wrote: query token
 * j of request b attends to the slots of its own entries, row (b, j) of the
 * [B, queries, per_query] map, read from request b's cache rows.
 *   q:        device bf16 [B, queries, num_heads, 576];
 *   out_slot: device int32 [B, queries, per_query];
 *   out:      device fp32 [B, queries, num_heads, 512];
 *   lse:      device fp32 [B, queries, num_heads].
 * queries x per_query <= top_k and B x queries <= 65535; the workspace size
 * comes from hisparse_mla_workspace_bytes_multi with the same queries,
 * per_query and num_heads.  With queries = 1 and per_query = top_k these are
 * hisparse_mla_workspace_bytes and hisparse_sparse_mla_decode.
 * [P2 Timeline: multi-token prediction among the features the method works
 * with.]  Errors: as hisparse_sparse_mla_decode, and INVALID_ARG for
 * queries or per_query out of range. */
int hisparse_mla_workspace_bytes_multi(hisparse_t h, int32_t queries, int32_t per_query,
                                       int32_t num_heads, size_t* bytes);
int hisparse_sparse_mla_decode_multi(hisparse_t h, hipStream_t stream, int32_t layer,
                                     int32_t queries, int32_t per_query, const void* q,
                                     const int32_t* out_slot, int32_t num_heads, float scale,
                                     void* workspace, float* out, float* lse);

/* ---- the attention for callers that cannot allocate ------------------------
 * For code that may not call hipMalloc or any allocating routine: work under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * hisparse_sparse_mla_decode_noalloc is hisparse_sparse_mla_decode without
 * the workspace argument: the per-split partials live in a fixed device array
 * of HISPARSE_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held
 * until the process ends (its address is looked up when a handle is created
 * on that GPU).  The caller still passes q, out_slot, out and lse.  A call
 * whose workspace (hisparse_mla_workspace_bytes) exceeds the array is
 * rejected with UNSUPPORTED before anything is launched; the array needs no
 * initialisation.  All calls on one GPU share its array: calls that overlap
 * in time on one GPU (streams not ordered with each other, several handles
 * included) race on it and must be ordered by the caller.  Errors: as
 * hisparse_sparse_mla_decode, and UNSUPPORTED for a workspace beyond the
 * array. */
#define HISPARSE_NOALLOC_SCRATCH_BYTES ((size_t)40 << 20)
int hisparse_sparse_mla_decode_noalloc(hisparse_t h, hipStream_t stream, int32_t layer,
                                       const void* q, const int32_t* out_slot, int32_t num_heads,
                                       float scale, float* out, float* lse);

/* ---- top-k selection over indexer scores ----------------------------------
 * The step before resolution: from one score per position (a token for
 * DSA-style per-layer selection, a 16-token page for Quest-style selection),
 * pick the positions the resolver is handed.  [P3 Abstract: decoding attends
 * to the top-k positions an indexer selects, and the hierarchical cache does
 * not depend on which indexer; P2 Timeline: token- and page-granular
 * selection.]  Readings (the pages give none): among positions [0, ctx) the
 * k largest scores are taken, equal scores going to the lower position, -0
 * equal to +0; the row is written in ascending position order (the pages
 * give a selection no order) and padded with -1 when ctx < k.  Scores must
 * not be NaN (a NaN is ordered above +inf).
 *
 * hisparse_topk_workspace_bytes: device workspace for rows of up to max_len
 *   positions: two 16 KiB histograms (top 12 and next 12 key bits) and a
 *   few counters per row, a position bitmap and room for max_len boundary
 *   candidates (8 bytes each) per row.  Host
 *   only.  The workspace must be zero-filled once before its first use;
 *   every call leaves the parts it needs zeroed again.
 * hisparse_topk (async on `stream`, graph-capturable: three launches, no
 *   memset; calls sharing a workspace must be ordered):
 *   scores:     device fp32, row b at scores + b * row_stride, 16-byte
 *               aligned, row_stride >= max_len and a multiple of 4;
 *   num_rows:   1..65535 (e.g. requests of one layer);
 *   max_len:    1..2^31 - 4097, the workspace's row capacity;
 *   ctx_len:    device int32 [num_rows]; clamped to [0, max_len];
 *   k:          1..4096;
 *   out_sel:    device int32 [num_rows, k]: ready to pass to
 *               hisparse_resolve as `sel` (with the same ctx_len).
 * Errors: INVALID_ARG (NULL, misaligned, sizes out of range), HIP. */
int hisparse_topk_workspace_bytes(int32_t num_rows, int64_t max_len, size_t* bytes);
int hisparse_topk(hipStream_t stream, const float* scores, int64_t row_stride, int32_t num_rows,
                  int64_t max_len, const int32_t* ctx_len, int32_t k, void* workspace,
                  int32_t* out_sel);

/* Text for a return code, and the last failure of the calling thread. */
const char* hisparse_strerror(int code);
const char* hisparse_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HISPARSE_H */
