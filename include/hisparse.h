/*
 * hisparse.h -- C ABI of the HiSparse decode-step swap-in resolver for
 * AMD Instinct MI355X (gfx950).
 *
 * The method (sources):
 *   [SGL]  SGLang guide "HiSparse: Hierarchical Sparse Attention":
 *          "Decode Workflow" (fast path, hit detection -> LRU reorder -> miss
 *          copy host to device, eager backup), "HiSparse Config Parameters"
 *          (top_k, device_buffer_size), "Shared-index prefetch" (the anchor's
 *          miss plan replayed by a copy-only kernel on a side stream).
 *   [vLLM] vLLM design note "HiSparse local KV offload architecture":
 *          "Resident device pages" (one fused resolver: resident page, then
 *          hot row, then pinned host memory; resident hits exit first; the
 *          graph-stable request mapping; speculative verify rows),
 *          "Hot lookup and LRU", "Performance invariants" (no device readback,
 *          no extra kernel launch, graph-capturable).
 *
 * Terms and layouts (all sizes in elements unless stated):
 *   K   top_k              B   device_buffer_size (token slots per request)
 *   R   max_requests       rb  row_bytes (one token's KV row, multiple of 16)
 *   host pool of a layer   [R][max_seq_len][rb] bytes, pinned host memory that
 *                          the GPU can address (see hisparse_host_alloc)
 *   hot buffer of a layer  [R][B+1][rb] bytes, device memory.  Rows 0..B-1 are
 *                          the LRU-managed slots; row B holds the newest token
 *                          while the sequence is longer than B.
 *   batch row b            serves request r = req_idx[b] (r = b if req_idx is
 *                          NULL): the graph-stable mapping taken from the
 *                          caller's attention metadata.
 *   seq_lens[b]  L         tokens with KV, the newest (position L-1) included.
 *   top-k entries          positions in [0, L), distinct, or -1 (padding).
 *
 * Output slot ids (out_slots[b][i]):
 *   resident request       the position itself (the caller's resident block
 *                          table maps it; resident requests touch no state);
 *   L <= B (fast path)     the position itself (slot = position);
 *   otherwise              a row of hot[r]: the slot holding that position, or
 *                          B for the newest position L-1; -1 for padding.
 *
 * Every pointer argument of the hot calls (store_newest, swap_in,
 * store_swap_in, store_swap_in_backup, swap_in_paged, replay_plan, backup,
 * spill, import, spill_dma, import_dma) is device memory unless stated; all of them are
 * asynchronous on the given stream, allocate nothing, never read device data
 * back to the host, and may be captured in a HIP graph.  Ownership: the caller
 * owns host pools, hot buffers, inputs, outputs and plan buffers; the library
 * owns only the per-anchor-layer LRU state ([R][B] int32 lru and slot map)
 * and one device error word.  Calls that use one anchor layer's state
 * (swap_in, store_swap_in, store_swap_in_backup, swap_in_paged, admit,
 * get/set_state) must be ordered by the caller (one stream, or events), and
 * so must a call that writes a layer's host pool (backup,
 * store_swap_in_backup, spill, import) and a later one that may read the
 * rows it wrote; calls on different anchor layers, and replays of different
 * skip layers, may run concurrently.  A context belongs to the device that
 * was current at hisparse_init: every later call on it must be made with that
 * device current (else HISPARSE_EINVAL; the library never switches devices).
 *
 * Errors: a call returns 0, or a negative code: HISPARSE_EINVAL (bad argument
 * seen on the host), HISPARSE_ENOMEM, or HISPARSE_EHIP(e) = -(1000 + e) for a
 * HIP runtime error e.  Host-side checks never read device data.  Broken
 * device-side preconditions never fault; each sets a bit in the device error
 * word (hisparse_get_error).  In the swap-in calls (a top-k entry out of
 * range or repeated, L beyond the host pool, a request index out of range,
 * corrupt state, a bad block-table entry) the affected batch row resolves to
 * all -1 with a plan count of 0 and leaves state and buffers untouched; the
 * per-request fast path and resident tier address no memory with top-k
 * entries and do not check them.  Admission, replay, backup, spill and
 * import skip the offending entry, row, pair or transfer and carry on with
 * the rest; the runtime-copy forms of spill and import, whose transfer list
 * is on the host, refuse a list with a bad transfer before issuing anything
 * (HISPARSE_EINVAL).
 */
#ifndef HISPARSE_H
#define HISPARSE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HISPARSE_OK 0
#define HISPARSE_EINVAL (-22)
#define HISPARSE_ENOMEM (-12)
#define HISPARSE_EBUSY (-16)    /* hisparse_init_static: the device's scratch is in use */
#define HISPARSE_ENOSPC (-28)   /* hisparse_init_static: state larger than the scratch array */
#define HISPARSE_EHIP(e) (-(1000 + (int)(e)))

/* Device error word bits (hisparse_get_error). */
#define HISPARSE_DERR_TOPK_RANGE 0x1u  /* entry < -1 or >= L */
#define HISPARSE_DERR_TOPK_DUP   0x2u  /* repeated position in a top-k row */
#define HISPARSE_DERR_SEQ_LEN    0x4u  /* L < 1, or L > max_seq_len where the host pool is addressed */
#define HISPARSE_DERR_REQ_IDX    0x8u  /* req_idx[b] outside [0, R) */
#define HISPARSE_DERR_STATE      0x10u /* corrupt LRU state, as far as a swap-in can see it: an lru
                                          entry outside [0, B), a slot-map position outside
                                          [-1, max_seq_len), two slots holding one position the row
                                          asks for, or repeated lru entries that leave fewer non-hit
                                          slots than misses.  The library never produces such state;
                                          only hisparse_set_state can bring it in, unchecked. */
#define HISPARSE_DERR_PLAN       0x20u /* replay: count > K, or a (pos, slot) pair out of range */
#define HISPARSE_DERR_PAGE       0x40u /* paged: block-table entry < -1, or a physical row beyond INT32_MAX;
                                          spill / import: a transfer coordinate out of range */

/* Per-request counters (hisparse_set_stats), one row of HISPARSE_STAT_COUNT
 * uint64 per request. */
#define HISPARSE_STAT_ENTRIES  0   /* valid top-k entries resolved (not -1)              */
#define HISPARSE_STAT_RESIDENT 1   /* resolved in tier 0: resident request or page      */
#define HISPARSE_STAT_FAST     2   /* resolved by the L <= B fast path (slot = position) */
#define HISPARSE_STAT_NEWEST   3   /* the newest token's own row                          */
#define HISPARSE_STAT_HIT      4   /* held in a hot slot                                  */
#define HISPARSE_STAT_MISS     5   /* copied from the host pool (the plan count)          */
#define HISPARSE_STAT_COUNT    6

/* hisparse_host_alloc flags */
#define HISPARSE_HOST_DEFAULT     0u   /* HIP's default pinned, mapped allocation */
#define HISPARSE_HOST_COHERENT    1u   /* fine-grained: GPU accesses bypass its caches */
#define HISPARSE_HOST_NONCOHERENT 2u   /* coarse-grained: GPU may cache; coherent at kernel boundaries */

typedef struct hisparse_ctx hisparse_ctx;

typedef struct {
    int32_t top_k;               /* K, 1 <= K <= B, K <= 4096                       */
    int32_t device_buffer_size;  /* B, 1 <= B <= 16384 (token slots per request)    */
    int32_t num_layers;          /* layers served by this context, <= 256            */
    int32_t max_requests;        /* R                                               */
    int32_t max_seq_len;         /* host rows per request                           */
    int32_t row_bytes;           /* rb, > 0, multiple of 16                          */
    void* const* host_pool;      /* [num_layers] host pointers, see the layout above;
                                    each must lie in pinned, GPU-mapped host memory */
    void* const* hot_buffer;     /* [num_layers] device pointers, [R][B+1][rb]       */
    const int32_t* anchor_of;    /* [num_layers] host array: the layer whose top-k and
                                    LRU state this layer shares (== itself for an
                                    anchor; anchor_of[anchor_of[l]] == anchor_of[l]).
                                    Skip layers own no LRU state.                    */
    int32_t block_size;          /* swap-in workgroup size: 0 = default (1024), else a
                                    multiple of 64 in [128, 1024]                     */
    int32_t replay_grid;         /* workgroups of the replay kernel: 0 = default     */
} hisparse_config;

/* One plan row (device): for batch row b, pairs (host position pos[b][m],
 * device slot slot[b][m]) for m < count[b], in ascending top-k index.  Entries
 * at m >= count[b] are left as they were.  Layout pos/slot [nb][K], count [nb]. */
typedef struct {
    int32_t* pos;
    int32_t* slot;
    int32_t* count;
} hisparse_plan;

/* Create a context: validates the configuration on the host, allocates the
 * LRU state of every anchor layer ([R][B] lru + [R][B] slot map, int32) and
 * the error word on the current device.  Besides the limits in
 * hisparse_config, R * (B + 1) must not exceed INT32_MAX (hot-buffer rows are
 * 32-bit indices), else HISPARSE_EINVAL.  State starts as if every request
 * had been admitted with a prompt longer than B.  [vLLM] "Main classes"
 * (per-cache runtime owning host/hot views, GPU LRU and the fused resolve). */
int hisparse_init(const hisparse_config* cfg, hisparse_ctx** out);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops that must not call hipMalloc, harnesses that forbid
 * it): hisparse_init with no allocation at all.  The library-owned device
 * memory (every anchor layer's [R][B] lru and slot map, the error word) is
 * carved from one static array of the library, hisparse_static_scratch_bytes()
 * = 32 MiB, which each device the library runs on holds until the process
 * ends; the context object is a static slot of that device.  The state needs
 * 256 bytes plus 2 * ceil256(R * B * 4) bytes per anchor layer; a
 * configuration that does not fit returns HISPARSE_ENOSPC.  One such context per device at a
 * time: while one is live (until hisparse_destroy), another call on that
 * device returns HISPARSE_EBUSY.  The array keeps the previous context's
 * contents, so this call first waits for all work on the device (a destroyed
 * context's last launches may still be running), then writes every byte the
 * new context uses (state as after hisparse_init, error word 0) on the null
 * stream, and waits for it.
 * Like hisparse_init it is a set-up call, made before any capture: it
 * launches on the null stream and waits.  Checks, limits and error codes are
 * otherwise those of hisparse_init, and every other call works on the
 * context exactly as on one from hisparse_init; calls on it follow the same
 * ordering rules (calls that overlap on one anchor layer's state race). */
int hisparse_init_static(const hisparse_config* cfg, hisparse_ctx** out);
size_t hisparse_static_scratch_bytes(void);

/* Free the library-owned state.  Caller-owned memory is untouched.
 * Not defined by the pages (library infrastructure). */
void hisparse_destroy(hisparse_ctx* ctx);

/* A request enters decode with host rows [0, seq_len0) valid (the prefill's
 * KV).  For each i < n, request r = req_ids[i], L0 = seq_len0[i] (device
 * arrays): the anchor layer's state is reset (lru = 0..B-1; slot map =
 * identity if L0 <= B, else empty), and when L0 <= B the rows [0, L0) of
 * every layer sharing this anchor are copied from the host pool into the hot
 * buffer at slot = position.  An entry with r outside [0, R), L0 < 0 or
 * L0 > max_seq_len is skipped (state and rows untouched) and sets
 * HISPARSE_DERR_REQ_IDX or HISPARSE_DERR_SEQ_LEN.  [SGL] "Decode Workflow"
 * (fast path: every KV row already in the buffer). */
int hisparse_admit(hisparse_ctx* ctx, int32_t anchor_layer, const int32_t* req_ids,
                   const int32_t* seq_len0, int32_t n, hipStream_t stream);

/* The forward's KV write: new_rows[b] (device, [nb][rb]) goes to the newest
 * token's row of hot[layer][r]: row L-1 when L <= B, else row B.  Resident
 * batch rows are skipped.  [SGL] "Decode Workflow" (forward decode, then
 * eager backup of that token). */
int hisparse_store_newest(hisparse_ctx* ctx, int32_t layer, const void* new_rows,
                          const int32_t* seq_lens, const uint8_t* resident_mask,
                          const int32_t* req_idx, int32_t nb, hipStream_t stream);

/* The fused resolver, one kernel launch.  For every batch row b (topk_idx
 * [nb][K], seq_lens [nb], resident_mask [nb] or NULL, req_idx [nb] or NULL):
 *   resident           -> out = topk, nothing else;           [vLLM] resident tier
 *   L <= B             -> out = topk (slot = position);        [SGL] fast path
 *   else, per entry i in ascending index:
 *     -1 -> -1;  L-1 -> B (newest row);
 *     held in a slot s (hit) -> s, the row does not move;      [SGL] hit detection
 *     otherwise (miss)  -> taken later;
 *   LRU reorder: slots not hit keep their order, hit slots keep their prior
 *   order behind them;                                         [SGL] LRU reorder
 *   the m-th miss (ascending i) takes the m-th least recent non-hit slot v,
 *   the slot map records it, the pinned host row is copied into hot[r][v]
 *   over the host link, and (pos, v) goes to plan_row; loaded slots become
 *   the most recent, in miss order.                            [vLLM] "Hot lookup and LRU"
 * plan_row.count[b] = number of misses (0 for resident / fast-path rows).
 * Uses the anchor layer's state, host pool and hot buffer.  Speculative
 * verify steps call this once per step on the same state with their own
 * plan row, consuming each result before the next call.  [vLLM] "Resident
 * device pages" (verify rows). */
int hisparse_swap_in(hisparse_ctx* ctx, int32_t anchor_layer,
                     const int32_t* topk_idx, const int32_t* seq_lens,
                     const uint8_t* resident_mask, const int32_t* req_idx, int32_t nb,
                     int32_t* out_slots, hisparse_plan plan_row, hipStream_t stream);

/* hisparse_store_newest followed by hisparse_swap_in on the anchor layer,
 * in one launch: new_rows [nb][rb] (device) is the forward's KV row of each
 * batch row, written to the newest token's row (L-1 when L <= B, else B;
 * resident rows skipped) by the resolver's own workgroup.  The resolver
 * never reads that row and never evicts it, so results are exactly those of
 * the two calls in sequence, without the second launch ([vLLM]
 * "Performance invariants": the abstraction adds no kernel launch). */
int hisparse_store_swap_in(hisparse_ctx* ctx, int32_t anchor_layer, const void* new_rows,
                           const int32_t* topk_idx, const int32_t* seq_lens,
                           const uint8_t* resident_mask, const int32_t* req_idx, int32_t nb,
                           int32_t* out_slots, hisparse_plan plan_row, hipStream_t stream);

/* hisparse_store_newest, hisparse_swap_in and hisparse_backup on the anchor
 * layer, in one launch: as hisparse_store_swap_in, and each new row also goes
 * straight to host[anchor][r][L-1] (resident rows skipped; a row with
 * L > max_seq_len is not backed up and sets HISPARSE_DERR_SEQ_LEN, as
 * hisparse_backup does).  That is the byte the backup would copy from the
 * newest row, and no swap-in of this call reads host position L-1 (it
 * resolves to the newest row), so results are exactly those of the three
 * calls in sequence.  The host write leaves over the link's device-to-host
 * direction while the misses arrive over the other.  Use it for the first
 * verify row of an anchor layer (later verify rows: hisparse_swap_in); skip
 * layers still call hisparse_backup after their replay.  [SGL] "Decode
 * Workflow" (forward, swap-in, eager backup); [vLLM] "Performance
 * invariants" (no extra launch). */
int hisparse_store_swap_in_backup(hisparse_ctx* ctx, int32_t anchor_layer, const void* new_rows,
                                  const int32_t* topk_idx, const int32_t* seq_lens,
                                  const uint8_t* resident_mask, const int32_t* req_idx, int32_t nb,
                                  int32_t* out_slots, hisparse_plan plan_row, hipStream_t stream);

/* The same fused resolver with per-page residency ([vLLM] "Resident device
 * pages": resident pages are checked first, then hot rows, then pinned host
 * memory; non-resident pages are host-backed holes).  block_table [nb]
 * [max_pages] (device) holds, for page p of batch row b (positions
 * [p*page_size, (p+1)*page_size)), the physical page in the caller's resident
 * cache, or -1 for a host-backed page; pages at or beyond max_pages are
 * host-backed (max_pages may be 0, block_table then NULL).  Output ids are
 * rows of one view chosen by the caller, as in a packed resident + hot
 * allocation ([vLLM] "Performance invariants"):
 *   resident position t      block_table[b][t / page_size] * page_size + t % page_size
 *   hot slot s (0..B, B = newest)   hot_row_base + r * (B + 1) + s
 *   padding                  -1
 * Resident positions never enter hit detection, the LRU, the plan or the
 * copy; the newest token resolves in tier 0 when its page is resident.  With
 * L <= B every non-resident position resolves to hot_row_base + r*(B+1) + t.
 * There is no resident_mask: a fully resident request has every page in the
 * table.  Host checks: page_size >= 1, max_pages >= 0, hot_row_base >= 0 and
 * hot_row_base + R*(B+1) <= INT32_MAX (else HISPARSE_EINVAL).  A block-table
 * entry below -1, or a physical row beyond INT32_MAX, fails the batch row
 * (HISPARSE_DERR_PAGE), like every other device-side precondition. */
int hisparse_swap_in_paged(hisparse_ctx* ctx, int32_t anchor_layer,
                           const int32_t* topk_idx, const int32_t* seq_lens,
                           const int32_t* block_table, int32_t max_pages, int32_t page_size,
                           int32_t hot_row_base, const int32_t* req_idx, int32_t nb,
                           int32_t* out_rows, hisparse_plan plan_row, hipStream_t stream);

/* hisparse_store_newest, hisparse_swap_in_paged and hisparse_backup on the
 * anchor layer in one launch, as hisparse_store_swap_in_backup is for
 * hisparse_swap_in: each new row goes to the newest token's hot row (L-1
 * when L <= B, else B) and to host[anchor][r][L-1] (not for L > max_seq_len,
 * which sets HISPARSE_DERR_SEQ_LEN).  A resident copy of the newest token,
 * when its page is resident, stays the caller's write to its resident cache,
 * as with the separate calls.  Host checks as hisparse_swap_in_paged, and
 * new_rows must be 16-byte aligned.  [SGL] "Decode Workflow"; [vLLM]
 * "Resident device pages", "Performance invariants". */
int hisparse_store_swap_in_paged_backup(hisparse_ctx* ctx, int32_t anchor_layer, const void* new_rows,
                                        const int32_t* topk_idx, const int32_t* seq_lens,
                                        const int32_t* block_table, int32_t max_pages, int32_t page_size,
                                        int32_t hot_row_base, const int32_t* req_idx, int32_t nb,
                                        int32_t* out_rows, hisparse_plan plan_row, hipStream_t stream);

/* Copy-only replay of an anchor's plan row on a skip layer: for each batch
 * row b and m < count[b], hot[skip][r][slot] <- host[skip][r][pos].  Runs on
 * a small fixed grid (replay_grid workgroups) so it can overlap other work on
 * a side stream; the caller orders it after the anchor's swap-in (event) and
 * before the skip layer's attention.  The grid splits the plan's rows evenly,
 * whatever the per-row counts.  A batch row with a count outside [0, K] or a
 * request index outside [0, R) is skipped, and so is a single (pos, slot)
 * pair outside the pool or the buffer; each sets HISPARSE_DERR_PLAN or
 * HISPARSE_DERR_REQ_IDX.  [SGL] "Shared-index prefetch". */
int hisparse_replay_plan(hisparse_ctx* ctx, int32_t skip_layer, hisparse_plan plan_row,
                         const int32_t* req_idx, int32_t nb, hipStream_t side_stream);

/* Eager backup: for every non-resident batch row, host[layer][r][L-1] <-
 * the newest token's row of hot[layer][r] (row L-1 when L <= B, else B).
 * Must run after the forward wrote that row and before a later swap-in can
 * ask for position L-1 from the host pool.  [SGL] "Decode Workflow"
 * (eager backup). */
int hisparse_backup(hisparse_ctx* ctx, int32_t layer, const int32_t* seq_lens,
                    const uint8_t* resident_mask, const int32_t* req_idx, int32_t nb,
                    hipStream_t stream);

/* Spill ([vLLM] "Spill transaction"): before a resident block is reused,
 * its contents are copied to the request's host page.  resident_cache
 * (device) holds resident_pages pages of page_size rows of rb bytes;
 * transfers [n][4] (device) = (resident page, request, host page, -1), the
 * physical copy coordinates only.  Host page hp of request r is rows
 * [hp*page_size, (hp+1)*page_size) of its host pool, cut at max_seq_len.
 * "Enqueued" is this call's return (stream order protects the resident page
 * from later work on the stream); "completed" is an event the caller
 * records after it on the same stream, after which the host page may be
 * published and the table entry replaced by -1.  A transfer with a
 * coordinate out of range is skipped and sets HISPARSE_DERR_PAGE. */
int hisparse_spill(hisparse_ctx* ctx, int32_t layer, const void* resident_cache, int32_t resident_pages,
                   int32_t page_size, const int32_t* transfers, int32_t n, hipStream_t stream);

/* Host import ([vLLM] "P/D import target"): pages arrive in a bounded
 * device staging pool (staging_pages pages) and are copied into registered
 * host memory; a page needed right away is mirrored into a resident page in
 * the same pass.  transfers [n][4] (device) = (staging page, request, host
 * page, resident page or -1).  resident_cache may be NULL when
 * resident_pages is 0.  Out-of-range transfers are skipped
 * (HISPARSE_DERR_PAGE). */
int hisparse_import(hisparse_ctx* ctx, int32_t layer, const void* staging, int32_t staging_pages,
                    int32_t page_size, void* resident_cache, int32_t resident_pages,
                    const int32_t* transfers, int32_t n, hipStream_t stream);

/* Runtime-copy forms of hisparse_spill and hisparse_import: the same page
 * transfers, with the same results, handed to the HIP runtime as
 * asynchronous copies instead of a kernel of this library, for transfers
 * that run beside other work ([HiCache] gathers pages with the GPU copy
 * engine rather than SM kernels; [vLLM] "Spill transaction": the worker
 * enqueues the GPU-to-host copy from its own list of physical copy
 * coordinates).  Which engine carries each copy (an SDMA engine, or the
 * runtime's own blit kernel) is the runtime's choice.  Here `transfers` is
 * HOST memory, [n][4] as above, read during the call.  Consecutive transfers
 * that are contiguous on every side (same request, next host page, next
 * source page, next mirror page or none, previous page not cut at
 * max_seq_len) merge into one copy; each merged run is one hipMemcpyAsync
 * device-to-host on `stream` (plus one device-to-device copy into the
 * mirror).  Every transfer is checked before anything is issued: one with a
 * coordinate out of range makes the call return HISPARSE_EINVAL with nothing
 * enqueued.  On a HIP error the runs before the failing one stay enqueued.
 * The caller keeps the host pool reachable by the runtime's copies (memory
 * from hisparse_host_alloc is). */
int hisparse_spill_dma(hisparse_ctx* ctx, int32_t layer, const void* resident_cache, int32_t resident_pages,
                       int32_t page_size, const int32_t* transfers, int32_t n, hipStream_t stream);
int hisparse_import_dma(hisparse_ctx* ctx, int32_t layer, const void* staging, int32_t staging_pages,
                        int32_t page_size, void* resident_cache, int32_t resident_pages,
                        const int32_t* transfers, int32_t n, hipStream_t stream);

/* Copy an anchor layer's state out of / into the library ([R][B] int32 each,
 * device pointers).  For tests and checkpointing; asynchronous on stream.
 * set_state does not check what it copies in: each lru row must be a
 * permutation of 0..B-1 and each slot map hold distinct positions or -1, as
 * get_state returns them.  A swap-in flags the corruptions it can see
 * (HISPARSE_DERR_STATE) and fails that row; others (say, an lru row that
 * repeats a slot no entry hits) give wrong slot ids but never an access out
 * of bounds.  Not defined by the pages (library infrastructure). */
int hisparse_get_state(hisparse_ctx* ctx, int32_t anchor_layer, int32_t* lru,
                       int32_t* slot_tok, hipStream_t stream);
int hisparse_set_state(hisparse_ctx* ctx, int32_t anchor_layer, const int32_t* lru,
                       const int32_t* slot_tok, hipStream_t stream);

/* Count what the resolver serves, per request, without any readback on the
 * hot path (hit rates are what the [HiCache] page reports for its tiers).
 * stats: device memory, [R][HISPARSE_STAT_COUNT] uint64, 8-byte aligned,
 * caller-owned and valid while set; NULL stops counting.  Every later launch
 * of a swap-in call (all forms) adds each batch row's counts to row req_idx[b]
 * with device atomics: its valid entries, split into resident, fast path,
 * newest row, hits and misses (these five sum to the entries).  A batch row
 * that fails its device-side checks adds nothing.  The library never reads or
 * clears the buffer: the caller zeroes it and reads it when it likes, ordered
 * after the launches it wants counted.  Host-only (stores the pointer); a
 * launch captured in a HIP graph keeps the pointer set at capture.  Not
 * defined by the pages (library infrastructure). */
int hisparse_set_stats(hisparse_ctx* ctx, uint64_t* stats);

/* Read (and optionally clear) the device error word.  Synchronizes the
 * stream: a diagnostic, never part of a decode step.  Not defined by the
 * pages (library infrastructure). */
int hisparse_get_error(hisparse_ctx* ctx, uint32_t* flags, int clear, hipStream_t stream);

/* Pinned, GPU-mapped host memory for host pools (flags: HISPARSE_HOST_*).
 * The pages have misses copied straight from registered pinned host memory
 * and give the pinned pool's lifetime to the worker ([vLLM] "Performance
 * invariants", "Ownership"); this allocator itself is library
 * infrastructure, not defined by the pages. */
int hisparse_host_alloc(size_t bytes, uint32_t flags, void** out);
int hisparse_host_free(void* p);

/* Bytes of LDS one swap-in workgroup uses for this configuration (0 for a
 * non-positive argument).  Not defined by the pages (library
 * infrastructure). */
size_t hisparse_swap_in_lds_bytes(int32_t top_k, int32_t device_buffer_size);

/* Static text for a return code; never NULL.  Version of this ABI.  Not
 * defined by the pages (library infrastructure). */
const char* hisparse_strerror(int code);
int hisparse_version(void);

#ifdef __cplusplus
}
#endif
#endif /* HISPARSE_H */
