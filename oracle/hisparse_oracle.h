/*
 * hisparse_oracle.h -- plain, slow CPU oracle of the HiSparse decode-step
 * swap-in resolver.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
 * its Python binding) may include, link, load or call this code; only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg do.  It shares
 * no code, header, table or helper with the HIP path.
 *
 * Sources (the method as stated on the pages; see hisparse_oracle.c for the
 * passage each function follows):
 *   [vLLM]  "HiSparse local KV offload architecture" (vLLM design note):
 *           sections "Resident device pages", "Hot lookup and LRU",
 *           "Performance invariants".
 *   [SGL]   "HiSparse: Hierarchical Sparse Attention" (SGLang guide):
 *           sections "Decode Workflow", "Shared-index prefetch".
 *
 * Every array is plain host memory.  Layouts:
 *   lru, tok        [R][B]            int32, per anchor layer
 *   host pool       [R][max_seq][rb]  bytes, one per layer
 *   hot buffer      [R][B+1][rb]      bytes, one per layer (row B = newest token)
 *   topk, out       [nb][K]           int32
 *   plan pos/slot   [nb][K], count [nb]  int32
 *
 * Return codes: 0 on success, ORC_EINVAL for a bad argument, ORC_EPRECOND when
 * the inputs break a precondition of the method (duplicate or out-of-range
 * top-k entry, sequence longer than the host pool, corrupt state).
 */
#ifndef HISPARSE_ORACLE_H
#define HISPARSE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_OK 0
#define ORC_EINVAL (-22)
#define ORC_ENOMEM (-12)
#define ORC_EPRECOND (-2001)

/* Row that holds the newest token's KV for a request of length L. */
int32_t orc_newest_row(int32_t B, int32_t L);

/* Request enters decode with host rows [0, L0) valid. */
int orc_admit_state(int32_t B, int32_t L0, int32_t* lru, int32_t* tok);
int orc_admit_fill(int32_t B, int32_t L0, int64_t rb,
                   const uint8_t* host_req, uint8_t* hot_req);

/* Forward writes the newest token's KV row into the hot buffer. */
int orc_store_newest(int32_t B, int32_t L, int64_t rb,
                     const uint8_t* new_row, uint8_t* hot_req);

/* Resolve one request's top-k row (all tiers), with miss copies. */
int orc_swap_in_row(int32_t B, int32_t K, int64_t rb, int32_t max_seq,
                    int32_t L, int32_t resident,
                    const int32_t* topk, int32_t* out,
                    int32_t* lru, int32_t* tok,
                    const uint8_t* host_req, uint8_t* hot_req,
                    int32_t* plan_pos, int32_t* plan_slot, int32_t* plan_count);

/* Batched form: batch row b serves request req_idx[b] (identity if NULL). */
int orc_swap_in(int32_t R, int32_t B, int32_t K, int64_t rb, int32_t max_seq,
                int32_t nb, const int32_t* req_idx,
                const int32_t* topk, const int32_t* seq_lens,
                const uint8_t* resident_mask, int32_t* out,
                int32_t* lru, int32_t* tok,
                const uint8_t* host, uint8_t* hot,
                int32_t* plan_pos, int32_t* plan_slot, int32_t* plan_count);

/* Per-page residency: block_row[p] = physical page of page p (-1 = host
 * backed); outputs are physical rows in the caller's view (resident rows
 * block_row[t/P]*P + t%P, hot rows hot_base + slot). */
int orc_swap_in_row_paged(int32_t B, int32_t K, int64_t rb, int32_t max_seq,
                          int32_t L, const int32_t* block_row, int32_t max_pages,
                          int32_t page_size, int64_t hot_base,
                          const int32_t* topk, int32_t* out,
                          int32_t* lru, int32_t* tok,
                          const uint8_t* host_req, uint8_t* hot_req,
                          int32_t* plan_pos, int32_t* plan_slot, int32_t* plan_count);

/* Batched form; request r's hot rows start at hot_row_base + r*(B+1). */
int orc_swap_in_paged(int32_t R, int32_t B, int32_t K, int64_t rb, int32_t max_seq,
                      int32_t nb, const int32_t* req_idx,
                      const int32_t* topk, const int32_t* seq_lens,
                      const int32_t* block_table, int32_t max_pages, int32_t page_size,
                      int64_t hot_row_base, int32_t* out,
                      int32_t* lru, int32_t* tok,
                      const uint8_t* host, uint8_t* hot,
                      int32_t* plan_pos, int32_t* plan_slot, int32_t* plan_count);

/* Skip layer: repeat the anchor's recorded misses on another layer's pool. */
int orc_replay(int32_t R, int32_t B, int32_t K, int64_t rb, int32_t max_seq,
               int32_t nb, const int32_t* req_idx,
               const int32_t* plan_pos, const int32_t* plan_slot,
               const int32_t* plan_count,
               const uint8_t* host, uint8_t* hot);

/* Eager backup of the newest token's row to the host pool. */
int orc_backup(int32_t R, int32_t B, int64_t rb, int32_t max_seq,
               int32_t nb, const int32_t* req_idx,
               const int32_t* seq_lens, const uint8_t* resident_mask,
               const uint8_t* hot, uint8_t* host);

/* Page transfers: spill (resident page -> host page) and host import
 * (staging page -> host page, optionally mirrored into a resident page).
 * transfers [n][4] = (source page, request, host page, mirror page or -1). */
int orc_page_copy(int32_t R, int32_t max_seq, int64_t rb, int32_t page_size,
                  const uint8_t* src, int32_t src_pages,
                  uint8_t* host, uint8_t* mirror, int32_t mirror_pages,
                  int32_t n, const int32_t* transfers);

#ifdef __cplusplus
}
#endif
#endif
