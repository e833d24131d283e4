/*
 * oracle_timing.h -- timing harness for the CPU baseline (TEST
 * INFRASTRUCTURE ONLY; the product path never loads it).  It times a whole
 * decode run through the unchanged oracle functions of hisparse_oracle.h,
 * with the requests split into disjoint shares, one thread per share.
 */
#ifndef ORACLE_TIMING_H
#define ORACLE_TIMING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One decode run: every array is plain host memory, owned by the caller. */
typedef struct {
    int32_t layers, R, B, K, max_seq, spec;
    int64_t rb;
    const int32_t* anchor_of;       /* [layers]; anchor_of[l] <= l, anchors are their own */
    uint8_t* const* host;           /* [layers] -> [R][max_seq][rb] */
    uint8_t* const* hot;            /* [layers] -> [R][B+1][rb] */
    int32_t* const* lru;            /* [layers] -> [R][B] for anchors (unused for skip layers) */
    int32_t* const* tok;            /* [layers] -> [R][B] for anchors */
    const int32_t* L0;              /* [R] host rows valid at admission */
    const uint8_t* resident;        /* [R] or NULL (per-request residency) */
    const int32_t* block_table;     /* [R][max_pages] or NULL (per-page residency) */
    int32_t max_pages, page_size;   /* page_size > 0 selects the per-page resolver */
    int64_t hot_row_base;
    int32_t n_steps, first_timed;   /* steps [0, n_steps); [first_timed, n_steps) are timed */
    const int32_t* topk;            /* [n_steps][layers][spec][R][K]; read for anchor layers only */
    const uint8_t* new_kv;          /* [n_steps][layers][R][rb] */
    const int32_t* seq_lens;        /* [n_steps][R] */
} orc_decode;

/* Admit every request, run steps [0, first_timed) untimed, then time steps
 * [first_timed, n_steps) across `threads` shares of the requests (at most
 * R).  *seconds = wall time from the moment every share is ready to the
 * moment the last one finishes.  Returns 0 or the first oracle error. */
int orc_time_decode(const orc_decode* d, int32_t threads, double* seconds);

#ifdef __cplusplus
}
#endif
#endif
