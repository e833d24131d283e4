/*
 * oracle_timing.c -- timing harness for the CPU baseline: runs a whole
 * decode through the oracle's functions, with the requests split into
 * disjoint shares, one POSIX thread per share.
 *
 * TEST INFRASTRUCTURE ONLY: the benchmark's CPU-baseline leg loads it; the
 * product path never does.  It adds no arithmetic of the method: every step
 * calls the unchanged functions of hisparse_oracle.c (admission, the
 * forward's KV write, the swap-in per verify row, the skip layers' replay,
 * the eager backup) in the order the pages give for one decode step (SGLang
 * guide "HiSparse: Hierarchical Sparse Attention", "Decode Workflow" and
 * "Shared-index prefetch"; vLLM design note "HiSparse local KV offload
 * architecture", "Resident device pages" for the verify rows).  Requests are
 * independent of each other and the oracle keeps no global state, so the
 * shares run side by side and each runs every step of its own requests in
 * one C loop, with no per-step hand-off.
 */
#define _POSIX_C_SOURCE 200809L

#include "oracle_timing.h"

#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

#include "hisparse_oracle.h"

typedef struct {
    pthread_mutex_t m;
    pthread_cond_t c;
    int go;                      /* set once the barrier below is initialised */
    pthread_barrier_t bar;       /* every started share + the timing thread */
} gate_t;

typedef struct {
    const orc_decode* d;
    int32_t lo, hi;              /* requests [lo, hi) */
    gate_t* gate;
    int rc;
} share_t;

static double now_s(void)
{
    struct timespec ts;
    clock_gettime(CLOCK_MONOTONIC, &ts);
    return (double)ts.tv_sec + 1e-9 * (double)ts.tv_nsec;
}

static int admit_share(const orc_decode* d, int32_t lo, int32_t hi)
{
    for (int32_t r = lo; r < hi; ++r) {
        for (int32_t l = 0; l < d->layers; ++l) {
            const int32_t g = d->anchor_of[l];
            int rc;
            if (g == l) {
                rc = orc_admit_state(d->B, d->L0[r], d->lru[g] + (size_t)r * d->B, d->tok[g] + (size_t)r * d->B);
                if (rc) return rc;
            }
            rc = orc_admit_fill(d->B, d->L0[r], d->rb, d->host[l] + (size_t)r * d->max_seq * d->rb,
                                d->hot[l] + (size_t)r * (d->B + 1) * d->rb);
            if (rc) return rc;
        }
    }
    return ORC_OK;
}

/* Steps [k0, k1) of requests [lo, hi): per layer, the forward's KV write,
 * then on an anchor one swap-in per verify row (each with its own plan row)
 * or on a skip layer the replay of each of its anchor's plan rows, then the
 * eager backup. */
static int run_steps(const orc_decode* d, int32_t lo, int32_t hi, int32_t k0, int32_t k1,
                     int32_t* req_idx, int32_t* out, int32_t* pos, int32_t* slot, int32_t* count)
{
    const int32_t nb = hi - lo, K = d->K, R = d->R, S = d->spec;
    const int64_t rb = d->rb;
    const uint8_t* res = d->resident ? d->resident + lo : NULL;
    for (int32_t k = k0; k < k1; ++k) {
        const int32_t* L = d->seq_lens + (size_t)k * R + lo;
        for (int32_t l = 0; l < d->layers; ++l) {
            const int32_t g = d->anchor_of[l];
            const uint8_t* nk = d->new_kv + ((size_t)k * d->layers + l) * R * rb;
            for (int32_t b = 0; b < nb; ++b) {
                const int32_t r = lo + b;
                if (res && res[b]) continue;
                int rc = orc_store_newest(d->B, L[b], rb, nk + (size_t)r * rb,
                                          d->hot[l] + (size_t)r * (d->B + 1) * rb);
                if (rc) return rc;
            }
            for (int32_t s = 0; s < S; ++s) {
                /* plan row s of anchor g, for this share: [nb][K] pairs, [nb] counts */
                const size_t pr = (size_t)g * S + s;
                int32_t* pp = pos + pr * nb * K;
                int32_t* ps = slot + pr * nb * K;
                int32_t* pc = count + pr * nb;
                int rc;
                if (g == l) {
                    const int32_t* tk = d->topk + ((((size_t)k * d->layers + l) * S + s) * R + lo) * K;
                    if (d->page_size > 0)
                        rc = orc_swap_in_paged(R, d->B, K, rb, d->max_seq, nb, req_idx, tk, L,
                                               d->block_table ? d->block_table + (size_t)lo * d->max_pages : NULL,
                                               d->max_pages, d->page_size, d->hot_row_base, out, d->lru[l],
                                               d->tok[l], d->host[l], d->hot[l], pp, ps, pc);
                    else
                        rc = orc_swap_in(R, d->B, K, rb, d->max_seq, nb, req_idx, tk, L, res, out, d->lru[l],
                                         d->tok[l], d->host[l], d->hot[l], pp, ps, pc);
                } else {
                    rc = orc_replay(R, d->B, K, rb, d->max_seq, nb, req_idx, pp, ps, pc, d->host[l], d->hot[l]);
                }
                if (rc) return rc;
            }
            int rc = orc_backup(R, d->B, rb, d->max_seq, nb, req_idx, L, res, d->hot[l], d->host[l]);
            if (rc) return rc;
        }
    }
    return ORC_OK;
}

static void* share_main(void* arg)
{
    share_t* sh = (share_t*)arg;
    const orc_decode* d = sh->d;
    const int32_t nb = sh->hi - sh->lo;
    const size_t plan_ints = (size_t)d->layers * d->spec * nb * d->K;
    int32_t* req_idx = malloc(sizeof(int32_t) * (size_t)(nb > 0 ? nb : 1));
    int32_t* out = malloc(sizeof(int32_t) * ((size_t)nb * d->K + 1));
    int32_t* pos = malloc(sizeof(int32_t) * (plan_ints + 1));
    int32_t* slot = malloc(sizeof(int32_t) * (plan_ints + 1));
    int32_t* count = malloc(sizeof(int32_t) * ((size_t)d->layers * d->spec * nb + 1));
    pthread_mutex_lock(&sh->gate->m);
    while (!sh->gate->go) pthread_cond_wait(&sh->gate->c, &sh->gate->m);
    pthread_mutex_unlock(&sh->gate->m);
    sh->rc = (req_idx && out && pos && slot && count) ? ORC_OK : ORC_ENOMEM;
    if (sh->rc == ORC_OK) {
        for (int32_t b = 0; b < nb; ++b) req_idx[b] = sh->lo + b;
        sh->rc = admit_share(d, sh->lo, sh->hi);
    }
    if (sh->rc == ORC_OK)
        sh->rc = run_steps(d, sh->lo, sh->hi, 0, d->first_timed, req_idx, out, pos, slot, count);
    pthread_barrier_wait(&sh->gate->bar);                 /* timed region starts */
    if (sh->rc == ORC_OK)
        sh->rc = run_steps(d, sh->lo, sh->hi, d->first_timed, d->n_steps, req_idx, out, pos, slot, count);
    pthread_barrier_wait(&sh->gate->bar);                 /* timed region ends */
    free(req_idx);
    free(out);
    free(pos);
    free(slot);
    free(count);
    return NULL;
}

int orc_time_decode(const orc_decode* d, int32_t threads, double* seconds)
{
    if (!d || !seconds || threads < 1 || d->layers < 1 || d->R < 1 || d->spec < 1 || d->n_steps < 0 ||
        d->first_timed < 0 || d->first_timed > d->n_steps || !d->anchor_of || !d->host || !d->hot || !d->lru ||
        !d->tok || !d->L0 || !d->topk || !d->new_kv || !d->seq_lens)
        return ORC_EINVAL;
    if (threads > d->R) threads = d->R;
    share_t* sh = calloc((size_t)threads, sizeof(share_t));
    pthread_t* th = calloc((size_t)threads, sizeof(pthread_t));
    gate_t gate;
    gate.go = 0;
    if (!sh || !th || pthread_mutex_init(&gate.m, NULL) != 0) {
        free(sh);
        free(th);
        return ORC_ENOMEM;
    }
    pthread_cond_init(&gate.c, NULL);
    /* Threads wait at the gate until the barrier is sized for the shares
     * that did start; a share that could not start leaves its requests
     * unrun and the call reports ORC_ENOMEM. */
    int32_t started = 0;
    for (int32_t i = 0; i < threads; ++i) {
        sh[started].d = d;
        sh[started].lo = (int32_t)((int64_t)d->R * i / threads);
        sh[started].hi = (int32_t)((int64_t)d->R * (i + 1) / threads);
        sh[started].gate = &gate;
        if (pthread_create(&th[started], NULL, share_main, &sh[started]) == 0) ++started;
    }
    int rc = started == threads ? ORC_OK : ORC_ENOMEM;
    pthread_barrier_init(&gate.bar, NULL, (unsigned)started + 1);
    pthread_mutex_lock(&gate.m);
    gate.go = 1;
    pthread_cond_broadcast(&gate.c);
    pthread_mutex_unlock(&gate.m);
    pthread_barrier_wait(&gate.bar);
    const double t0 = now_s();
    pthread_barrier_wait(&gate.bar);
    const double t1 = now_s();
    for (int32_t i = 0; i < started; ++i) {
        pthread_join(th[i], NULL);
        if (rc == ORC_OK && sh[i].rc != ORC_OK) rc = sh[i].rc;
    }
    pthread_barrier_destroy(&gate.bar);
    pthread_cond_destroy(&gate.c);
    pthread_mutex_destroy(&gate.m);
    free(sh);
    free(th);
    *seconds = t1 - t0;
    return rc;
}
