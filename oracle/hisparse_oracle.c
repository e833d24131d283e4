/*
 * hisparse_oracle.c -- plain, slow CPU oracle of the HiSparse decode-step
 * swap-in resolver.
 *
 * TEST INFRASTRUCTURE ONLY: used by the test suite, the smoke check and the
 * benchmark's CPU-baseline leg; never by the product path.  It shares no code
 * with the HIP library.
 *
 * What is computed, and where the pages state it:
 *   - SGLang guide "HiSparse: Hierarchical Sparse Attention", section
 *     "Decode Workflow": each step selects top-k positions, then a swap-in
 *     either takes the short-sequence fast path (sequence length not above
 *     the device buffer size: every KV row is already in the buffer, so the
 *     slot is the position) or runs hit detection, an LRU reorder and miss
 *     handling (host to device copy); after attention the previous token's KV
 *     is copied back to the host (eager backup).
 *   - vLLM design note "HiSparse local KV offload architecture", sections
 *     "Resident device pages" and "Hot lookup and LRU": resident pages are
 *     checked first and exit before any hot lookup or host copy; then hot
 *     rows (hit -> existing row, LRU updated); else an LRU victim is chosen
 *     and the pinned host row is copied into it.
 *   - SGLang guide, section "Shared-index prefetch": the anchor layer's
 *     swap-in records which host slot goes to which device slot; skip layers
 *     replay that record with a copy-only pass.
 *   - vLLM design note, "Resident device pages" (speculative decoding): each
 *     verify step is resolved and consumed in order on shared hot state and
 *     gets its own plan row (the caller passes a separate plan row per step).
 *
 * Points the pages leave open, and the reading taken here:
 *   - Victims come from the least-recently-used end of the LRU list, in order,
 *     and misses take them in ascending top-k array index.
 *   - The LRU reorder is a stable partition: slots not hit keep their order,
 *     hit slots keep their prior relative order and move behind them; the
 *     slots just loaded become the most recent, in miss order:
 *         new_lru = N[M:] ++ H ++ N[:M]
 *     (N = non-hit slots in LRU order, H = hit slots in LRU order, M misses).
 *   - The newest token (position L-1, when L exceeds the buffer size) lives
 *     in one extra row B of the request's hot buffer, outside the LRU; the
 *     forward writes it there and the eager backup copies it to the host.
 *   - Admission: lru = 0..B-1; tok = identity when the prompt fits the
 *     buffer (its rows sit at slot = position), else all empty (-1).
 *   - The fast path and the resident tier change no state, record no plan
 *     entry and copy nothing.
 *   - A top-k entry of -1 is padding and resolves to -1.
 *
 * No floating point anywhere: indices are int32, payload rows opaque bytes.
 */
#include "hisparse_oracle.h"

#include <stdlib.h>
#include <string.h>
#include <stdint.h>

int32_t orc_newest_row(int32_t B, int32_t L)
{
    /* Fast path: the newest token sits at its own position; otherwise it
     * sits in the extra row B. */
    if (L <= B)
        return L - 1;
    return B;
}

int orc_admit_state(int32_t B, int32_t L0, int32_t* lru, int32_t* tok)
{
    if (B <= 0 || L0 < 0 || !lru || !tok)
        return ORC_EINVAL;
    for (int32_t s = 0; s < B; ++s) {
        lru[s] = s;
        tok[s] = (L0 <= B) ? s : -1;
    }
    return ORC_OK;
}

int orc_admit_fill(int32_t B, int32_t L0, int64_t rb,
                   const uint8_t* host_req, uint8_t* hot_req)
{
    if (B <= 0 || L0 < 0 || rb <= 0 || !host_req || !hot_req)
        return ORC_EINVAL;
    if (L0 > B)
        return ORC_OK; /* long prompt: stays in the host pool only */
    for (int32_t p = 0; p < L0; ++p)
        memcpy(hot_req + (int64_t)p * rb, host_req + (int64_t)p * rb, (size_t)rb);
    return ORC_OK;
}

int orc_store_newest(int32_t B, int32_t L, int64_t rb,
                     const uint8_t* new_row, uint8_t* hot_req)
{
    if (B <= 0 || L < 1 || rb <= 0 || !new_row || !hot_req)
        return ORC_EINVAL;
    int32_t row = orc_newest_row(B, L);
    memcpy(hot_req + (int64_t)row * rb, new_row, (size_t)rb);
    return ORC_OK;
}

/* Preconditions on the top-k row: every entry is -1 or a distinct position
 * in [0, L).  Returns ORC_OK or ORC_EPRECOND. */
static int check_topk(int32_t K, int32_t L, const int32_t* topk)
{
    uint8_t* seen = (uint8_t*)calloc((size_t)L + 1, 1);
    if (!seen)
        return ORC_ENOMEM;
    int rc = ORC_OK;
    for (int32_t i = 0; i < K; ++i) {
        int32_t t = topk[i];
        if (t == -1)
            continue;
        if (t < -1 || t >= L || seen[t]) {
            rc = ORC_EPRECOND;
            break;
        }
        seen[t] = 1;
    }
    free(seen);
    return rc;
}

/* Preconditions on the state: lru is a permutation of 0..B-1 and every
 * entry of tok is -1 or a distinct position below max_seq. */
static int check_state(int32_t B, int32_t max_seq,
                       const int32_t* lru, const int32_t* tok)
{
    uint8_t* seen_slot = (uint8_t*)calloc((size_t)B, 1);
    uint8_t* seen_tok = (uint8_t*)calloc((size_t)max_seq, 1);
    if (!seen_slot || !seen_tok) {
        free(seen_slot); free(seen_tok);
        return ORC_ENOMEM;
    }
    int rc = ORC_OK;
    for (int32_t j = 0; j < B; ++j) {
        int32_t s = lru[j];
        if (s < 0 || s >= B || seen_slot[s]) {
            rc = ORC_EPRECOND;
            break;
        }
        seen_slot[s] = 1;
    }
    for (int32_t s = 0; s < B && rc == ORC_OK; ++s) {
        int32_t t = tok[s];
        if (t == -1)
            continue;
        if (t < -1 || t >= max_seq || seen_tok[t]) {
            rc = ORC_EPRECOND;
            break;
        }
        seen_tok[t] = 1;
    }
    free(seen_slot); free(seen_tok);
    return rc;
}

int orc_swap_in_row(int32_t B, int32_t K, int64_t rb, int32_t max_seq,
                    int32_t L, int32_t resident,
                    const int32_t* topk, int32_t* out,
                    int32_t* lru, int32_t* tok,
                    const uint8_t* host_req, uint8_t* hot_req,
                    int32_t* plan_pos, int32_t* plan_slot, int32_t* plan_count)
{
    if (B <= 0 || K <= 0 || K > B || rb <= 0 || !topk || !out || !plan_count)
        return ORC_EINVAL;
    *plan_count = 0;

    /* Tier 0: a resident request resolves to its own positions and touches
     * nothing else (vLLM design note, "Resident device pages"). */
    if (resident) {
        for (int32_t i = 0; i < K; ++i)
            out[i] = topk[i];
        return ORC_OK;
    }
    if (L < 1 || L > max_seq)
        return ORC_EPRECOND;
    int rc = check_topk(K, L, topk);
    if (rc != ORC_OK)
        return rc;

    /* Short-sequence fast path: slot = position (SGLang guide, "Decode
     * Workflow"). */
    if (L <= B) {
        for (int32_t i = 0; i < K; ++i)
            out[i] = topk[i];
        return ORC_OK;
    }

    if (!lru || !tok || !host_req || !hot_req || !plan_pos || !plan_slot)
        return ORC_EINVAL;
    rc = check_state(B, max_seq, lru, tok);
    if (rc != ORC_OK)
        return rc;

    /* Token -> slot+1 lookup for "is position t in the hot buffer, and where"
     * (0 = absent).  Only positions below L can be asked for. */
    int32_t* where = (int32_t*)calloc((size_t)L, sizeof(int32_t));
    uint8_t* is_hit = (uint8_t*)calloc((size_t)B, 1);
    int32_t* misses = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
    int32_t* N = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
    int32_t* H = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
    if (!where || !is_hit || !misses || !N || !H) {
        free(where); free(is_hit); free(misses); free(N); free(H);
        return ORC_ENOMEM;
    }
    for (int32_t s = 0; s < B; ++s)
        if (tok[s] >= 0 && tok[s] < L)
            where[tok[s]] = s + 1;

    /* Hit detection, in ascending top-k index. */
    int32_t M = 0;
    for (int32_t i = 0; i < K; ++i) {
        int32_t t = topk[i];
        if (t < 0) {
            out[i] = -1;                    /* padding */
        } else if (t == L - 1) {
            out[i] = B;                     /* newest token's own row */
        } else if (where[t] != 0) {
            int32_t s = where[t] - 1;       /* hit: the row stays where it is */
            out[i] = s;
            is_hit[s] = 1;
        } else {
            misses[M++] = i;                /* miss, handled below */
        }
    }

    /* LRU reorder: split the list into non-hit and hit slots, both stable. */
    int32_t nN = 0, nH = 0;
    for (int32_t j = 0; j < B; ++j) {
        int32_t s = lru[j];
        if (is_hit[s])
            H[nH++] = s;
        else
            N[nN++] = s;
    }

    /* Misses, in ascending top-k index, take victims from the LRU end in
     * order; the pinned host row is copied into the victim slot, and the
     * pair (host position, device slot) goes into the plan row. */
    for (int32_t m = 0; m < M; ++m) {
        int32_t i = misses[m];
        int32_t t = topk[i];
        int32_t v = N[m];
        tok[v] = t;
        out[i] = v;
        memcpy(hot_req + (int64_t)v * rb, host_req + (int64_t)t * rb, (size_t)rb);
        plan_pos[m] = t;
        plan_slot[m] = v;
    }
    *plan_count = M;

    /* New recency order, least recent first. */
    int32_t j = 0;
    for (int32_t k = M; k < nN; ++k)
        lru[j++] = N[k];
    for (int32_t k = 0; k < nH; ++k)
        lru[j++] = H[k];
    for (int32_t k = 0; k < M; ++k)
        lru[j++] = N[k];

    free(where); free(is_hit); free(misses); free(N); free(H);
    return ORC_OK;
}

int orc_swap_in(int32_t R, int32_t B, int32_t K, int64_t rb, int32_t max_seq,
                int32_t nb, const int32_t* req_idx,
                const int32_t* topk, const int32_t* seq_lens,
                const uint8_t* resident_mask, int32_t* out,
                int32_t* lru, int32_t* tok,
                const uint8_t* host, uint8_t* hot,
                int32_t* plan_pos, int32_t* plan_slot, int32_t* plan_count)
{
    if (R <= 0 || nb < 0 || nb > R)
        return ORC_EINVAL;
    for (int32_t b = 0; b < nb; ++b) {
        int32_t r = req_idx ? req_idx[b] : b;
        if (r < 0 || r >= R)
            return ORC_EINVAL;
        int rc = orc_swap_in_row(
            B, K, rb, max_seq, seq_lens[b], resident_mask ? resident_mask[b] : 0,
            topk + (int64_t)b * K, out + (int64_t)b * K,
            lru + (int64_t)r * B, tok + (int64_t)r * B,
            host + (int64_t)r * max_seq * rb, hot + (int64_t)r * (B + 1) * rb,
            plan_pos + (int64_t)b * K, plan_slot + (int64_t)b * K, plan_count + b);
        if (rc != ORC_OK)
            return rc;
    }
    return ORC_OK;
}

/* Per-page residency (vLLM design note, "Resident device pages" and "Hot
 * lookup and LRU": a resident page is checked first and resolves to its
 * resident physical row, before any hot lookup or host copy; pages that are
 * not resident are host-backed holes served by the hot buffer).
 *
 * block_row[p] is the physical page holding positions [p*P, (p+1)*P) of this
 * request, or -1 for a host-backed page; pages at or beyond max_pages are
 * host-backed.  Output ids live in one row space chosen by the caller:
 *   resident position t  ->  block_row[t / P] * P + t % P
 *   hot row s (0..B)     ->  hot_base + s
 *   padding              ->  -1
 * The resident entries are taken out of the row (replaced by padding, which
 * the hot tiers ignore) and the rest is resolved exactly as orc_swap_in_row
 * does, so resident positions never touch the LRU state, the plan or the
 * hot buffer. */
int orc_swap_in_row_paged(int32_t B, int32_t K, int64_t rb, int32_t max_seq,
                          int32_t L, const int32_t* block_row, int32_t max_pages,
                          int32_t page_size, int64_t hot_base,
                          const int32_t* topk, int32_t* out,
                          int32_t* lru, int32_t* tok,
                          const uint8_t* host_req, uint8_t* hot_req,
                          int32_t* plan_pos, int32_t* plan_slot, int32_t* plan_count)
{
    if (B <= 0 || K <= 0 || K > B || page_size <= 0 || max_pages < 0 || hot_base < 0 ||
        !topk || !out || !plan_count || (max_pages > 0 && !block_row))
        return ORC_EINVAL;
    if (L < 1 || L > max_seq)
        return ORC_EPRECOND;
    int rc = check_topk(K, L, topk);
    if (rc != ORC_OK)
        return rc;

    int32_t* hot_row = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
    int64_t* res_row = (int64_t*)malloc(sizeof(int64_t) * (size_t)K);
    if (!hot_row || !res_row) {
        free(hot_row); free(res_row);
        return ORC_ENOMEM;
    }
    /* Tier 0, per entry: is the position's page resident? */
    for (int32_t i = 0; i < K; ++i) {
        int32_t t = topk[i];
        res_row[i] = -1;
        hot_row[i] = t;
        if (t < 0)
            continue;
        int32_t pg = t / page_size;
        int32_t phys = pg < max_pages ? block_row[pg] : -1;
        if (phys < -1) {
            free(hot_row); free(res_row);
            return ORC_EPRECOND;
        }
        if (phys >= 0) {
            res_row[i] = (int64_t)phys * page_size + t % page_size;
            hot_row[i] = -1;                 /* leaves the hot tiers untouched */
        }
    }
    /* The remaining entries go through the hot tiers as usual. */
    rc = orc_swap_in_row(B, K, rb, max_seq, L, 0, hot_row, out, lru, tok, host_req, hot_req,
                         plan_pos, plan_slot, plan_count);
    if (rc == ORC_OK) {
        for (int32_t i = 0; i < K; ++i) {
            int64_t v;
            if (res_row[i] >= 0)
                v = res_row[i];
            else if (out[i] < 0)
                v = -1;
            else
                v = hot_base + out[i];
            if (v > INT32_MAX) {
                rc = ORC_EPRECOND;
                break;
            }
            out[i] = (int32_t)v;
        }
    }
    free(hot_row); free(res_row);
    return rc;
}

int orc_swap_in_paged(int32_t R, int32_t B, int32_t K, int64_t rb, int32_t max_seq,
                      int32_t nb, const int32_t* req_idx,
                      const int32_t* topk, const int32_t* seq_lens,
                      const int32_t* block_table, int32_t max_pages, int32_t page_size,
                      int64_t hot_row_base, int32_t* out,
                      int32_t* lru, int32_t* tok,
                      const uint8_t* host, uint8_t* hot,
                      int32_t* plan_pos, int32_t* plan_slot, int32_t* plan_count)
{
    if (R <= 0 || nb < 0 || nb > R)
        return ORC_EINVAL;
    for (int32_t b = 0; b < nb; ++b) {
        int32_t r = req_idx ? req_idx[b] : b;
        if (r < 0 || r >= R)
            return ORC_EINVAL;
        int rc = orc_swap_in_row_paged(
            B, K, rb, max_seq, seq_lens[b],
            block_table ? block_table + (int64_t)b * max_pages : NULL, max_pages, page_size,
            hot_row_base + (int64_t)r * (B + 1),
            topk + (int64_t)b * K, out + (int64_t)b * K,
            lru + (int64_t)r * B, tok + (int64_t)r * B,
            host + (int64_t)r * max_seq * rb, hot + (int64_t)r * (B + 1) * rb,
            plan_pos + (int64_t)b * K, plan_slot + (int64_t)b * K, plan_count + b);
        if (rc != ORC_OK)
            return rc;
    }
    return ORC_OK;
}

int orc_replay(int32_t R, int32_t B, int32_t K, int64_t rb, int32_t max_seq,
               int32_t nb, const int32_t* req_idx,
               const int32_t* plan_pos, const int32_t* plan_slot,
               const int32_t* plan_count,
               const uint8_t* host, uint8_t* hot)
{
    if (R <= 0 || nb < 0 || nb > R || rb <= 0)
        return ORC_EINVAL;
    for (int32_t b = 0; b < nb; ++b) {
        int32_t r = req_idx ? req_idx[b] : b;
        if (r < 0 || r >= R)
            return ORC_EINVAL;
        int32_t cnt = plan_count[b];
        if (cnt < 0 || cnt > K)
            return ORC_EPRECOND;
        for (int32_t m = 0; m < cnt; ++m) {
            int32_t t = plan_pos[(int64_t)b * K + m];
            int32_t v = plan_slot[(int64_t)b * K + m];
            if (t < 0 || t >= max_seq || v < 0 || v >= B)
                return ORC_EPRECOND;
            memcpy(hot + ((int64_t)r * (B + 1) + v) * rb,
                   host + ((int64_t)r * max_seq + t) * rb, (size_t)rb);
        }
    }
    return ORC_OK;
}

int orc_backup(int32_t R, int32_t B, int64_t rb, int32_t max_seq,
               int32_t nb, const int32_t* req_idx,
               const int32_t* seq_lens, const uint8_t* resident_mask,
               const uint8_t* hot, uint8_t* host)
{
    if (R <= 0 || nb < 0 || nb > R || rb <= 0)
        return ORC_EINVAL;
    for (int32_t b = 0; b < nb; ++b) {
        int32_t r = req_idx ? req_idx[b] : b;
        if (r < 0 || r >= R)
            return ORC_EINVAL;
        if (resident_mask && resident_mask[b])
            continue;                        /* resident KV is not host-backed */
        int32_t L = seq_lens[b];
        if (L < 1 || L > max_seq)
            return ORC_EPRECOND;
        int32_t row = orc_newest_row(B, L);
        memcpy(host + ((int64_t)r * max_seq + (L - 1)) * rb,
               hot + ((int64_t)r * (B + 1) + row) * rb, (size_t)rb);
    }
    return ORC_OK;
}

/* Page transfers (vLLM design note, "Spill transaction": a resident page's
 * contents are copied to its host page before the resident block is reused;
 * "P/D import target": an import copies a bounded device staging pool into
 * registered host memory and mirrors the pages needed right away into
 * resident destinations during that copy).  A transfer carries physical copy
 * coordinates only: (source page, request, host page, mirror page or -1).
 * A page holds page_size consecutive positions; a host page that runs past
 * max_seq is copied up to max_seq.  src holds src_pages pages, mirror holds
 * mirror_pages pages, host is [R][max_seq][rb]. */
int orc_page_copy(int32_t R, int32_t max_seq, int64_t rb, int32_t page_size,
                  const uint8_t* src, int32_t src_pages,
                  uint8_t* host, uint8_t* mirror, int32_t mirror_pages,
                  int32_t n, const int32_t* transfers)
{
    if (R <= 0 || max_seq <= 0 || rb <= 0 || page_size <= 0 || n < 0 || !src || !host)
        return ORC_EINVAL;
    for (int32_t x = 0; x < n; ++x) {
        int32_t sp = transfers[4 * x + 0];
        int32_t r = transfers[4 * x + 1];
        int32_t hp = transfers[4 * x + 2];
        int32_t mp = transfers[4 * x + 3];
        if (sp < 0 || sp >= src_pages || r < 0 || r >= R || hp < 0 ||
            (int64_t)hp * page_size >= max_seq || mp < -1 || mp >= mirror_pages || (mp >= 0 && !mirror))
            return ORC_EPRECOND;
        int64_t rows = max_seq - (int64_t)hp * page_size;
        if (rows > page_size)
            rows = page_size;
        const uint8_t* from = src + (int64_t)sp * page_size * rb;
        memcpy(host + ((int64_t)r * max_seq + (int64_t)hp * page_size) * rb, from, (size_t)(rows * rb));
        if (mp >= 0)
            memcpy(mirror + (int64_t)mp * page_size * rb, from, (size_t)(rows * rb));
    }
    return ORC_OK;
}
