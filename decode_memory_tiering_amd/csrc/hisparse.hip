// hisparse.hip -- HiSparse decode-step swap-in resolver for MI355X (gfx950).
//
// Kernels (all wave64):
//   swap_in_kernel   the fused resolver: resident / fast-path exit, LDS hash
//                    hit detection, ballot-scan LRU compaction, victim
//                    assignment, plan record and the miss copy from pinned
//                    host memory, in one launch with one workgroup per
//                    batch row; per-request or per-page residency; on
//                    request, the forward's KV write and the eager backup
//                    of the newest row in the same launch.  SGLang guide
//                    "HiSparse: Hierarchical Sparse Attention", "Decode
//                    Workflow"; vLLM design note "HiSparse local KV offload
//                    architecture", "Resident device pages" and "Hot lookup
//                    and LRU".
//   replay_kernel    copy-only replay of a plan row on a skip layer, small
//                    fixed grid.  SGLang guide, "Shared-index prefetch".
//   backup_kernel    newest token's row, hot buffer -> host pool.  SGLang
//                    guide, "Decode Workflow" (eager backup).
//   page_copy_kernel whole pages: resident -> host (spill), staging -> host
//                    with an optional resident mirror (import).  vLLM design
//                    note, "Spill transaction" and "P/D import target".  The
//                    same transfers also go as runtime copies from a host-side
//                    list (hisparse_spill_dma / hisparse_import_dma).
//   store_newest_kernel, admit_*_kernel, init_state_kernel, clear_word_kernel:
//                    the forward's KV write, request admission, context
//                    set-up.
// Host side: the C ABI of include/hisparse.h, with contexts either on memory
// from hipMalloc (hisparse_init) or in a static per-device scratch array
// (hisparse_init_static), and optional per-request counters that the
// swap-in launches add to (hisparse_set_stats).
//
// Tie-breaks the pages leave open (same readings as the oracle, reached
// independently here): victims come from the least-recent end of the LRU list
// in order; misses take them in ascending top-k index; the reorder is stable
// (new order = untouched non-hit slots, then hit slots, then loaded slots).
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>

#include "hisparse.h"

namespace {

constexpr int kWave = 64;
constexpr int kMissMark = INT_MIN;   // out_s value of an entry still waiting for a victim
constexpr int kMaxB = 16384;
constexpr int kMaxK = 4096;
constexpr int kDefaultBlock = 1024;
constexpr int kMaxLayers = 256;
constexpr int kDefaultReplayGrid = 12;   // enough to fill the host link without crowding the fabric (measured)
// Copy-loop shape: batches of kCopyUnroll 16-byte loads per thread, kCopyBuffers
// batches in rotation (measured on MI355X; see RowCopy).  The swap-in's
// miss copy runs in every slow batch row's workgroup at once (up to one per
// CU), so it keeps fewer loads in flight per thread than the replay's small
// grid does: 4 x 2 measured best across the workloads (8 x 2 and 2 x 2 were
// 0.5-1.5% slower), the replay keeps 8 x 2.
#ifndef HISPARSE_COPY_UNROLL
#define HISPARSE_COPY_UNROLL 8
#endif
#ifndef HISPARSE_SWAP_IN_COPY_UNROLL
#define HISPARSE_SWAP_IN_COPY_UNROLL 4
#endif
#ifndef HISPARSE_COPY_BUFFERS
#define HISPARSE_COPY_BUFFERS 2
#endif
constexpr int kCopyUnroll = HISPARSE_COPY_UNROLL;
constexpr int kSwapInCopyUnroll = HISPARSE_SWAP_IN_COPY_UNROLL;
constexpr int kReplayStage = 2048;   // plan rows staged in LDS per replay block
constexpr int kCopyBuffers = HISPARSE_COPY_BUFFERS;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lanes_below(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

// Adds v, summed over the wave, to *dst: one device atomic per wave.
__device__ __forceinline__ void wave_add_stat(unsigned long long* dst, int v)
{
#pragma unroll
    for (int d = kWave / 2; d > 0; d >>= 1) v += __shfl_xor(v, d, kWave);
    if ((threadIdx.x & (kWave - 1)) == 0 && v) atomicAdd(dst, static_cast<unsigned long long>(v));
}

__device__ __forceinline__ uint32_t hash_slot(int32_t t, int bits)
{
    return (static_cast<uint32_t>(t) * 0x9E3779B1u) >> (32 - bits);
}

// Exclusive prefix sum, in place, of a[0..n) by one wave, n <= 4 * 64;
// returns the total to every lane.  Lane l owns a[4l .. 4l+4) and issues its
// four reads together (entries past n read a[0] and count as 0): the rest of
// the workgroup waits at a barrier meanwhile, so this phase is pure latency.
constexpr int kScanPerLane = 4;
static_assert(kMaxB / kWave <= kScanPerLane * kWave && kMaxK / kWave <= kScanPerLane * kWave,
              "one wave scans the per-chunk counts of the largest buffer and top-k row");

__device__ int wave_exclusive_scan(int* a, int n)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int base = lane * kScanPerLane;
    int v[kScanPerLane];
#pragma unroll
    for (int k = 0; k < kScanPerLane; ++k) v[k] = a[base + k < n ? base + k : 0];
    int own = 0;
#pragma unroll
    for (int k = 0; k < kScanPerLane; ++k) {
        if (base + k >= n) v[k] = 0;
        own += v[k];
    }
    int incl = own;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        int y = __shfl_up(incl, d, kWave);
        if (lane >= d) incl += y;
    }
    int run = incl - own;
#pragma unroll
    for (int k = 0; k < kScanPerLane; ++k) {
        if (base + k < n) a[base + k] = run;
        run += v[k];
    }
    return __shfl(incl, kWave - 1, kWave);
}

// RowCopy / copy_rows: copy `rows` rows of rb bytes (rb % 16 == 0) from src
// rows to dst rows, the row numbers given by src_row(m) / dst_row(m).  Chunk c of the flattened
// (row, 16-byte column) space goes to thread c % nthr; the (row, column) walk
// is incremental, so no chunk needs a division.
//
// Software-pipelined over NB rotating register batches of U 16-byte loads:
// batch p is stored while the loads of the following NB-1 batches are in
// flight.  Rotating (not copying) the batches matters: moving a register that
// a load has not filled yet, or loading into one whose store is still
// pending, makes the compiler drain the loads.  Loads are never predicated
// for the same reason: a chunk past the end reads 16 bytes of dst instead
// (device memory) and the value is dropped.  They are plain loads: host rows
// leave the L2 as whole 128-byte lines whatever the load's cache policy, and
// plain loads gathered 656-byte rows 1-2% faster than nontemporal ones
// (measured); the L2's lines of host memory do not outlive the kernel.
struct KeepAll {
    __device__ bool operator()(int) const { return true; }
};

template <int U, int NB, typename SrcRow, typename DstRow, typename Keep = KeepAll>
struct RowCopy {
    const uint8_t* src;
    uint8_t* dst;
    int rb, nthr, cpr, total, drow, dcol, last;
    int row, col, c;                              // position and flat index of the next chunk to load
    bool idle;                                    // this thread has no chunk
    SrcRow src_row;
    DstRow dst_row;
    Keep keep;
    u32x4 v[NB][U];
    int vr[NB][U], vc[NB][U];

    __device__ __forceinline__ RowCopy(const uint8_t* src_, uint8_t* dst_, int rows, int rb_, int tid, int nthr_,
                                       SrcRow sr, DstRow dr, Keep kp)
        : src(src_), dst(dst_), rb(rb_), nthr(nthr_), src_row(sr), dst_row(dr), keep(kp)
    {
        cpr = rb >> 4;
        total = rows * cpr;
        idle = tid >= total;
        drow = nthr / cpr;
        dcol = nthr - drow * cpr;
        last = rows - 1;
        row = tid / cpr;
        col = tid - row * cpr;
        c = tid;
    }

    __device__ __forceinline__ void load_batch(int p)
    {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool in = c < total;
            const int rr = in ? row : last;       // keeps src_row's index in range
            const uint8_t* q = src + static_cast<size_t>(src_row(rr)) * rb + (static_cast<size_t>(col) << 4);
            v[p][u] = *reinterpret_cast<const u32x4*>(in ? q : dst);
            vr[p][u] = row;
            vc[p][u] = col;
            c += nthr;
            col += dcol;
            row += drow;
            if (col >= cpr) { col -= cpr; ++row; }
        }
    }

    __device__ __forceinline__ void store_batch(int p, int base)
    {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (base + u * nthr < total && keep(vr[p][u]))
                *reinterpret_cast<u32x4*>(dst + static_cast<size_t>(dst_row(vr[p][u])) * rb +
                                          (static_cast<size_t>(vc[p][u]) << 4)) = v[p][u];
        }
    }

    // Issue the loads of the first NB-1 batches.  Only src_row is used, so
    // this may run before the destination rows are known.
    __device__ __forceinline__ void prime()
    {
        if (idle) return;
#pragma unroll
        for (int p = 0; p < NB - 1; ++p) load_batch(p);
    }

    // The rest of the copy; dst_row must be valid from here on.
    __device__ __forceinline__ void finish(int tid)
    {
        if (idle) return;
        for (int base = tid;;) {
#pragma unroll
            for (int p = 0; p < NB; ++p) {
                load_batch((p + NB - 1) % NB);
                store_batch(p, base);
                base += U * nthr;
                if (base >= total) return;
            }
        }
    }
};

template <int U, int NB, typename SrcRow, typename DstRow, typename Keep = KeepAll>
__device__ __forceinline__ RowCopy<U, NB, SrcRow, DstRow, Keep>
make_row_copy(const uint8_t* src, uint8_t* dst, int rows, int rb, int tid, int nthr, SrcRow src_row, DstRow dst_row,
              Keep keep = Keep())
{
    return RowCopy<U, NB, SrcRow, DstRow, Keep>(src, dst, rows, rb, tid, nthr, src_row, dst_row, keep);
}

template <int U, int NB, typename SrcRow, typename DstRow, typename Keep = KeepAll>
__device__ __forceinline__ void copy_rows(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                          int rows, int rb, int tid, int nthr,
                                          SrcRow src_row, DstRow dst_row, Keep keep = Keep())
{
    auto cp = make_row_copy<U, NB>(src, dst, rows, rb, tid, nthr, src_row, dst_row, keep);
    cp.prime();
    cp.finish(tid);
}

// Replay's variant: row m goes from host row src_row[m] to hot row
// dst_row[m] (both absolute, from LDS); a row marked -1 is not copied (its
// load reads host row 0, which always exists, and is dropped).
__device__ __forceinline__ void copy_rows_staged(const uint8_t* __restrict__ host, uint8_t* __restrict__ hot,
                                                 const long long* src_row, const int* dst_row,
                                                 int rows, int rb, int tid, int nthr)
{
    copy_rows<kCopyUnroll, kCopyBuffers>(
        host, hot, rows, rb, tid, nthr,
        [src_row](int m) { return src_row[m] < 0 ? 0ll : src_row[m]; },
        [dst_row](int m) { return dst_row[m] < 0 ? 0 : dst_row[m]; },
        [dst_row](int m) { return dst_row[m] >= 0; });
}

// ---------------------------------------------------------------------------
// the fused resolver
// ---------------------------------------------------------------------------
struct SwapInArgs {
    const int32_t* topk;         // [nb][K]
    const int32_t* seq_lens;     // [nb]
    const uint8_t* resident;     // [nb] or null
    const int32_t* req_idx;      // [nb] or null
    int32_t* out;                // [nb][K]
    int32_t* plan_pos;           // [nb][K]
    int32_t* plan_slot;          // [nb][K]
    int32_t* plan_count;         // [nb]
    int32_t* lru;                // [R][B]  least recent first
    int32_t* tok;                // [R][B]  position held by each slot, -1 = empty
    const uint8_t* host;         // [R][max_seq][rb]
    uint8_t* hot;                // [R][B+1][rb]
    uint32_t* err;
    int32_t R, B, K, rb, max_seq, hash_bits;
    // per-page residency (paged != 0): block_table [nb][max_pages] physical
    // page or -1; outputs are rows of the caller's view (resident rows
    // page * page_size + t % page_size, hot rows hot_row_base + r*(B+1) + slot)
    const int32_t* block_table;
    int32_t paged, max_pages, page_size, hot_row_base;
    const uint8_t* new_rows;     // [nb][rb] or null: the forward's KV write fused into this launch
    uint8_t* backup_host;        // [R][max_seq][rb] or null: with new_rows, the eager backup fused in too
    unsigned long long* stats;   // [R][HISPARSE_STAT_COUNT] or null: per-request counters, added to
};

constexpr unsigned long long kHashEmpty = ~0ull;
constexpr uint32_t kResidentIdx = 0x80000000u;   // hash value flag: the entry resolved in tier 0

// Tier 0 of the paged resolver: the physical row of position t (0 <= t) when
// its page is resident, else -1; a bad block-table entry sets *err.
__device__ __forceinline__ int resident_row(const int32_t* bt_row, int max_pages, int page_size, int t,
                                            uint32_t* err)
{
    const int pg = t / page_size;
    if (pg >= max_pages) return -1;          // past the table: host-backed
    const int phys = bt_row[pg];
    if (phys < 0) {
        if (phys < -1) *err |= HISPARSE_DERR_PAGE;
        return -1;
    }
    const long long row = static_cast<long long>(phys) * page_size + t % page_size;
    if (row > INT_MAX) { *err |= HISPARSE_DERR_PAGE; return -1; }
    return static_cast<int>(row);
}

struct SwapInLds {
    unsigned long long* hash;  // [1 << hash_bits]  (position << 32) | top-k index; kHashEmpty = free
    int* out_s;     // [K]   -1 / B / slot of a hit / kMissMark
    int* plan_t;    // [K]   m-th miss: host position
    int* plan_v;    // [K]   m-th least recent non-hit slot (victim of the m-th miss)
    int* cnt_b;     // [ceil(B/64)]  hits per 64-entry chunk of the LRU list, then prefix
    int* cnt_k;     // [ceil(K/64)]  misses per 64-entry chunk of the top-k row, then prefix
    int* totals;    // [4]   hits, misses
    uint8_t* hit;   // [B]   slot was hit this step
};

__host__ __device__ inline size_t swap_in_lds_bytes_impl(int B, int K, int hash_bits)
{
    const size_t ints = 3 * size_t(K) + (B + 63) / 64 + (K + 63) / 64 + 4;
    return (size_t(1) << hash_bits) * 8 + ints * 4 + ((size_t(B) + 3) & ~size_t(3));
}

__device__ inline SwapInLds carve_lds(unsigned long long* smem, int B, int K, int hash_bits)
{
    SwapInLds s;
    s.hash = smem;
    s.out_s = reinterpret_cast<int*>(s.hash + (size_t(1) << hash_bits));
    s.plan_t = s.out_s + K;
    s.plan_v = s.plan_t + K;
    s.cnt_b = s.plan_v + K;
    s.cnt_k = s.cnt_b + (B + 63) / 64;
    s.totals = s.cnt_k + (K + 63) / 64;
    s.hit = reinterpret_cast<uint8_t*>(s.totals + 4);
    return s;
}

// A batch row whose device-side preconditions fail resolves to -1 and changes
// nothing else; every thread passes the flags it saw.
__device__ void fail_row(const SwapInArgs& a, int b, uint32_t flags)
{
    for (int i = threadIdx.x; i < a.K; i += blockDim.x) a.out[size_t(b) * a.K + i] = -1;
    if (flags) atomicOr(a.err, flags);
    if (threadIdx.x == 0) a.plan_count[b] = 0;
}

// EB / EK: 64-entry chunks of the LRU list / top-k row held per wave.
// STATS: the per-request counters of hisparse_set_stats are kept (a.stats
// set); the instantiations without it are used otherwise and carry no cost.
template <int EB, int EK, bool STATS>
__global__ __launch_bounds__(1024) void swap_in_kernel(SwapInArgs a)
{
    extern __shared__ unsigned long long smem[];
    const int b = blockIdx.x;
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave, nwaves = nthr / kWave;
    const int B = a.B, K = a.K;
    const int32_t* topk = a.topk + size_t(b) * K;
    int32_t* out = a.out + size_t(b) * K;
    const int L = a.seq_lens[b];

    // The forward's KV write, when fused into this launch: the newest token's
    // row goes to row L-1 (L <= B) or B, as store_newest_kernel does, and,
    // with the backup fused in too, to host position L-1, as backup_kernel
    // would copy it from there.  The resolver never reads that row, never
    // picks it as a victim and never reads host position L-1 (it resolves to
    // the newest row), so neither write needs ordering against the rest.
    if (a.new_rows && !(a.resident && a.resident[b])) {
        const int rs = a.req_idx ? a.req_idx[b] : b;
        if (rs >= 0 && rs < a.R && L >= 1) {
            const int row = L <= B ? L - 1 : B;
            const uint8_t* src = a.new_rows + size_t(b) * a.rb;
            uint8_t* dst = a.hot + (size_t(rs) * (B + 1) + row) * a.rb;
            uint8_t* bdst = a.backup_host && L <= a.max_seq
                                ? a.backup_host + (size_t(rs) * a.max_seq + (L - 1)) * a.rb : nullptr;
            for (int c = tid; c < (a.rb >> 4); c += nthr) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(src + (size_t(c) << 4));
                *reinterpret_cast<u32x4*>(dst + (size_t(c) << 4)) = v;
                if (bdst) *reinterpret_cast<u32x4*>(bdst + (size_t(c) << 4)) = v;
            }
            if (a.backup_host && L > a.max_seq && tid == 0) atomicOr(a.err, HISPARSE_DERR_SEQ_LEN);
        } else if (tid == 0) {
            atomicOr(a.err, (rs < 0 || rs >= a.R) ? HISPARSE_DERR_REQ_IDX : HISPARSE_DERR_SEQ_LEN);
        }
    }

    // Tier 0 (resident request) and the short-sequence fast path: the slot
    // is the position; no state, no plan, no copy.
    if (!a.paged && ((a.resident && a.resident[b]) || L <= B)) {
        int valid = 0;
        for (int i = tid; i < K; i += nthr) {
            const int t = topk[i];
            out[i] = t;
            valid += t >= 0;
        }
        if (tid == 0) a.plan_count[b] = 0;
        const int rq = a.req_idx ? a.req_idx[b] : b;
        if (STATS && rq >= 0 && rq < a.R) {
            unsigned long long* st = a.stats + size_t(rq) * HISPARSE_STAT_COUNT;
            wave_add_stat(st + HISPARSE_STAT_ENTRIES, valid);
            wave_add_stat(st + ((a.resident && a.resident[b]) ? HISPARSE_STAT_RESIDENT : HISPARSE_STAT_FAST), valid);
        }
        return;
    }
    const int r = a.req_idx ? a.req_idx[b] : b;
    if (r < 0 || r >= a.R) { fail_row(a, b, HISPARSE_DERR_REQ_IDX); return; }
    const int32_t* bt_row = a.paged ? a.block_table + size_t(b) * a.max_pages : nullptr;
    const int hot_base = a.paged ? a.hot_row_base + r * (B + 1) : 0;
    if (a.paged && L <= B) {
        // Paged fast path: resident pages resolve in tier 0, every other
        // position sits at slot = position.  Checked first, written second,
        // so a bad row changes nothing.
        uint32_t perr = 0;
        for (int i = tid; i < K; i += nthr) {
            const int t = topk[i];
            if (t < -1 || t >= L) perr |= HISPARSE_DERR_TOPK_RANGE;
            else if (t >= 0) (void)resident_row(bt_row, a.max_pages, a.page_size, t, &perr);
        }
        if (__syncthreads_or(perr != 0)) { fail_row(a, b, perr); return; }
        int n_res = 0, n_fast = 0;
        for (int i = tid; i < K; i += nthr) {
            const int t = topk[i];
            uint32_t unused = 0;
            const int rr = t >= 0 ? resident_row(bt_row, a.max_pages, a.page_size, t, &unused) : -1;
            out[i] = t < 0 ? -1 : (rr >= 0 ? rr : hot_base + t);
            n_res += rr >= 0;
            n_fast += t >= 0 && rr < 0;
        }
        if (tid == 0) a.plan_count[b] = 0;
        if (STATS) {
            unsigned long long* st = a.stats + size_t(r) * HISPARSE_STAT_COUNT;
            wave_add_stat(st + HISPARSE_STAT_ENTRIES, n_res + n_fast);
            wave_add_stat(st + HISPARSE_STAT_RESIDENT, n_res);
            wave_add_stat(st + HISPARSE_STAT_FAST, n_fast);
        }
        return;
    }
    if (L > a.max_seq) { fail_row(a, b, HISPARSE_DERR_SEQ_LEN); return; }

    SwapInLds s = carve_lds(smem, B, K, a.hash_bits);
    const int hmask = (1 << a.hash_bits) - 1;
    const int ncb = (B + 63) / 64, nck = (K + 63) / 64;
    int32_t* lru = a.lru + size_t(r) * B;
    int32_t* tok = a.tok + size_t(r) * B;

    // Every global read of the resolve is issued here, before any barrier,
    // so the whole pass waits on one memory latency.  Entry e of chunk
    // c = k * nwaves + wave is e = c * 64 + lane (top-k row, slot map and
    // LRU list alike).
    // (The LRU list is read here only when the registers allow it; the
    // largest buffers read it after the probe instead of spilling.)
    constexpr bool kEarlyLru = EB <= 8;
    int t_own[EK], tok_own[EB], lru_own[EB];
#pragma unroll
    for (int k = 0; k < EK; ++k) {
        const int c = k * nwaves + wave, i = c * kWave + lane;
        t_own[k] = (c < nck && i < K) ? topk[i] : -1;
    }
#pragma unroll
    for (int k = 0; k < EB; ++k) {
        const int c = k * nwaves + wave, x = c * kWave + lane;
        const bool in = c < ncb && x < B;
        tok_own[k] = in ? tok[x] : -1;
        lru_own[k] = (kEarlyLru && in) ? lru[x] : 0;
    }
    for (int h = tid; h <= hmask; h += nthr) s.hash[h] = kHashEmpty;
    for (int q = tid; q < (B + 3) / 4; q += nthr) reinterpret_cast<uint32_t*>(s.hit)[q] = 0u;   // padded to 4 bytes

    // -- classify the top-k row ------------------------------------------
    uint32_t err = 0;
    uint32_t rbits = 0;                            // entries resolved in tier 0 (resident page)
#pragma unroll
    for (int k = 0; k < EK; ++k) {
        const int c = k * nwaves + wave, i = c * kWave + lane;
        if (c < nck && i < K) {
            const int t = t_own[k];
            int cls;
            if (t == -1) cls = -1;
            else if (t < -1 || t >= L) { cls = -1; err |= HISPARSE_DERR_TOPK_RANGE; }
            else {
                const int rr = a.paged ? resident_row(bt_row, a.max_pages, a.page_size, t, &err) : -1;
                if (rr >= 0) { cls = rr; rbits |= 1u << k; }   // resident page: physical row
                else if (t == L - 1) cls = B;                 // newest token: its own row
                else cls = kMissMark;
            }
            s.out_s[i] = cls;
        }
    }
    __syncthreads();

    // -- LDS hash of candidate positions: position -> top-k index --------
#pragma unroll
    for (int k = 0; k < EK; ++k) {
        const int c = k * nwaves + wave, i = c * kWave + lane;
        const int t = t_own[k];
        const bool res = (rbits >> k) & 1u;
        // resident entries go in too (flagged), so a repeated position is
        // caught whatever its tier and a slot holding it is never a hit
        if (c < nck && i < K && t >= 0 && t < L && (res || t < L - 1)) {
            const unsigned long long e = (static_cast<unsigned long long>(static_cast<uint32_t>(t)) << 32) |
                                         (static_cast<uint32_t>(i) | (res ? kResidentIdx : 0u));
            uint32_t h = hash_slot(t, a.hash_bits);
            for (;;) {   // at most K of the table's >= 2K entries are used (load <= 1/2), so a free one is always reached
                const unsigned long long prev = atomicCAS(&s.hash[h], kHashEmpty, e);
                if (prev == kHashEmpty) break;
                if (static_cast<uint32_t>(prev >> 32) == static_cast<uint32_t>(t)) {
                    err |= HISPARSE_DERR_TOPK_DUP;
                    break;
                }
                h = (h + 1) & hmask;
            }
        }
    }
    if (__syncthreads_or(err != 0)) {
        fail_row(a, b, err);
        return;
    }

    // -- hit detection: probe every slot's position ----------------------
    // A thread's probes advance in lockstep, one table entry per round, in
    // groups of up to 8 chains.  (Each chain's read still waits on its own
    // result before the next chain's; the workgroup's 16 waves are what keep
    // the LDS busy, so the phase is bound by LDS throughput, not latency.)
    constexpr int kG = EB < 8 ? EB : 8;
#pragma unroll
    for (int g0 = 0; g0 < EB; g0 += kG) {
        uint32_t h[kG];
        uint32_t pending = 0;
#pragma unroll
        for (int q = 0; q < kG; ++q) {
            const int k = g0 + q;
            const int c = k * nwaves + wave, x = c * kWave + lane;
            const int t = tok_own[k];
            h[q] = 0;
            if (c < ncb && x < B) {
                if (t >= 0 && t < L - 1) {
                    h[q] = hash_slot(t, a.hash_bits);
                    pending |= 1u << q;
                } else if (t < -1 || t >= a.max_seq) {
                    err |= HISPARSE_DERR_STATE;
                }
            }
        }
        while (pending) {   // ends: every chain stops at a free entry, and the table is at most half full
#pragma unroll
            for (int q = 0; q < kG; ++q) {
                if (!((pending >> q) & 1u)) continue;
                const int k = g0 + q;
                const unsigned long long e = s.hash[h[q]];
                if (e == kHashEmpty) {
                    pending &= ~(1u << q);
                } else if (static_cast<uint32_t>(e >> 32) == static_cast<uint32_t>(tok_own[k])) {
                    const int x = (k * nwaves + wave) * kWave + lane;
                    const uint32_t v = static_cast<uint32_t>(e);
                    if (!(v & kResidentIdx)) {        // a resident position is never a hot hit
                        const int i = static_cast<int>(v);
                        if (atomicCAS(&s.out_s[i], kMissMark, x) == kMissMark) s.hit[x] = 1;
                        else err |= HISPARSE_DERR_STATE;   // two slots claim one position
                    }
                    pending &= ~(1u << q);
                } else {
                    h[q] = (h[q] + 1) & hmask;
                }
            }
        }
    }
    __syncthreads();

    // -- misses along the top-k row, their ranks, the first copy loads -----
    // The m-th miss reads host row plan_t[m]; that is known as soon as the
    // miss ranks are, so the first batch of the copy's loads is issued
    // before the hits along the LRU list are even counted, and is in flight
    // while the LRU list is reordered and the victims are chosen (the copy's
    // stores wait for those).  Nothing global is written before the checks
    // below, so a row that fails them still changes nothing.
    int lp_k[EK];
    uint32_t mbits = 0;
#pragma unroll
    for (int k = 0; k < EK; ++k) {
        const int c = k * nwaves + wave, i = c * kWave + lane;
        lp_k[k] = 0;
        if (c < nck) {
            const bool miss = i < K && s.out_s[i] == kMissMark;
            const uint64_t m = __ballot(miss);
            lp_k[k] = lanes_below(m);
            mbits |= uint32_t(miss) << k;
            if (lane == 0) s.cnt_k[c] = __popcll(m);
        }
    }
    __syncthreads();
    if (wave == 0) {
        const int n_miss = wave_exclusive_scan(s.cnt_k, nck);
        if (lane == 0) s.totals[1] = n_miss;
    }
    __syncthreads();
    const int M = s.totals[1];
    int m_own[EK];
#pragma unroll
    for (int k = 0; k < EK; ++k) {
        const int c = k * nwaves + wave;
        m_own[k] = -1;
        if (c < nck && ((mbits >> k) & 1u)) {
            const int m = s.cnt_k[c] + lp_k[k];
            s.plan_t[m] = t_own[k];
            m_own[k] = m;
        }
    }
    __syncthreads();
    const uint8_t* src = a.host + size_t(r) * a.max_seq * a.rb;
    uint8_t* dst = a.hot + size_t(r) * (B + 1) * a.rb;
    const int* pt = s.plan_t;
    const int* pv = s.plan_v;
    auto copy = make_row_copy<kSwapInCopyUnroll, kCopyBuffers>(src, dst, M, a.rb, tid, nthr,
                                                               [pt](int m) { return pt[m]; },
                                                               [pv](int m) { return pv[m]; });
    copy.prime();

    // -- hits along the LRU list and their ranks ---------------------------
    int lp_b[EB];
    uint32_t hbits = 0;
#pragma unroll
    for (int k = 0; k < EB; ++k) {
        const int c = k * nwaves + wave, j = c * kWave + lane;
        lp_b[k] = 0;
        if (c < ncb) {
            bool f = false;
            if (j < B) {
                int x = kEarlyLru ? lru_own[k] : lru[j];
                if (x < 0 || x >= B) { err |= HISPARSE_DERR_STATE; x = 0; }
                lru_own[k] = x;
                f = s.hit[x] != 0;
            }
            const uint64_t m = __ballot(f);
            lp_b[k] = lanes_below(m);
            hbits |= uint32_t(f) << k;
            if (lane == 0) s.cnt_b[c] = __popcll(m);
        }
    }
    if (__syncthreads_or(err != 0)) {
        fail_row(a, b, err);
        return;
    }
    if (wave == 0) {
        const int n_hit = wave_exclusive_scan(s.cnt_b, ncb);
        if (lane == 0) s.totals[0] = n_hit;
    }
    __syncthreads();
    const int n_hit = s.totals[0];
    const int n_keep = B - n_hit;   // non-hit slots; >= M because K <= B
    if (n_keep < M) {               // only when the LRU list repeats a slot
        fail_row(a, b, HISPARSE_DERR_STATE);
        return;
    }

    // -- LRU reorder and victim choice ------------------------------------
    // new order: non-hit slots n >= M, then hit slots, then victims n < M.
#pragma unroll
    for (int k = 0; k < EB; ++k) {
        const int c = k * nwaves + wave, j = c * kWave + lane;
        if (c < ncb && j < B) {
            const int hits_before = s.cnt_b[c] + lp_b[k];
            const int x = lru_own[k];
            int pos;
            if ((hbits >> k) & 1u) {
                pos = n_keep - M + hits_before;
            } else {
                const int n = j - hits_before;
                if (n >= M) {
                    pos = n - M;
                } else {
                    pos = B - M + n;
                    s.plan_v[n] = x;
                }
            }
            lru[pos] = x;
        }
    }
    __syncthreads();

    // -- outputs, slot map, plan row ----------------------------------------
#pragma unroll
    for (int k = 0; k < EK; ++k) {
        const int c = k * nwaves + wave, i = c * kWave + lane;
        if (c < nck && i < K) {
            const int o = m_own[k] >= 0 ? s.plan_v[m_own[k]] : s.out_s[i];
            out[i] = ((rbits >> k) & 1u) || o < 0 ? o : hot_base + o;   // hot rows into the caller's view
        }
    }
    int32_t* pp = a.plan_pos + size_t(b) * K;
    int32_t* ps = a.plan_slot + size_t(b) * K;
    for (int m = tid; m < M; m += nthr) {
        const int t = s.plan_t[m], v = s.plan_v[m];
        tok[v] = t;
        pp[m] = t;
        ps[m] = v;
    }
    if (tid == 0) a.plan_count[b] = M;

    // -- miss copy: pinned host rows -> victim slots -----------------------
    copy.finish(tid);

    // -- per-request counters (hisparse_set_stats) --------------------------
    // After the copy, so the copy's registers are free: every valid entry
    // is resident (paged tier 0, looked up again), the newest row (its out_s
    // stayed B), a hit (one per hit slot) or a miss.  Wave counts come from
    // ballots (wave-uniform); the LDS read here was written before the last
    // barrier.
    if (STATS) {
        int n_res = 0, n_newest = 0;
#pragma unroll
        for (int k = 0; k < EK; ++k) {
            const int c = k * nwaves + wave, i = c * kWave + lane;
            const bool in = c < nck && i < K;
            bool res = false;
            if (in && a.paged) {
                const int t = topk[i];
                uint32_t unused = 0;
                res = t >= 0 && resident_row(bt_row, a.max_pages, a.page_size, t, &unused) >= 0;
            }
            const bool nw = in && !res && s.out_s[i] == B;
            n_res += __popcll(__ballot(res));
            n_newest += __popcll(__ballot(nw));
        }
        unsigned long long* st = a.stats + size_t(r) * HISPARSE_STAT_COUNT;
        if (lane == 0 && n_res + n_newest) {
            atomicAdd(st + HISPARSE_STAT_RESIDENT, static_cast<unsigned long long>(n_res));
            atomicAdd(st + HISPARSE_STAT_NEWEST, static_cast<unsigned long long>(n_newest));
            atomicAdd(st + HISPARSE_STAT_ENTRIES, static_cast<unsigned long long>(n_res + n_newest));
        }
        if (tid == 0) {
            const int hits = s.totals[0], misses = s.totals[1];
            atomicAdd(st + HISPARSE_STAT_HIT, static_cast<unsigned long long>(hits));
            atomicAdd(st + HISPARSE_STAT_MISS, static_cast<unsigned long long>(misses));
            atomicAdd(st + HISPARSE_STAT_ENTRIES, static_cast<unsigned long long>(hits + misses));
        }
    }
}

// ---------------------------------------------------------------------------
// replay, backup, forward write, admission
// ---------------------------------------------------------------------------
struct ReplayArgs {
    const int32_t* pos;
    const int32_t* slot;
    const int32_t* count;
    const int32_t* req_idx;
    const uint8_t* host;
    uint8_t* hot;
    uint32_t* err;
    int32_t nb, R, B, K, rb, max_seq;
};

// Small fixed grid.  The plan's rows, across all batch rows, are numbered
// 0..total-1 (an exclusive prefix of the counts, computed by every workgroup
// in LDS), and the flattened (row, 16-byte column) space is split evenly over
// the grid: each workgroup copies one contiguous range, so the grid stays
// busy until the end whatever the counts are.  A row with an invalid count or
// request index is skipped as a whole, a pair out of range on its own; both
// set the error word.
__global__ __launch_bounds__(256) void replay_kernel(ReplayArgs a)
{
    extern __shared__ int start[];           // [nb + 1] first flattened row of each batch row; [nb] = total
    __shared__ int wave_total[1024 / kWave];
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;

    // -- exclusive prefix of the valid counts over the batch ------------------
    const int seg = (a.nb + nthr - 1) / nthr;
    int mine = 0;
    uint32_t flags = 0;
    for (int q = 0; q < seg; ++q) {
        const int b = tid * seg + q;
        if (b >= a.nb) break;
        int cnt = a.count[b];
        const int r = a.req_idx ? a.req_idx[b] : b;
        if (r < 0 || r >= a.R) { flags |= HISPARSE_DERR_REQ_IDX; cnt = 0; }
        else if (cnt < 0 || cnt > a.K) { flags |= HISPARSE_DERR_PLAN; cnt = 0; }
        start[b] = cnt;
        mine += cnt;
    }
    if (flags && blockIdx.x == 0) atomicOr(a.err, flags);
    int incl = mine;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int y = __shfl_up(incl, d, kWave);
        if (lane >= d) incl += y;
    }
    if (lane == kWave - 1) wave_total[wave] = incl;
    __syncthreads();
    int run = incl - mine, total_rows = 0;
    for (int w = 0; w < nthr / kWave; ++w) {
        const int t = wave_total[w];
        if (w < wave) run += t;
        total_rows += t;
    }
    for (int q = 0; q < seg; ++q) {
        const int b = tid * seg + q;
        if (b >= a.nb) break;
        const int cnt = start[b];
        start[b] = run;
        run += cnt;
    }
    if (tid == 0) start[a.nb] = total_rows;
    __syncthreads();

    // -- this workgroup's range of plan rows, in LDS-staged blocks ----------
    // Rows are split evenly over the grid; each block of up to kReplayStage
    // rows has its (host row, hot row) pairs gathered into LDS with coalesced
    // reads, then copied by the same pipelined loop as the swap-in's misses.
    const int per = (total_rows + gridDim.x - 1) / gridDim.x;
    const int row_lo = per * blockIdx.x;
    const int row_hi = row_lo + per < total_rows ? row_lo + per : total_rows;
    long long* src_row = reinterpret_cast<long long*>(start + ((a.nb + 2) & ~1));   // 8-byte aligned
    int* dst_row = reinterpret_cast<int*>(src_row + kReplayStage);
    int b = 0;                               // batch row holding row_lo
    for (int lo_b = 0, hi_b = a.nb - 1; lo_b < hi_b;) {
        const int mid = (lo_b + hi_b + 1) >> 1;
        if (start[mid] <= row_lo) lo_b = mid; else hi_b = mid - 1;
        b = lo_b;
    }
    for (int f0 = row_lo; f0 < row_hi; f0 += kReplayStage) {
        const int n = row_hi - f0 < kReplayStage ? row_hi - f0 : kReplayStage;
        // every thread walks b forward to its row; rows are consecutive, so
        // the walk per thread is short
        int bt = b;
        for (int q = tid; q < n; q += nthr) {
            const int f = f0 + q;
            while (bt + 1 < a.nb && start[bt + 1] <= f) ++bt;
            const int m = f - start[bt];
            const int r = a.req_idx ? a.req_idx[bt] : bt;
            const int t = a.pos[size_t(bt) * a.K + m];
            const int v = a.slot[size_t(bt) * a.K + m];
            if (t < 0 || t >= a.max_seq || v < 0 || v >= a.B) {
                atomicOr(a.err, HISPARSE_DERR_PLAN);
                src_row[q] = -1;             // skipped: copied onto itself below
                dst_row[q] = -1;
            } else {
                src_row[q] = static_cast<long long>(r) * a.max_seq + t;
                dst_row[q] = r * (a.B + 1) + v;
            }
        }
        __syncthreads();
        copy_rows_staged(a.host, a.hot, src_row, dst_row, n, a.rb, tid, nthr);
        __syncthreads();
        while (b + 1 < a.nb && start[b + 1] <= f0 + n) ++b;
    }
}

struct RowArgs {
    const int32_t* seq_lens;
    const uint8_t* resident;
    const int32_t* req_idx;
    const uint8_t* src;          // store_newest: new rows [nb][rb]
    const uint8_t* host_c;       // backup: hot buffer (read)
    uint8_t* host;               // backup: host pool (written)
    uint8_t* hot;                // store_newest: hot buffer (written)
    uint32_t* err;
    int32_t nb, R, B, rb, max_seq;
};

__device__ __forceinline__ void copy_one_row(const uint8_t* src, uint8_t* dst, int rb)
{
    for (int c = threadIdx.x; c < (rb >> 4); c += blockDim.x) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(src + (size_t(c) << 4));
        *reinterpret_cast<u32x4*>(dst + (size_t(c) << 4)) = v;
    }
}

// One wave per batch row: the forward's new KV row -> newest-token row.
__global__ __launch_bounds__(64) void store_newest_kernel(RowArgs a)
{
    const int b = blockIdx.x;
    if (a.resident && a.resident[b]) return;
    const int r = a.req_idx ? a.req_idx[b] : b;
    const int L = a.seq_lens[b];
    if (r < 0 || r >= a.R || L < 1) {
        if (threadIdx.x == 0) atomicOr(a.err, (r < 0 || r >= a.R) ? HISPARSE_DERR_REQ_IDX : HISPARSE_DERR_SEQ_LEN);
        return;
    }
    const int row = L <= a.B ? L - 1 : a.B;
    copy_one_row(a.src + size_t(b) * a.rb, a.hot + (size_t(r) * (a.B + 1) + row) * a.rb, a.rb);
}

// One wave per batch row: newest-token row -> host pool position L-1.
__global__ __launch_bounds__(64) void backup_kernel(RowArgs a)
{
    const int b = blockIdx.x;
    if (a.resident && a.resident[b]) return;
    const int r = a.req_idx ? a.req_idx[b] : b;
    const int L = a.seq_lens[b];
    if (r < 0 || r >= a.R || L < 1 || L > a.max_seq) {
        if (threadIdx.x == 0) atomicOr(a.err, (r < 0 || r >= a.R) ? HISPARSE_DERR_REQ_IDX : HISPARSE_DERR_SEQ_LEN);
        return;
    }
    const int row = L <= a.B ? L - 1 : a.B;
    copy_one_row(a.host_c + (size_t(r) * (a.B + 1) + row) * a.rb,
                 a.host + (size_t(r) * a.max_seq + (L - 1)) * a.rb, a.rb);
}

// Page transfers: spill (resident page -> host page) and host import
// (staging page -> host page, mirrored into a resident page when asked).
// transfers [n][4] = (source page, request, host page, mirror page or -1);
// a page is page_size consecutive positions, cut at max_seq.  Each
// workgroup copies whole pages (contiguous rows on both sides); a transfer
// with a coordinate out of range is skipped and sets HISPARSE_DERR_PAGE.
struct PageCopyArgs {
    const uint8_t* src;          // [src_pages * P][rb], device
    uint8_t* host;               // [R][max_seq][rb], pinned host
    uint8_t* mirror;             // [mirror_pages * P][rb], device, or null
    const int32_t* transfers;
    uint32_t* err;
    int32_t src_pages, mirror_pages, n, R, max_seq, rb, P;
};

__global__ __launch_bounds__(256) void page_copy_kernel(PageCopyArgs a)
{
    const int tid = threadIdx.x, nthr = blockDim.x;
    for (int x = blockIdx.x; x < a.n; x += gridDim.x) {
        const int sp = a.transfers[4 * x + 0], r = a.transfers[4 * x + 1];
        const int hp = a.transfers[4 * x + 2], mp = a.transfers[4 * x + 3];
        const bool ok = sp >= 0 && sp < a.src_pages && r >= 0 && r < a.R && hp >= 0 &&
                        static_cast<long long>(hp) * a.P < a.max_seq && mp >= -1 && mp < a.mirror_pages;
        if (!ok) {
            if (tid == 0) atomicOr(a.err, HISPARSE_DERR_PAGE);
            continue;
        }
        const int rows = a.max_seq - hp * a.P < a.P ? a.max_seq - hp * a.P : a.P;
        const int chunks = rows * (a.rb >> 4);
        const uint8_t* src = a.src + size_t(sp) * a.P * a.rb;
        uint8_t* dst = a.host + (size_t(r) * a.max_seq + size_t(hp) * a.P) * a.rb;
        uint8_t* mdst = mp >= 0 ? a.mirror + size_t(mp) * a.P * a.rb : nullptr;
        for (int c0 = tid; c0 < chunks; c0 += kCopyUnroll * nthr) {
            u32x4 v[kCopyUnroll];
#pragma unroll
            for (int u = 0; u < kCopyUnroll; ++u) {
                const int c = c0 + u * nthr;
                if (c < chunks) v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (size_t(c) << 4)));
            }
#pragma unroll
            for (int u = 0; u < kCopyUnroll; ++u) {
                const int c = c0 + u * nthr;
                if (c < chunks) {
                    *reinterpret_cast<u32x4*>(dst + (size_t(c) << 4)) = v[u];
                    if (mdst) *reinterpret_cast<u32x4*>(mdst + (size_t(c) << 4)) = v[u];
                }
            }
        }
    }
}

__global__ __launch_bounds__(256) void init_state_kernel(int32_t* lru, int32_t* tok, int R, int B)
{
    const size_t n = size_t(R) * B;
    for (size_t e = size_t(blockIdx.x) * blockDim.x + threadIdx.x; e < n; e += size_t(gridDim.x) * blockDim.x) {
        lru[e] = int32_t(e % B);
        tok[e] = -1;
    }
}

__global__ __launch_bounds__(64) void clear_word_kernel(uint32_t* w)
{
    if (threadIdx.x == 0) *w = 0u;
}

__global__ __launch_bounds__(256) void admit_state_kernel(int32_t* lru, int32_t* tok, const int32_t* req_ids,
                                                          const int32_t* L0s, int R, int B, int max_seq,
                                                          uint32_t* err)
{
    const int r = req_ids[blockIdx.x];
    const int L0 = L0s[blockIdx.x];
    if (r < 0 || r >= R || L0 < 0 || L0 > max_seq) {   // admit_fill_kernel skips the same entries
        if (threadIdx.x == 0) atomicOr(err, (r < 0 || r >= R) ? HISPARSE_DERR_REQ_IDX : HISPARSE_DERR_SEQ_LEN);
        return;
    }
    for (int x = threadIdx.x; x < B; x += blockDim.x) {
        lru[size_t(r) * B + x] = x;
        tok[size_t(r) * B + x] = L0 <= B ? x : -1;
    }
}

// grid (n, parts): rows [0, L0) of a request, host pool -> hot buffer (same
// offsets: slot = position), split over `parts` workgroups.
__global__ __launch_bounds__(256) void admit_fill_kernel(const uint8_t* host, uint8_t* hot, const int32_t* req_ids,
                                                         const int32_t* L0s, int R, int B, int rb, int max_seq)
{
    const int r = req_ids[blockIdx.x];
    const int L0 = L0s[blockIdx.x];
    if (r < 0 || r >= R || L0 <= 0 || L0 > B || L0 > max_seq) return;
    const size_t chunks = size_t(L0) * (rb >> 4);
    const uint8_t* src = host + size_t(r) * max_seq * rb;
    uint8_t* dst = hot + size_t(r) * (B + 1) * rb;
    for (size_t c = size_t(blockIdx.y) * blockDim.x + threadIdx.x; c < chunks; c += size_t(gridDim.y) * blockDim.x) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (c << 4)));
        *reinterpret_cast<u32x4*>(dst + (c << 4)) = v;
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
typedef void (*SwapInFn)(SwapInArgs);

template <int EB, int EK>
SwapInFn pick2(bool stats) { return stats ? &swap_in_kernel<EB, EK, true> : &swap_in_kernel<EB, EK, false>; }

// K <= B gives EK <= EB, so only those instantiations exist.
template <int EB>
SwapInFn pick_k(int ek, bool stats)
{
    if (ek <= 1) return pick2<EB, 1>(stats);
    if constexpr (EB >= 2) {
        if (ek <= 2) return pick2<EB, 2>(stats);
    }
    if constexpr (EB >= 4) {
        if (ek <= 4) return pick2<EB, 4>(stats);
    }
    return nullptr;
}

SwapInFn pick_kernel(int eb, int ek, bool stats)
{
    if (eb <= 1) return pick_k<1>(ek, stats);
    if (eb <= 2) return pick_k<2>(ek, stats);
    if (eb <= 4) return pick_k<4>(ek, stats);
    if (eb <= 8) return pick_k<8>(ek, stats);
    if (eb <= 16) return pick_k<16>(ek, stats);
    return nullptr;
}

// Open-addressed LDS table: 4K entries (load factor at most 1/4, short probe
// chains) when that fits the workgroup's LDS budget, else 2K (at most 1/2).
int hash_bits_for(int K, int B, size_t lds_budget)
{
    int bits = 2;
    while ((1 << bits) < 4 * K) ++bits;
    if (swap_in_lds_bytes_impl(B, K, bits) > lds_budget) --bits;
    return bits;
}

constexpr size_t kGfx950LdsPerWorkgroup = 160 * 1024;

// Dynamic LDS of the replay kernel: the prefix of the plan counts (padded to
// 8 bytes), then one staged block of (host row, hot row) pairs.
size_t replay_lds_bytes(int nb)
{
    return size_t((nb + 2) & ~1) * sizeof(int) + size_t(kReplayStage) * (sizeof(long long) + sizeof(int));
}

}  // namespace

struct hisparse_ctx {
    int device = 0;
    int32_t K = 0, B = 0, layers = 0, R = 0, max_seq = 0, rb = 0;
    int block = kDefaultBlock, replay_grid = kDefaultReplayGrid, hash_bits = 1;
    size_t lds = 0;
    SwapInFn swap_in_fn[2] = {nullptr, nullptr};   // without / with the per-request counters
    // per layer (fixed arrays: a context holds no heap memory beyond itself)
    const uint8_t* host[kMaxLayers] = {};   // device-usable address of each layer's host pool
    uint8_t* host_ptr[kMaxLayers] = {};     // the same pool's host address (runtime-copy transfers)
    uint8_t* hot[kMaxLayers] = {};
    int32_t anchor_of[kMaxLayers] = {};
    int32_t* lru[kMaxLayers] = {};          // null for skip layers
    int32_t* tok[kMaxLayers] = {};
    uint32_t* err = nullptr;
    unsigned long long* stats = nullptr;    // caller's per-request counters, or null (hisparse_set_stats)
    bool in_scratch = false;                // state lives in the static scratch array (hisparse_init_static)
};

namespace {

int hip_rc(hipError_t e) { return e == hipSuccess ? HISPARSE_OK : HISPARSE_EHIP(e); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The host pool must be pinned host memory the GPU can address; returns the
// device-side address of `p`, or null.
const uint8_t* device_view_of_host(void* p, size_t bytes)
{
    hipPointerAttribute_t at;
    if (hipPointerGetAttributes(&at, p) != hipSuccess) { (void)hipGetLastError(); return nullptr; }
    if (at.type != hipMemoryTypeHost || at.devicePointer == nullptr) return nullptr;
    hipPointerAttribute_t at2;
    void* last = static_cast<uint8_t*>(p) + bytes - 1;
    if (hipPointerGetAttributes(&at2, last) != hipSuccess) { (void)hipGetLastError(); return nullptr; }
    if (at2.type != hipMemoryTypeHost || at2.devicePointer == nullptr) return nullptr;
    if (static_cast<uint8_t*>(at2.devicePointer) - static_cast<uint8_t*>(at.devicePointer) != ptrdiff_t(bytes - 1))
        return nullptr;
    return static_cast<const uint8_t*>(at.devicePointer);
}

bool is_device_memory(void* p, size_t bytes)
{
    hipPointerAttribute_t at;
    if (hipPointerGetAttributes(&at, p) != hipSuccess) { (void)hipGetLastError(); return false; }
    if (at.type != hipMemoryTypeDevice) return false;
    void* last = static_cast<uint8_t*>(p) + bytes - 1;
    if (hipPointerGetAttributes(&at, last) != hipSuccess) { (void)hipGetLastError(); return false; }
    return at.type == hipMemoryTypeDevice;
}

// A context is used on the device that was current at init: any other
// current device would launch its kernels with another device's pointers.
bool usable(const hisparse_ctx* c)
{
    int d = -1;
    if (!c || hipGetDevice(&d) != hipSuccess) return false;
    return d == c->device;
}

bool is_anchor(const hisparse_ctx* c, int32_t l)
{
    return l >= 0 && l < c->layers && c->anchor_of[l] == l;
}

// hisparse_init_static keeps the library-owned device memory of one context
// per device (each anchor layer's LRU list and slot map, and the error word)
// in the file-scope array `scratch` below instead of memory from hipMalloc,
// and the context object itself in a static slot, so that call allocates
// nothing.  In host code the array's name only stands for the symbol: its
// address on a device is looked up once, with that device current
// (hipGetSymbolAddress), kept in the device's slot, and only that address is
// used.
constexpr size_t kScratchBytes = size_t(32) << 20;   // 32 MiB per device, held until the process ends
constexpr size_t kScratchAlign = 256;
constexpr int kMaxDevices = 64;

struct ScratchSlot {
    uint8_t* ptr = nullptr;   // device address of `scratch` on this device, once looked up
    bool busy = false;        // a live context of hisparse_init_static uses it
    hisparse_ctx ctx;         // that context
};
ScratchSlot g_slots[kMaxDevices];
std::mutex g_slots_mu;

size_t scratch_align(size_t x) { return (x + kScratchAlign - 1) & ~(kScratchAlign - 1); }

void release_static(hisparse_ctx* c)
{
    std::lock_guard<std::mutex> lk(g_slots_mu);
    for (ScratchSlot& s : g_slots)
        if (&s.ctx == c) s.busy = false;
}

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

extern "C" {

int hisparse_version(void) { return 1; }

size_t hisparse_swap_in_lds_bytes(int32_t top_k, int32_t device_buffer_size)
{
    if (top_k <= 0 || device_buffer_size <= 0) return 0;
    return swap_in_lds_bytes_impl(device_buffer_size, top_k,
                                  hash_bits_for(top_k, device_buffer_size, kGfx950LdsPerWorkgroup));
}

const char* hisparse_strerror(int code)
{
    if (code == HISPARSE_OK) return "ok";
    if (code == HISPARSE_EINVAL) return "invalid argument";
    if (code == HISPARSE_ENOMEM) return "out of memory";
    if (code == HISPARSE_EBUSY) return "the device's static scratch is in use by another context";
    if (code == HISPARSE_ENOSPC) return "the configuration's state does not fit the static scratch array";
    if (code <= -1000) return hipGetErrorString(static_cast<hipError_t>(-code - 1000));
    return "unknown error";
}

int hisparse_host_alloc(size_t bytes, uint32_t flags, void** out)
{
    if (!out || bytes == 0 || (flags & ~3u) || flags == 3u) return HISPARSE_EINVAL;
    unsigned hf = hipHostMallocMapped | hipHostMallocPortable;
    if (flags == HISPARSE_HOST_COHERENT) hf |= hipHostMallocCoherent;
    if (flags == HISPARSE_HOST_NONCOHERENT) hf |= hipHostMallocNonCoherent;
    void* p = nullptr;
    hipError_t e = hipHostMalloc(&p, bytes, hf);
    if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation) { (void)hipGetLastError(); return HISPARSE_ENOMEM; }
    if (e != hipSuccess) { (void)hipGetLastError(); return HISPARSE_EHIP(e); }
    *out = p;
    return HISPARSE_OK;
}

int hisparse_host_free(void* p)
{
    if (!p) return HISPARSE_OK;
    return hip_rc(hipHostFree(p));
}

namespace {

// Everything hisparse_init and hisparse_init_static share: the checks of the
// configuration and of the memory it names, the kernel instantiation and its
// LDS, all filled into *c.  No device memory is allocated here.
int init_common(const hisparse_config* cfg, hisparse_ctx* c)
{
    const int K = cfg->top_k, B = cfg->device_buffer_size;
    if (K < 1 || B < 1 || K > B || B > kMaxB || K > kMaxK) return HISPARSE_EINVAL;
    if (cfg->num_layers < 1 || cfg->num_layers > kMaxLayers || cfg->max_requests < 1 || cfg->max_seq_len < 1)
        return HISPARSE_EINVAL;
    if (cfg->row_bytes < 16 || cfg->row_bytes % 16) return HISPARSE_EINVAL;
    if (!cfg->host_pool || !cfg->hot_buffer || !cfg->anchor_of) return HISPARSE_EINVAL;
    int block = cfg->block_size ? cfg->block_size : kDefaultBlock;
    if (block < 128 || block > 1024 || block % kWave) return HISPARSE_EINVAL;
    int replay_grid = cfg->replay_grid ? cfg->replay_grid : kDefaultReplayGrid;
    if (replay_grid < 1 || replay_grid > 65535) return HISPARSE_EINVAL;
    const size_t host_bytes = size_t(cfg->max_requests) * cfg->max_seq_len * cfg->row_bytes;
    const size_t hot_bytes = size_t(cfg->max_requests) * (B + 1) * size_t(cfg->row_bytes);
    if (size_t(cfg->max_requests) * cfg->max_seq_len > size_t(INT32_MAX) * 64) return HISPARSE_EINVAL;
    // the replay stages absolute hot rows r * (B + 1) + slot as int32
    if (size_t(cfg->max_requests) * (size_t(B) + 1) > size_t(INT32_MAX)) return HISPARSE_EINVAL;

    c->K = K; c->B = B; c->layers = cfg->num_layers; c->R = cfg->max_requests;
    c->max_seq = cfg->max_seq_len; c->rb = cfg->row_bytes;
    c->block = block; c->replay_grid = replay_grid;
    for (int l = 0; l < c->layers; ++l) c->anchor_of[l] = cfg->anchor_of[l];

    for (int l = 0; l < c->layers; ++l) {
        const int g = c->anchor_of[l];
        if (g < 0 || g >= c->layers || c->anchor_of[g] != g) return HISPARSE_EINVAL;
        void* hp = cfg->host_pool[l];
        void* dp = cfg->hot_buffer[l];
        if (!hp || !dp || !aligned16(hp) || !aligned16(dp)) return HISPARSE_EINVAL;
        const uint8_t* dv = device_view_of_host(hp, host_bytes);
        if (!dv || !aligned16(dv)) return HISPARSE_EINVAL;
        if (!is_device_memory(dp, hot_bytes)) return HISPARSE_EINVAL;
        c->host[l] = dv;
        c->host_ptr[l] = static_cast<uint8_t*>(hp);
        c->hot[l] = static_cast<uint8_t*>(dp);
    }
    if (hipGetDevice(&c->device) != hipSuccess) return HISPARSE_EHIP(hipGetLastError());

    const int nwaves = block / kWave;
    const int eb = ((B + 63) / 64 + nwaves - 1) / nwaves;
    const int ek = ((K + 63) / 64 + nwaves - 1) / nwaves;
    c->swap_in_fn[0] = pick_kernel(eb, ek, false);
    c->swap_in_fn[1] = pick_kernel(eb, ek, true);
    if (!c->swap_in_fn[0] || !c->swap_in_fn[1]) return HISPARSE_EINVAL;
    int max_lds = 0;
    if (hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, c->device) != hipSuccess)
        return HISPARSE_EHIP(hipGetLastError());
    c->hash_bits = hash_bits_for(K, B, size_t(max_lds));
    c->lds = swap_in_lds_bytes_impl(B, K, c->hash_bits);
    if (c->lds > size_t(max_lds)) return HISPARSE_EINVAL;
    const size_t rlds = replay_lds_bytes(c->R) + 16 * sizeof(int);
    if (rlds > size_t(max_lds)) return HISPARSE_EINVAL;
    if (rlds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&replay_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, int(replay_lds_bytes(c->R)));
        if (e != hipSuccess) return HISPARSE_EHIP(e);
    }
    if (c->lds > 64 * 1024) {
        for (SwapInFn fn : c->swap_in_fn) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, int(c->lds));
            if (e != hipSuccess) return HISPARSE_EHIP(e);
        }
    }
    return HISPARSE_OK;
}

// Every anchor layer's state as if each request were admitted with a prompt
// longer than B, and a clear error word; on the null stream, then waited for.
int reset_state(hisparse_ctx* c)
{
    for (int l = 0; l < c->layers; ++l) {
        if (!is_anchor(c, l)) continue;
        hipLaunchKernelGGL(init_state_kernel, dim3(1024), dim3(256), 0, nullptr, c->lru[l], c->tok[l], c->R, c->B);
    }
    hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(64), 0, nullptr, c->err);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = hipDeviceSynchronize();
    return hip_rc(e);
}

}  // namespace

int hisparse_init(const hisparse_config* cfg, hisparse_ctx** out)
{
    if (!cfg || !out) return HISPARSE_EINVAL;
    *out = nullptr;
    hisparse_ctx* c = new (std::nothrow) hisparse_ctx;
    if (!c) return HISPARSE_ENOMEM;
    auto fail = [&](int rc) { hisparse_destroy(c); return rc; };
    const int rc = init_common(cfg, c);
    if (rc != HISPARSE_OK) return fail(rc);

    const size_t state_bytes = size_t(c->R) * c->B * sizeof(int32_t);
    for (int l = 0; l < c->layers; ++l) {
        if (!is_anchor(c, l)) continue;   // skip layers share their anchor's state
        hipError_t e1 = hipMalloc(&c->lru[l], state_bytes);
        hipError_t e2 = e1 == hipSuccess ? hipMalloc(&c->tok[l], state_bytes) : e1;
        if (e1 != hipSuccess || e2 != hipSuccess) { (void)hipGetLastError(); return fail(HISPARSE_ENOMEM); }
    }
    if (hipMalloc(&c->err, sizeof(uint32_t)) != hipSuccess) { (void)hipGetLastError(); return fail(HISPARSE_ENOMEM); }
    const int rs = reset_state(c);
    if (rs != HISPARSE_OK) return fail(rs);
    *out = c;
    return HISPARSE_OK;
}

int hisparse_init_static(const hisparse_config* cfg, hisparse_ctx** out)
{
    if (!cfg || !out) return HISPARSE_EINVAL;
    *out = nullptr;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return HISPARSE_EHIP(hipGetLastError());
    if (dev < 0 || dev >= kMaxDevices) return HISPARSE_EINVAL;
    std::lock_guard<std::mutex> lk(g_slots_mu);
    ScratchSlot& slot = g_slots[dev];
    if (slot.busy) return HISPARSE_EBUSY;
    if (!slot.ptr) {
        void* p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) { (void)hipGetLastError(); return HISPARSE_EHIP(e); }
        if (!p) return HISPARSE_EHIP(hipErrorInvalidSymbol);
        slot.ptr = static_cast<uint8_t*>(p);
    }
    hisparse_ctx* c = &slot.ctx;
    *c = hisparse_ctx{};
    int rc = init_common(cfg, c);
    if (rc != HISPARSE_OK) return rc;
    // layout: error word, then each anchor layer's lru and slot map
    const size_t state = scratch_align(size_t(c->R) * c->B * sizeof(int32_t));
    size_t need = kScratchAlign;
    for (int l = 0; l < c->layers; ++l)
        if (is_anchor(c, l)) need += 2 * state;
    if (need > kScratchBytes) return HISPARSE_ENOSPC;
    uint8_t* p = slot.ptr;
    c->err = reinterpret_cast<uint32_t*>(p);
    p += kScratchAlign;
    for (int l = 0; l < c->layers; ++l) {
        if (!is_anchor(c, l)) continue;
        c->lru[l] = reinterpret_cast<int32_t*>(p);
        p += state;
        c->tok[l] = reinterpret_cast<int32_t*>(p);
        p += state;
    }
    c->in_scratch = true;
    // Work a previous context queued on other streams (which need not wait for
    // the null stream) may still use the array: let it finish first.
    if (hipDeviceSynchronize() != hipSuccess) return HISPARSE_EHIP(hipGetLastError());
    rc = reset_state(c);   // the array keeps the last context's contents: every byte used is written here
    if (rc != HISPARSE_OK) return rc;
    slot.busy = true;
    *out = c;
    return HISPARSE_OK;
}

size_t hisparse_static_scratch_bytes(void) { return kScratchBytes; }

void hisparse_destroy(hisparse_ctx* c)
{
    if (!c) return;
    if (c->in_scratch) {   // hisparse_init_static: nothing to free, the device's scratch is released
        release_static(c);
        return;
    }
    for (int l = 0; l < kMaxLayers; ++l) {
        if (c->lru[l]) (void)hipFree(c->lru[l]);
        if (c->tok[l]) (void)hipFree(c->tok[l]);
    }
    if (c->err) (void)hipFree(c->err);
    delete c;
}

int hisparse_admit(hisparse_ctx* c, int32_t anchor_layer, const int32_t* req_ids, const int32_t* seq_len0,
                   int32_t n, hipStream_t stream)
{
    if (!usable(c) || !is_anchor(c, anchor_layer) || n < 0 || n > c->R) return HISPARSE_EINVAL;
    if (n == 0) return HISPARSE_OK;
    if (!req_ids || !seq_len0) return HISPARSE_EINVAL;
    hipLaunchKernelGGL(admit_state_kernel, dim3(n), dim3(256), 0, stream, c->lru[anchor_layer],
                       c->tok[anchor_layer], req_ids, seq_len0, c->R, c->B, c->max_seq, c->err);
    for (int l = 0; l < c->layers; ++l) {
        if (c->anchor_of[l] != anchor_layer) continue;
        hipLaunchKernelGGL(admit_fill_kernel, dim3(n, 64), dim3(256), 0, stream, c->host[l], c->hot[l],
                           req_ids, seq_len0, c->R, c->B, c->rb, c->max_seq);
    }
    return hip_rc(hipGetLastError());
}

int hisparse_store_newest(hisparse_ctx* c, int32_t layer, const void* new_rows, const int32_t* seq_lens,
                          const uint8_t* resident_mask, const int32_t* req_idx, int32_t nb, hipStream_t stream)
{
    if (!usable(c) || layer < 0 || layer >= c->layers || nb < 0 || nb > c->R) return HISPARSE_EINVAL;
    if (nb == 0) return HISPARSE_OK;
    if (!new_rows || !seq_lens || !aligned16(new_rows)) return HISPARSE_EINVAL;
    RowArgs a{};
    a.seq_lens = seq_lens; a.resident = resident_mask; a.req_idx = req_idx;
    a.src = static_cast<const uint8_t*>(new_rows); a.hot = c->hot[layer]; a.err = c->err;
    a.nb = nb; a.R = c->R; a.B = c->B; a.rb = c->rb; a.max_seq = c->max_seq;
    hipLaunchKernelGGL(store_newest_kernel, dim3(nb), dim3(64), 0, stream, a);
    return hip_rc(hipGetLastError());
}

namespace {

int launch_swap_in(hisparse_ctx* c, int32_t anchor_layer, const int32_t* topk_idx, const int32_t* seq_lens,
                   const uint8_t* resident_mask, const int32_t* req_idx, int32_t nb, int32_t* out,
                   hisparse_plan plan_row, const int32_t* block_table, int32_t paged, int32_t max_pages,
                   int32_t page_size, int32_t hot_row_base, const void* new_rows, bool backup,
                   hipStream_t stream)
{
    if (!usable(c) || !is_anchor(c, anchor_layer) || nb < 0 || nb > c->R) return HISPARSE_EINVAL;
    if (nb == 0) return HISPARSE_OK;
    if (!topk_idx || !seq_lens || !out || !plan_row.pos || !plan_row.slot || !plan_row.count)
        return HISPARSE_EINVAL;
    SwapInArgs a{};
    a.topk = topk_idx; a.seq_lens = seq_lens; a.resident = resident_mask; a.req_idx = req_idx;
    a.out = out; a.plan_pos = plan_row.pos; a.plan_slot = plan_row.slot; a.plan_count = plan_row.count;
    a.lru = c->lru[anchor_layer]; a.tok = c->tok[anchor_layer];
    a.host = c->host[anchor_layer]; a.hot = c->hot[anchor_layer]; a.err = c->err;
    a.R = c->R; a.B = c->B; a.K = c->K; a.rb = c->rb; a.max_seq = c->max_seq; a.hash_bits = c->hash_bits;
    a.block_table = block_table; a.paged = paged; a.max_pages = max_pages; a.page_size = page_size;
    a.hot_row_base = hot_row_base;
    a.new_rows = static_cast<const uint8_t*>(new_rows);
    a.backup_host = backup ? const_cast<uint8_t*>(c->host[anchor_layer]) : nullptr;
    a.stats = c->stats;
    void* args[] = {&a};
    return hip_rc(hipLaunchKernel(reinterpret_cast<const void*>(c->swap_in_fn[c->stats ? 1 : 0]), dim3(nb),
                                  dim3(c->block), args, c->lds, stream));
}

}  // namespace

int hisparse_swap_in(hisparse_ctx* c, int32_t anchor_layer, const int32_t* topk_idx, const int32_t* seq_lens,
                     const uint8_t* resident_mask, const int32_t* req_idx, int32_t nb, int32_t* out_slots,
                     hisparse_plan plan_row, hipStream_t stream)
{
    return launch_swap_in(c, anchor_layer, topk_idx, seq_lens, resident_mask, req_idx, nb, out_slots, plan_row,
                          nullptr, 0, 0, 1, 0, nullptr, false, stream);
}

int hisparse_store_swap_in(hisparse_ctx* c, int32_t anchor_layer, const void* new_rows, const int32_t* topk_idx,
                           const int32_t* seq_lens, const uint8_t* resident_mask, const int32_t* req_idx,
                           int32_t nb, int32_t* out_slots, hisparse_plan plan_row, hipStream_t stream)
{
    if (!new_rows || !aligned16(new_rows)) return HISPARSE_EINVAL;
    return launch_swap_in(c, anchor_layer, topk_idx, seq_lens, resident_mask, req_idx, nb, out_slots, plan_row,
                          nullptr, 0, 0, 1, 0, new_rows, false, stream);
}

int hisparse_store_swap_in_backup(hisparse_ctx* c, int32_t anchor_layer, const void* new_rows,
                                  const int32_t* topk_idx, const int32_t* seq_lens, const uint8_t* resident_mask,
                                  const int32_t* req_idx, int32_t nb, int32_t* out_slots, hisparse_plan plan_row,
                                  hipStream_t stream)
{
    if (!new_rows || !aligned16(new_rows)) return HISPARSE_EINVAL;
    return launch_swap_in(c, anchor_layer, topk_idx, seq_lens, resident_mask, req_idx, nb, out_slots, plan_row,
                          nullptr, 0, 0, 1, 0, new_rows, true, stream);
}

namespace {

bool paged_args_ok(const hisparse_ctx* c, const int32_t* block_table, int32_t max_pages, int32_t page_size,
                   int32_t hot_row_base)
{
    if (!usable(c) || page_size < 1 || max_pages < 0 || (max_pages > 0 && !block_table) || hot_row_base < 0)
        return false;
    return static_cast<long long>(hot_row_base) + static_cast<long long>(c->R) * (c->B + 1) <= INT_MAX;
}

}  // namespace

int hisparse_swap_in_paged(hisparse_ctx* c, int32_t anchor_layer, const int32_t* topk_idx, const int32_t* seq_lens,
                           const int32_t* block_table, int32_t max_pages, int32_t page_size, int32_t hot_row_base,
                           const int32_t* req_idx, int32_t nb, int32_t* out_rows, hisparse_plan plan_row,
                           hipStream_t stream)
{
    if (!paged_args_ok(c, block_table, max_pages, page_size, hot_row_base)) return HISPARSE_EINVAL;
    return launch_swap_in(c, anchor_layer, topk_idx, seq_lens, nullptr, req_idx, nb, out_rows, plan_row,
                          block_table, 1, max_pages, page_size, hot_row_base, nullptr, false, stream);
}

int hisparse_store_swap_in_paged_backup(hisparse_ctx* c, int32_t anchor_layer, const void* new_rows,
                                        const int32_t* topk_idx, const int32_t* seq_lens, const int32_t* block_table,
                                        int32_t max_pages, int32_t page_size, int32_t hot_row_base,
                                        const int32_t* req_idx, int32_t nb, int32_t* out_rows,
                                        hisparse_plan plan_row, hipStream_t stream)
{
    if (!paged_args_ok(c, block_table, max_pages, page_size, hot_row_base)) return HISPARSE_EINVAL;
    if (!new_rows || !aligned16(new_rows)) return HISPARSE_EINVAL;
    return launch_swap_in(c, anchor_layer, topk_idx, seq_lens, nullptr, req_idx, nb, out_rows, plan_row,
                          block_table, 1, max_pages, page_size, hot_row_base, new_rows, true, stream);
}

int hisparse_replay_plan(hisparse_ctx* c, int32_t skip_layer, hisparse_plan plan_row, const int32_t* req_idx,
                         int32_t nb, hipStream_t side_stream)
{
    if (!usable(c) || skip_layer < 0 || skip_layer >= c->layers || nb < 0 || nb > c->R) return HISPARSE_EINVAL;
    if (nb == 0) return HISPARSE_OK;
    if (!plan_row.pos || !plan_row.slot || !plan_row.count) return HISPARSE_EINVAL;
    ReplayArgs a{};
    a.pos = plan_row.pos; a.slot = plan_row.slot; a.count = plan_row.count; a.req_idx = req_idx;
    a.host = c->host[skip_layer]; a.hot = c->hot[skip_layer]; a.err = c->err;
    a.nb = nb; a.R = c->R; a.B = c->B; a.K = c->K; a.rb = c->rb; a.max_seq = c->max_seq;
    hipLaunchKernelGGL(replay_kernel, dim3(c->replay_grid), dim3(256), replay_lds_bytes(nb), side_stream, a);
    return hip_rc(hipGetLastError());
}

namespace {

// 16 workgroups fill the host link (55.2 GB/s; 256 gave 54.1, 32 gave 55.4)
// and keep the fewest host writes in flight beside other work (measured)
#ifndef HISPARSE_PAGE_COPY_GRID
#define HISPARSE_PAGE_COPY_GRID 16
#endif
constexpr int kPageCopyGrid = HISPARSE_PAGE_COPY_GRID;

int launch_page_copy(hisparse_ctx* c, int32_t layer, const void* src, int32_t src_pages, int32_t page_size,
                     void* mirror, int32_t mirror_pages, const int32_t* transfers, int32_t n, hipStream_t stream)
{
    if (!usable(c) || layer < 0 || layer >= c->layers || n < 0 || page_size < 1 || src_pages < 0 || mirror_pages < 0)
        return HISPARSE_EINVAL;
    if (n == 0) return HISPARSE_OK;
    if (!src || !transfers || !aligned16(src) || (mirror_pages > 0 && (!mirror || !aligned16(mirror))))
        return HISPARSE_EINVAL;
    PageCopyArgs a{};
    a.src = static_cast<const uint8_t*>(src); a.host = const_cast<uint8_t*>(c->host[layer]);
    a.mirror = mirror_pages > 0 ? static_cast<uint8_t*>(mirror) : nullptr; a.transfers = transfers; a.err = c->err;
    a.src_pages = src_pages; a.mirror_pages = mirror_pages; a.n = n; a.R = c->R; a.max_seq = c->max_seq;
    a.rb = c->rb; a.P = page_size;
    hipLaunchKernelGGL(page_copy_kernel, dim3(n < kPageCopyGrid ? n : kPageCopyGrid), dim3(256), 0, stream, a);
    return hip_rc(hipGetLastError());
}

}  // namespace

namespace {

// Runtime-copy form of the page transfers.  The transfer list is host memory
// (the worker's own list of physical copy coordinates), checked whole before
// anything is issued; consecutive transfers that are contiguous on every side
// (same request, next host page, next source page, next mirror page or no
// mirror, previous page not cut at the pool end) merge into one run, and each
// run is one asynchronous runtime copy device -> pinned host (plus one device
// -> device copy into the mirror), with no kernel of this library.
int launch_page_copy_dma(hisparse_ctx* c, int32_t layer, const void* src, int32_t src_pages, int32_t page_size,
                         void* mirror, int32_t mirror_pages, const int32_t* transfers, int32_t n,
                         hipStream_t stream)
{
    if (!usable(c) || layer < 0 || layer >= c->layers || n < 0 || page_size < 1 || src_pages < 0 || mirror_pages < 0)
        return HISPARSE_EINVAL;
    if (n == 0) return HISPARSE_OK;
    if (!src || !transfers || (mirror_pages > 0 && !mirror)) return HISPARSE_EINVAL;
    const long long P = page_size;
    for (int32_t x = 0; x < n; ++x) {
        const int32_t* t = transfers + 4 * size_t(x);
        const bool ok = t[0] >= 0 && t[0] < src_pages && t[1] >= 0 && t[1] < c->R && t[2] >= 0 &&
                        t[2] * P < c->max_seq && t[3] >= -1 && t[3] < mirror_pages;
        if (!ok) return HISPARSE_EINVAL;
    }
    const size_t rb = size_t(c->rb);
    const uint8_t* s8 = static_cast<const uint8_t*>(src);
    uint8_t* m8 = static_cast<uint8_t*>(mirror);
    for (int32_t x = 0; x < n;) {
        const int32_t* t0 = transfers + 4 * size_t(x);
        long long rows = 0;
        int32_t y = x;
        for (;; ++y) {
            const int32_t* t = transfers + 4 * size_t(y);
            const long long hp = t[2];
            const long long page_rows = c->max_seq - hp * P < P ? c->max_seq - hp * P : P;
            rows += page_rows;
            if (y + 1 >= n || page_rows < P) break;
            const int32_t* u = t + 4;
            const bool mirror_next = t[3] < 0 ? u[3] < 0 : u[3] == t[3] + 1;
            if (u[1] != t[1] || u[2] != t[2] + 1 || u[0] != t[0] + 1 || !mirror_next) break;
        }
        const size_t bytes = size_t(rows) * rb;
        const uint8_t* from = s8 + size_t(t0[0]) * size_t(P) * rb;
        uint8_t* to = c->host_ptr[layer] + (size_t(t0[1]) * size_t(c->max_seq) + size_t(t0[2]) * size_t(P)) * rb;
        // Which engine carries the copy (an SDMA engine or the runtime's own
        // blit kernel) is the HIP runtime's choice.
        hipError_t e = hipMemcpyAsync(to, from, bytes, hipMemcpyDeviceToHost, stream);
        if (e == hipSuccess && t0[3] >= 0)
            e = hipMemcpyAsync(m8 + size_t(t0[3]) * size_t(P) * rb, from, bytes, hipMemcpyDeviceToDevice, stream);
        if (e != hipSuccess) return HISPARSE_EHIP(e);
        x = y + 1;
    }
    return HISPARSE_OK;
}

}  // namespace

int hisparse_spill_dma(hisparse_ctx* c, int32_t layer, const void* resident_cache, int32_t resident_pages,
                       int32_t page_size, const int32_t* transfers, int32_t n, hipStream_t stream)
{
    return launch_page_copy_dma(c, layer, resident_cache, resident_pages, page_size, nullptr, 0, transfers, n,
                                stream);
}

int hisparse_import_dma(hisparse_ctx* c, int32_t layer, const void* staging, int32_t staging_pages,
                        int32_t page_size, void* resident_cache, int32_t resident_pages, const int32_t* transfers,
                        int32_t n, hipStream_t stream)
{
    return launch_page_copy_dma(c, layer, staging, staging_pages, page_size, resident_cache, resident_pages,
                                transfers, n, stream);
}

int hisparse_spill(hisparse_ctx* c, int32_t layer, const void* resident_cache, int32_t resident_pages,
                   int32_t page_size, const int32_t* transfers, int32_t n, hipStream_t stream)
{
    return launch_page_copy(c, layer, resident_cache, resident_pages, page_size, nullptr, 0, transfers, n, stream);
}

int hisparse_import(hisparse_ctx* c, int32_t layer, const void* staging, int32_t staging_pages, int32_t page_size,
                    void* resident_cache, int32_t resident_pages, const int32_t* transfers, int32_t n,
                    hipStream_t stream)
{
    return launch_page_copy(c, layer, staging, staging_pages, page_size, resident_cache, resident_pages, transfers,
                            n, stream);
}

int hisparse_backup(hisparse_ctx* c, int32_t layer, const int32_t* seq_lens, const uint8_t* resident_mask,
                    const int32_t* req_idx, int32_t nb, hipStream_t stream)
{
    if (!usable(c) || layer < 0 || layer >= c->layers || nb < 0 || nb > c->R) return HISPARSE_EINVAL;
    if (nb == 0) return HISPARSE_OK;
    if (!seq_lens) return HISPARSE_EINVAL;
    RowArgs a{};
    a.seq_lens = seq_lens; a.resident = resident_mask; a.req_idx = req_idx;
    a.host_c = c->hot[layer]; a.host = const_cast<uint8_t*>(c->host[layer]); a.err = c->err;
    a.nb = nb; a.R = c->R; a.B = c->B; a.rb = c->rb; a.max_seq = c->max_seq;
    hipLaunchKernelGGL(backup_kernel, dim3(nb), dim3(64), 0, stream, a);
    return hip_rc(hipGetLastError());
}

int hisparse_get_state(hisparse_ctx* c, int32_t anchor_layer, int32_t* lru, int32_t* slot_tok, hipStream_t stream)
{
    if (!usable(c) || !is_anchor(c, anchor_layer) || !lru || !slot_tok) return HISPARSE_EINVAL;
    const size_t bytes = size_t(c->R) * c->B * sizeof(int32_t);
    hipError_t e = hipMemcpyAsync(lru, c->lru[anchor_layer], bytes, hipMemcpyDeviceToDevice, stream);
    if (e == hipSuccess) e = hipMemcpyAsync(slot_tok, c->tok[anchor_layer], bytes, hipMemcpyDeviceToDevice, stream);
    return hip_rc(e);
}

int hisparse_set_state(hisparse_ctx* c, int32_t anchor_layer, const int32_t* lru, const int32_t* slot_tok,
                       hipStream_t stream)
{
    if (!usable(c) || !is_anchor(c, anchor_layer) || !lru || !slot_tok) return HISPARSE_EINVAL;
    const size_t bytes = size_t(c->R) * c->B * sizeof(int32_t);
    hipError_t e = hipMemcpyAsync(c->lru[anchor_layer], lru, bytes, hipMemcpyDeviceToDevice, stream);
    if (e == hipSuccess) e = hipMemcpyAsync(c->tok[anchor_layer], slot_tok, bytes, hipMemcpyDeviceToDevice, stream);
    return hip_rc(e);
}

int hisparse_set_stats(hisparse_ctx* c, uint64_t* stats)
{
    if (!usable(c)) return HISPARSE_EINVAL;
    if (stats && (reinterpret_cast<uintptr_t>(stats) & 7u)) return HISPARSE_EINVAL;
    c->stats = reinterpret_cast<unsigned long long*>(stats);
    return HISPARSE_OK;
}

int hisparse_get_error(hisparse_ctx* c, uint32_t* flags, int clear, hipStream_t stream)
{
    if (!usable(c) || !flags) return HISPARSE_EINVAL;
    hipError_t e = hipMemcpyAsync(flags, c->err, sizeof(uint32_t), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess && clear) e = hipMemsetAsync(c->err, 0, sizeof(uint32_t), stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    return hip_rc(e);
}

}  // extern "C"
