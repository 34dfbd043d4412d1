// Device half of libkvevict: the HIP kernels of the eviction step for gfx950 and
// the C-ABI entry points that validate and launch them.
//
// Pages: "Q-Filters — Query-Agnostic Projection Eviction" ("How it works",
// "Metal kernels", "Adaptation notes") and "L2Norm — Intrinsic Key-Norm
// Eviction" ("How it works").  The Metal design on the first page rescored all
// rows, sorted on the host side to find the keep threshold and compacted with
// one threadgroup per group; here only incoming rows are scored, the threshold
// is found by an on-chip radix select, and the copy runs as a separate
// bandwidth-shaped kernel over all groups at once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "kvevict.h"
#include "kvx_common.h"
#include "kvx_rows.h"

// The allocation-free selection's workspace (kv_evict_topk_noalloc): a fixed
// array in device memory that every GPU the library runs on holds until the
// process ends.  In host code its name stands for a host-side handle, not a
// device address, so host code only ever uses the address that
// scratch_address() looks up per device.
static __device__ __align__(256) uint32_t scratch[KVX_NOALLOC_SCRATCH_BYTES / 4];

namespace kvx {
namespace {

// Tuning knobs (compile-time): rows in flight per lane and cache hints.
#ifndef KVX_SCORE_U
#define KVX_SCORE_U 2
#endif
#ifndef KVX_GATHER_U
#define KVX_GATHER_U 1
#endif
#ifndef KVX_GATHER_BLOCK
#define KVX_GATHER_BLOCK 1024
#endif
#ifndef KVX_SCORE_BLOCK
#define KVX_SCORE_BLOCK 256
#endif
// Streaming (non-temporal) hints per kernel: the compaction and the decode
// shift touch their rows once per call, so they need not displace other data
// in the caches.  Scoring streams the keys too unless the caller asks for
// KVX_SCORE_CACHE_KEYS (the compaction will re-read many of them while they
// still fit the last-level cache).
#ifndef KVX_GATHER_NT_LOAD
#define KVX_GATHER_NT_LOAD 1
#endif
#ifndef KVX_GATHER_NT_STORE
#define KVX_GATHER_NT_STORE 1
#endif
#ifndef KVX_DECODE_NT
#define KVX_DECODE_NT 1
#endif
#ifndef KVX_DECODE_U
#define KVX_DECODE_U 12
#endif
#ifndef KVX_DECODE_BLOCK
#define KVX_DECODE_BLOCK 1024
#endif
#ifndef KVX_SELECT_NT
#define KVX_SELECT_NT 1024
#endif
// Score-and-append (calls that evict nothing): threads per block and rows in
// flight per lane (1024 and 1 measured fastest: the copy dominates).
#ifndef KVX_APPEND_BLOCK
#define KVX_APPEND_BLOCK 1024
#endif
#ifndef KVX_APPEND_U
#define KVX_APPEND_U 1
#endif
// Threads of the register-held selection for groups of up to 32 keys per
// thread at this block size (KVX_SELECT_NT above that).
#ifndef KVX_SELECT_SMALL_NT
#define KVX_SELECT_SMALL_NT 1024
#endif

// Checked build (-DKVX_CHECK): the selection and the compaction verify the
// index lists they write and read, and record the first violation in the
// caller's status words {code, group, row, value} (kvx_check_status_word);
// later violations are dropped.  Every access stays clamped as in the normal
// build, so a violation never makes a kernel leave its buffers.
#ifdef KVX_CHECK
constexpr bool kCheck = true;
#else
constexpr bool kCheck = false;
#endif

__device__ __forceinline__ void check_record(int32_t *chk, int code, int g, int row, int value) {
    if (chk != nullptr && atomicCAS(chk, 0, code) == 0) {
        chk[1] = g;
        chk[2] = row;
        chk[3] = value;
    }
}

// Status words of the checked build (set by kvx_check_status_word; always
// nullptr in the normal build, whose kernels do not check).
std::atomic<int32_t *> g_check_word{nullptr};
int32_t *check_word() { return kCheck ? g_check_word.load(std::memory_order_relaxed) : nullptr; }

// Order-preserving map of a score to an unsigned key, "higher key = better".
// keep_low ranks by -s.  -0 becomes +0 first so that the two tie.
__device__ __forceinline__ uint32_t select_key(float s, int keep_low) {
    float c = keep_low ? -s : s;
    c = c + 0.0f;
    const uint32_t b = __float_as_uint(c);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// ---------------------------------------------------------------------------
// Step 1: scoring.  A row is read by kLanes lanes, 16 bytes each (bf16: 16
// lanes, 4 rows per wave per load).  Each lane sums its elements in order with
// fused multiply-adds and the row's lanes combine by an xor butterfly; that
// order is a function of the row alone, so a row's score does not depend on S,
// on the tile it falls in or on the grid.  A lane always covers the same slice
// of the head dim, so its slice of the group's filter stays in registers.
// ---------------------------------------------------------------------------
template <int DT, int HD, int MODE>
__device__ __forceinline__ float row_partial(uint4 raw, const float *f) {
    using R = Row<DT, HD>;
    float x[R::kElemsPerLane];
    widen<DT>(raw, x);
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < R::kElemsPerLane; ++e)
        acc = MODE == KVX_SCORE_L2 ? __builtin_fmaf(x[e], x[e], acc) : __builtin_fmaf(x[e], f[e], acc);
#pragma unroll
    for (int off = R::kLanes / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    return acc;
}

template <int DT, int HD>
__device__ __forceinline__ void load_filter_slice(const float *__restrict__ filt, uint32_t l, uint32_t h,
                                                  uint32_t H, uint32_t part, float *f) {
    using R = Row<DT, HD>;
    const float4 *f4 = reinterpret_cast<const float4 *>(filt + (size_t)(l * H + h) * HD + part * R::kElemsPerLane);
#pragma unroll
    for (int q = 0; q < R::kElemsPerLane / 4; ++q) {
        const float4 v = f4[q];
        f[4 * q] = v.x;
        f[4 * q + 1] = v.y;
        f[4 * q + 2] = v.z;
        f[4 * q + 3] = v.w;
    }
}

__device__ __forceinline__ float finish_score(int mode, float acc, float sign) {
    const float s = mode == KVX_SCORE_L2 ? __builtin_sqrtf(acc) : sign * acc;
    return s + 0.0f;  // -0 -> +0
}

// Group-major tiles: block b scores rows [tile*RPB, tile*RPB + RPB) of group
// b / tiles (used when a group has at least a tile of rows).
template <int DT, int HD, int MODE, int U, bool NT>
__global__ __launch_bounds__(KVX_SCORE_BLOCK) void score_tile_kernel(
    const char *__restrict__ k, uint32_t S, uint32_t tiles, uint32_t BH, uint32_t H,
    const float *__restrict__ filt, float sign, float *__restrict__ out) {
    using R = Row<DT, HD>;
    constexpr int kRowsPerLoad = 64 / R::kLanes;
    constexpr int kRowsPerWave = kRowsPerLoad * U;
    const uint32_t g = blockIdx.x / tiles;
    const uint32_t tile = blockIdx.x - g * tiles;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t sub = lane / R::kLanes, part = lane % R::kLanes;
    const uint32_t r0 = tile * (KVX_SCORE_BLOCK / 64) * kRowsPerWave + (threadIdx.x >> 6) * kRowsPerWave;
    const char *kg = k + (size_t)g * S * R::kBytes;
    float f[R::kElemsPerLane];
    if constexpr (MODE == KVX_SCORE_PROJ) load_filter_slice<DT, HD>(filt, g / BH, g % H, H, part, f);
    uint4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t r = r0 + u * kRowsPerLoad + sub;
        raw[u] = r < S ? ld16<NT>(kg + (size_t)r * R::kBytes + part * 16) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t r = r0 + u * kRowsPerLoad + sub;
        const float acc = row_partial<DT, HD, MODE>(raw[u], f);
        if (part == 0 && r < S) out[(size_t)g * S + r] = finish_score(MODE, acc, sign);
    }
}

// Flat rows (a group has fewer rows than a tile, e.g. one decode token): row r
// belongs to group r / S.
template <int DT, int HD, int MODE, int U, bool NT>
__global__ __launch_bounds__(KVX_SCORE_BLOCK) void score_flat_kernel(
    const char *__restrict__ k, uint32_t n_rows, uint32_t S, uint32_t BH, uint32_t H,
    const float *__restrict__ filt, float sign, float *__restrict__ out) {
    using R = Row<DT, HD>;
    constexpr int kRowsPerLoad = 64 / R::kLanes;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t sub = lane / R::kLanes, part = lane % R::kLanes;
    const uint32_t wave = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const uint32_t row0 = wave * (kRowsPerLoad * U);
    uint4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t r = row0 + u * kRowsPerLoad + sub;
        raw[u] = r < n_rows ? ld16<NT>(k + (size_t)r * R::kBytes + part * 16) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t r = row0 + u * kRowsPerLoad + sub;
        float f[R::kElemsPerLane];
        if constexpr (MODE == KVX_SCORE_PROJ) {
            const uint32_t g = r < n_rows ? r / S : 0u;
            load_filter_slice<DT, HD>(filt, g / BH, g % H, H, part, f);
        }
        const float acc = row_partial<DT, HD, MODE>(raw[u], f);
        if (part == 0 && r < n_rows) out[r] = finish_score(MODE, acc, sign);
    }
}

// ---------------------------------------------------------------------------
// Wave-wide inclusive prefix sum on the DPP lane network (no LDS round trip):
// Hillis-Steele inside each row of 16 lanes, then the row totals are carried
// across rows with the row broadcasts.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_prefix_incl(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true);   // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true);   // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true);   // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true);   // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}

// ---------------------------------------------------------------------------
// Steps 2-3: selection.
//
// Every row of the concatenation gets an order-preserving u32 key: protected
// rows (the first n_sink, the last `recent`) get 0xFFFFFFFF, above every real
// score's key.  tau = the budget-th largest key is found by four 8-bit radix
// passes; the kept rows are those with key > tau plus the first `quota` rows
// (in row order) with key == tau, and their indices are written in row order
// from per-64-row chunk counts.
//
// Up to 32 * 1024 rows one workgroup per group holds every key in registers
// (select_kernel); up to KVX_ONCHIP_TOTAL rows one workgroup per group streams
// the keys from memory in chunks at every pass (select_stream_kernel; the
// scores stay in the caches between passes).  Beyond that, a group's rows are
// split over blocks of MB_ROWS rows and the passes meet in a small device
// workspace (histogram, state, block counts).
// ---------------------------------------------------------------------------
struct SelRows {
    const float *sk;  // stored scores of the group's kept rows
    const float *sn;  // scores of the group's incoming rows
    int n_kept, n_total, n_sink, recent, keep_low;
};

// Load the keys of rows r0 + i*NT + t, i < M (rows past n_total get key 0 and
// are never counted).  Every load is issued before any is used: rows past the
// end read the last row instead, and the source array is picked by address,
// so no branch separates the loads.
template <int M, int NT>
__device__ __forceinline__ void load_scores(const SelRows &a, int r0, float *s) {
#pragma unroll
    for (int i = 0; i < M; ++i) {
        const int r = min(r0 + i * NT + (int)threadIdx.x, a.n_total - 1);
        s[i] = *(r < a.n_kept ? a.sk + r : a.sn + (r - a.n_kept));
    }
}
template <int M, int NT>
__device__ __forceinline__ void make_keys(const SelRows &a, int r0, const float *s, uint32_t *key) {
#pragma unroll
    for (int i = 0; i < M; ++i) {
        const int r = r0 + i * NT + (int)threadIdx.x;
        const bool prot = r < a.n_sink || r >= a.n_total - a.recent;
        key[i] = r < a.n_total ? (prot ? 0xFFFFFFFFu : select_key(s[i], a.keep_low)) : 0u;
    }
}
template <int M, int NT>
__device__ __forceinline__ void load_keys(const SelRows &a, int r0, uint32_t *key) {
    float s[M];
    load_scores<M, NT>(a, r0, s);
    make_keys<M, NT>(a, r0, s, key);
}

// Count the digit (key >> shift) & 255 of every key that matches the prefix
// into this wave's 256-bin LDS histogram h.  In the first pass every key
// counts and scores cluster in a few top digits, so each lane first sums its
// own equal digits (eight keys at a time, plain vector compares) and adds
// each distinct digit once; in later passes few keys are left, spread over
// more digits, and each adds itself.  (Merging equal digits across a wave with
// ballots costs scalar instructions that the CU's 16 waves share, and was
// slower in both cases.)
template <int M, int NT>
__device__ __forceinline__ void count_digits(const uint32_t *key, int r0, int n_total, uint32_t prefix,
                                             uint32_t pmask, int shift, uint32_t *h) {
    if (pmask != 0) {
#pragma unroll
        for (int i = 0; i < M; ++i) {
            const int r = r0 + i * NT + (int)threadIdx.x;
            if (r < n_total && (key[i] & pmask) == prefix) atomicAdd(&h[(key[i] >> shift) & 0xFFu], 1u);
        }
        return;
    }
    constexpr int W = M < 8 ? M : 8;
#pragma unroll
    for (int w0 = 0; w0 < M; w0 += W) {
        uint32_t d[W];
        bool act[W];
#pragma unroll
        for (int i = 0; i < W; ++i) {
            act[i] = r0 + (w0 + i) * NT + (int)threadIdx.x < n_total;
            d[i] = (key[w0 + i] >> shift) & 0xFFu;
        }
#pragma unroll
        for (int i = 0; i < W; ++i) {
            uint32_t c = 1;
#pragma unroll
            for (int j = i + 1; j < W; ++j) {
                const bool same = act[i] && act[j] && d[j] == d[i];
                c += same;
                act[j] = act[j] && !same;
            }
            if (act[i]) atomicAdd(&h[d[i]], c);
        }
    }
}

// One wave: lane l holds the counts of bins 255-4l (c.w) down to 252-4l (c.x).
// Finds the bin where the krem-th largest key falls; the owning lane returns
// true and sets the digit, the remaining rank inside that bin and, if asked,
// whether that rank is the bin's last (every key of the bin is kept).
__device__ __forceinline__ bool pick_digit(uint4 c, uint32_t krem, uint32_t *digit, uint32_t *nk,
                                           uint32_t *whole = nullptr) {
    const int lane = threadIdx.x & 63;
    const uint32_t c0 = c.w, c1 = c.z, c2 = c.y, c3 = c.x;
    const uint32_t local = c0 + c1 + c2 + c3;
    const uint32_t incl = wave_prefix_incl(local);  // keys in this lane's bins or higher ones
    const uint32_t above = incl - local;
    if (!(above < krem && krem <= incl)) return false;
    uint32_t cum = above, cnt;
    if (cum + c0 >= krem) {
        *digit = 255 - 4 * lane;
        cnt = c0;
    } else if ((cum += c0) + c1 >= krem) {
        *digit = 254 - 4 * lane;
        cnt = c1;
    } else if ((cum += c1) + c2 >= krem) {
        *digit = 253 - 4 * lane;
        cnt = c2;
    } else {
        cum += c2;
        *digit = 252 - 4 * lane;
        cnt = c3;
    }
    *nk = krem - cum;
    if (whole) *whole = *nk == cnt;
    return true;
}

// Number of set bits of m in the lanes below this one (v_mbcnt).
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Write the kept rows among rows r0 + i*NT + t (i < M) in row order:
// out[base_gt + #(key > tau before) + min(base_eq + #(key == tau before), quota)].
// `chunk` holds M*NT/64 counters.  Ends with the block synchronised.
template <int M, int NT>
__device__ __forceinline__ void write_kept(const uint32_t *key, int r0, int n_total, uint32_t tau, uint32_t quota,
                                           uint32_t base_gt, uint32_t base_eq, int32_t *out, int budget,
                                           uint32_t *chunk, uint32_t *total, int32_t *chk) {
    constexpr int NW = NT / 64, NCH = M * NW, CPL = (NCH + 63) / 64;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
#pragma unroll
    for (int i = 0; i < M; ++i) {
        const int c = i * NW + w;
        const int r = r0 + c * 64 + lane;
        const bool valid = r < n_total;
        const uint64_t gm = __ballot(valid && key[i] > tau);
        const uint64_t em = __ballot(valid && key[i] == tau);
        if (lane == 0) chunk[c] = ((uint32_t)__popcll(gm) << 16) | (uint32_t)__popcll(em);
    }
    __syncthreads();
    if (w == 0) {  // exclusive scan of the packed (gt << 16 | eq) chunk counts
        uint32_t a[CPL], local = 0;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = CPL * lane + j;
            a[j] = c < NCH ? chunk[c] : 0u;
            local += a[j];
        }
        uint32_t run = wave_prefix_incl(local) - local;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = CPL * lane + j;
            if (c < NCH) chunk[c] = run;
            run += a[j];
        }
        if (total && lane == 63) *total = run;  // (#gt << 16) | #eq over all M * NT rows
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < M; ++i) {
        const int c = i * NW + w;
        const int r = r0 + c * 64 + lane;
        const bool valid = r < n_total;
        const bool gt = valid && key[i] > tau, eq = valid && key[i] == tau;
        const uint32_t base = chunk[c];
        const uint32_t gb = base_gt + (base >> 16) + lanes_below(__ballot(gt));
        const uint32_t eb = base_eq + (base & 0xFFFFu) + lanes_below(__ballot(eq));
        // Exactly `budget` rows qualify, so every slot is below budget; the
        // bound check only keeps a corrupt input from writing past the row.
        uint32_t slot = 0xFFFFFFFFu;
        if (gt)
            slot = gb + min(eb, quota);
        else if (eq && eb < quota)
            slot = gb + eb;
        if (slot < (uint32_t)budget)
            out[slot] = r;
        else if constexpr (kCheck)
            if (slot != 0xFFFFFFFFu) check_record(chk, KVX_CHECK_SLOT, (int)blockIdx.x, r, (int)slot);
    }
    __syncthreads();
}

// One workgroup of NT threads per group; thread t holds the keys of rows
// t, t + NT, ... (M of them) in registers, so every load is coalesced.  All
// waves count into one LDS histogram: the LDS runs one wave's atomics at a
// time anyway, and what costs is many lanes of one instruction on one bin,
// which count_digits avoids where scores cluster.  The next pass's histogram
// is cleared while the current one is scanned.
template <int M, int NT>
__global__ __launch_bounds__(NT) void select_kernel(const float *__restrict__ s_kept,
                                                      const float *__restrict__ s_new, int n_kept,
                                                      int S, int budget, int n_sink, int recent,
                                                      int keep_low, int32_t *__restrict__ keep_idx,
                                                      int32_t *chk) {
    constexpr int NW = NT / 64;
    static_assert(NW >= 2, "wave 1 clears the histograms while wave 0 scans");
    const int g = blockIdx.x;
    const int t = threadIdx.x, w = t >> 6;
    const int n_total = n_kept + S;
    int32_t *out = keep_idx + (size_t)g * budget;
    if (n_total <= budget) {
        for (int r = t; r < n_total; r += NT) out[r] = r;
        return;
    }
    const SelRows rows{s_kept + (size_t)g * budget, s_new + (size_t)g * S, n_kept, n_total, n_sink, recent,
                       keep_low};

    __shared__ uint4 hist4[2][64];  // 256-bin histograms, two passes' worth
    __shared__ uint32_t sel[3], tot;
    __shared__ uint32_t chunk[M * NW];
    uint32_t(*hist)[256] = reinterpret_cast<uint32_t(*)[256]>(hist4);

    uint32_t key[M];
    load_keys<M, NT>(rows, 0, key);
    if (t < 64) hist4[0][t] = make_uint4(0, 0, 0, 0);
    __syncthreads();

    // After the four passes the prefix is the whole key: tau = prefix and
    // quota = krem.  A pass whose chosen bin is kept whole ends the passes
    // early: the kept rows are then exactly the keys >= the prefix, i.e. tau =
    // prefix - 1 with no quota.
    uint32_t prefix = 0, pmask = 0, krem = (uint32_t)budget;
    uint32_t tau = 0, quota = 0;
    bool whole = false;
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        count_digits<M, NT>(key, 0, n_total, prefix, pmask, shift, hist[pass & 1]);
        __syncthreads();
        if (w == 0) {
            const uint4 c = hist4[pass & 1][63 - t];
            uint32_t d, nk, all;
            if (pick_digit(c, krem, &d, &nk, &all)) {
                sel[0] = d;
                sel[1] = nk;
                sel[2] = all;
            }
        }
        if (pass < 3 && w == 1)  // wave 1 clears the next pass's histogram meanwhile
            hist4[(pass + 1) & 1][t - 64] = make_uint4(0, 0, 0, 0);
        __syncthreads();
        prefix |= sel[0] << shift;
        pmask |= 0xFFu << shift;
        krem = sel[1];
        if (pass < 3 && sel[2] && prefix != 0) {  // the same in every thread
            whole = true;
            break;
        }
    }
    if (whole) {
        tau = prefix - 1;
        quota = 0;
    } else {
        tau = prefix;
        quota = krem;
    }
    write_kept<M, NT>(key, 0, n_total, tau, quota, 0, 0, out, budget, chunk, &tot, chk);
    if constexpr (kCheck) {  // exactly `budget` rows kept
        const uint32_t kept = (tot >> 16) + min(tot & 0xFFFFu, quota);
        if (t == 0 && kept != (uint32_t)budget) check_record(chk, KVX_CHECK_COUNT, g, -1, (int)kept);
    }
}

// One workgroup of NT threads per group for n_total up to KVX_ONCHIP_TOTAL:
// every pass streams the group's keys in chunks of MS * NT rows through
// registers (the same counting, picking and early end as select_kernel), and
// the kept rows are written chunk by chunk in row order, each chunk's slots
// offset by the counts of the chunks before it.  Two score buffers are used
// in turn, so that a chunk's loads are in flight while the one before it is
// counted or written.
template <int MS, int NT>
__global__ __launch_bounds__(NT) void select_stream_kernel(const float *__restrict__ s_kept,
                                                             const float *__restrict__ s_new, int n_kept,
                                                             int S, int budget, int n_sink, int recent,
                                                             int keep_low, int32_t *__restrict__ keep_idx,
                                                             int32_t *chk) {
    constexpr int NW = NT / 64, CHUNK = MS * NT;
    static_assert(NW >= 2, "wave 1 clears the histograms while wave 0 scans");
    static_assert(CHUNK < 65536, "per-chunk counts are packed in 16 bits");
    const int g = blockIdx.x;
    const int t = threadIdx.x, w = t >> 6;
    const int n_total = n_kept + S;
    int32_t *out = keep_idx + (size_t)g * budget;
    if (n_total <= budget) {
        for (int r = t; r < n_total; r += NT) out[r] = r;
        return;
    }
    const SelRows rows{s_kept + (size_t)g * budget, s_new + (size_t)g * S, n_kept, n_total, n_sink, recent,
                       keep_low};
    __shared__ uint4 hist4[2][64];
    __shared__ uint32_t sel[3], tot;
    __shared__ uint32_t chunk[MS * NW];
    uint32_t(*hist)[256] = reinterpret_cast<uint32_t(*)[256]>(hist4);
    if (t < 64) hist4[0][t] = make_uint4(0, 0, 0, 0);
    __syncthreads();

    uint32_t prefix = 0, pmask = 0, krem = (uint32_t)budget;
    bool whole = false;
    uint32_t key[MS];
    float sa[MS], sb[MS];
#pragma unroll 1
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        load_scores<MS, NT>(rows, 0, sa);
        for (int r0 = 0; r0 < n_total; r0 += 2 * CHUNK) {
            make_keys<MS, NT>(rows, r0, sa, key);
            if (r0 + CHUNK < n_total) load_scores<MS, NT>(rows, r0 + CHUNK, sb);
            count_digits<MS, NT>(key, r0, n_total, prefix, pmask, shift, hist[pass & 1]);
            if (r0 + CHUNK >= n_total) break;
            make_keys<MS, NT>(rows, r0 + CHUNK, sb, key);
            if (r0 + 2 * CHUNK < n_total) load_scores<MS, NT>(rows, r0 + 2 * CHUNK, sa);
            count_digits<MS, NT>(key, r0 + CHUNK, n_total, prefix, pmask, shift, hist[pass & 1]);
        }
        __syncthreads();
        if (w == 0) {
            const uint4 c = hist4[pass & 1][63 - t];
            uint32_t d, nk, all;
            if (pick_digit(c, krem, &d, &nk, &all)) {
                sel[0] = d;
                sel[1] = nk;
                sel[2] = all;
            }
        }
        if (pass < 3 && w == 1) hist4[(pass + 1) & 1][t - 64] = make_uint4(0, 0, 0, 0);
        __syncthreads();
        prefix |= sel[0] << shift;
        pmask |= 0xFFu << shift;
        krem = sel[1];
        if (pass < 3 && sel[2] && prefix != 0) {  // the same in every thread
            whole = true;
            break;
        }
    }
    const uint32_t tau = whole ? prefix - 1 : prefix, quota = whole ? 0u : krem;
    uint32_t base_gt = 0, base_eq = 0;
    auto write_chunk = [&](int r0) {
        write_kept<MS, NT>(key, r0, n_total, tau, quota, base_gt, base_eq, out, budget, chunk, &tot, chk);
        const uint32_t c = tot;  // written before write_kept's last barrier
        base_gt += c >> 16;
        base_eq += c & 0xFFFFu;
        __syncthreads();  // tot and chunk are rewritten by the next chunk
    };
    load_scores<MS, NT>(rows, 0, sa);
    for (int r0 = 0; r0 < n_total; r0 += 2 * CHUNK) {
        make_keys<MS, NT>(rows, r0, sa, key);
        if (r0 + CHUNK < n_total) load_scores<MS, NT>(rows, r0 + CHUNK, sb);
        write_chunk(r0);
        if (r0 + CHUNK >= n_total) break;
        make_keys<MS, NT>(rows, r0 + CHUNK, sb, key);
        if (r0 + 2 * CHUNK < n_total) load_scores<MS, NT>(rows, r0 + 2 * CHUNK, sa);
        write_chunk(r0 + CHUNK);
    }
    if constexpr (kCheck) {  // exactly `budget` rows kept
        const uint32_t kept = base_gt + min(base_eq, quota);
        if (t == 0 && kept != (uint32_t)budget) check_record(chk, KVX_CHECK_COUNT, g, -1, (int)kept);
    }
}

// --- multi-block selection (n_total above the on-chip bound) --------------
// Workspace per group g: hist[256] | state[4] = {prefix, pmask, krem, -} |
// counts[W][2] = {#key > tau, #key == tau} of each of the W row blocks.
constexpr int MB_NT = 1024, MB_M = 16, MB_ROWS = MB_NT * MB_M;

__host__ __device__ __forceinline__ size_t mb_words(int W) { return 256 + 4 + 2 * (size_t)W; }

__global__ __launch_bounds__(256) void mb_init_kernel(uint32_t *__restrict__ ws, int W, int budget) {
    uint32_t *h = ws + (size_t)blockIdx.x * mb_words(W);
    h[threadIdx.x] = 0;
    if (threadIdx.x < 4) h[256 + threadIdx.x] = threadIdx.x == 2 ? (uint32_t)budget : 0u;
}

struct MbArgs {
    const float *s_kept, *s_new;
    int n_kept, S, budget, n_sink, recent, keep_low, W;
    uint32_t *ws;
    int32_t *chk;
};

__device__ __forceinline__ SelRows mb_rows(const MbArgs &a, int g) {
    return SelRows{a.s_kept + (size_t)g * a.budget, a.s_new + (size_t)g * a.S, a.n_kept, a.n_kept + a.S,
                   a.n_sink, a.recent, a.keep_low};
}

// Histogram of one radix pass over one row block, added into the group's
// workspace histogram.
__global__ __launch_bounds__(MB_NT) void mb_hist_kernel(MbArgs a, int shift) {
    const int g = blockIdx.x / a.W, blk = blockIdx.x - g * a.W;
    const int t = threadIdx.x;
    uint32_t *ws = a.ws + (size_t)g * mb_words(a.W);
    const uint32_t prefix = ws[256], pmask = ws[257];
    __shared__ uint32_t hist[256];
    if (t < 256) hist[t] = 0;
    __syncthreads();
    uint32_t key[MB_M];
    const SelRows rows = mb_rows(a, g);
    const int r0 = blk * MB_ROWS;
    load_keys<MB_M, MB_NT>(rows, r0, key);
    count_digits<MB_M, MB_NT>(key, r0, rows.n_total, prefix, pmask, shift, hist);
    __syncthreads();
    if (t < 256 && hist[t]) atomicAdd(&ws[t], hist[t]);
}

// One wave per group: choose the digit of this pass, advance the state and
// clear the histogram for the next pass.
__global__ __launch_bounds__(64) void mb_pick_kernel(uint32_t *__restrict__ ws_all, int W, int shift) {
    uint32_t *ws = ws_all + (size_t)blockIdx.x * mb_words(W);
    const int lane = threadIdx.x;
    uint4 c;
    c.x = ws[252 - 4 * lane];
    c.y = ws[253 - 4 * lane];
    c.z = ws[254 - 4 * lane];
    c.w = ws[255 - 4 * lane];
    const uint32_t krem = ws[258];
    uint32_t d, nk;
    const bool mine = pick_digit(c, krem, &d, &nk);
    for (int j = 0; j < 4; ++j) ws[252 - 4 * lane + j] = 0;  // each lane clears only the bins it read
    if (mine) {
        ws[256] |= d << shift;
        ws[257] |= 0xFFu << shift;
        ws[258] = nk;
    }
}

// Per row block: how many keys are above tau and equal to it.
__global__ __launch_bounds__(MB_NT) void mb_count_kernel(MbArgs a) {
    const int g = blockIdx.x / a.W, blk = blockIdx.x - g * a.W;
    const int t = threadIdx.x, lane = t & 63;
    uint32_t *ws = a.ws + (size_t)g * mb_words(a.W);
    const uint32_t tau = ws[256];
    __shared__ uint32_t tot[2];
    if (t < 2) tot[t] = 0;
    __syncthreads();
    uint32_t key[MB_M];
    const SelRows rows = mb_rows(a, g);
    const int r0 = blk * MB_ROWS;
    load_keys<MB_M, MB_NT>(rows, r0, key);
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < MB_M; ++i) {
        const int r = r0 + i * MB_NT + t;
        const bool valid = r < rows.n_total;
        gt += (uint32_t)__popcll(__ballot(valid && key[i] > tau));
        eq += (uint32_t)__popcll(__ballot(valid && key[i] == tau));
    }
    if (lane == 0) {
        atomicAdd(&tot[0], gt);
        atomicAdd(&tot[1], eq);
    }
    __syncthreads();
    if (t == 0) {
        ws[260 + 2 * blk] = tot[0];
        ws[260 + 2 * blk + 1] = tot[1];
    }
}

// Per row block: write the kept indices, offset by the counts of the blocks
// before it.
__global__ __launch_bounds__(MB_NT) void mb_write_kernel(MbArgs a, int32_t *__restrict__ keep_idx) {
    const int g = blockIdx.x / a.W, blk = blockIdx.x - g * a.W;
    const int t = threadIdx.x;
    const uint32_t *ws = a.ws + (size_t)g * mb_words(a.W);
    __shared__ uint32_t base[2];
    __shared__ uint32_t chunk[MB_M * (MB_NT / 64)];
    if (t < 2) {
        uint32_t s = 0;
        for (int b = 0; b < blk; ++b) s += ws[260 + 2 * b + t];
        base[t] = s;
    }
    uint32_t key[MB_M];
    const SelRows rows = mb_rows(a, g);
    const int r0 = blk * MB_ROWS;
    load_keys<MB_M, MB_NT>(rows, r0, key);
    __syncthreads();
    write_kept<MB_M, MB_NT>(key, r0, rows.n_total, ws[256], ws[258], base[0], base[1],
                            keep_idx + (size_t)g * a.budget, a.budget, chunk, nullptr, a.chk);
    if constexpr (kCheck) {  // exactly `budget` rows kept, over all row blocks
        if (blk == a.W - 1 && t == 0) {
            uint32_t n_gt = 0, n_eq = 0;
            for (int b = 0; b < a.W; ++b) {
                n_gt += ws[260 + 2 * b];
                n_eq += ws[260 + 2 * b + 1];
            }
            const uint32_t kept = n_gt + min(n_eq, ws[258]);
            if (kept != (uint32_t)a.budget) check_record(a.chk, KVX_CHECK_COUNT, g, -1, (int)kept);
        }
    }
}

// ---------------------------------------------------------------------------
// Steps 1-4 of a call that evicts nothing: every incoming row is kept, so it
// is scored and appended in the same pass and its key is read once.  A row is
// kLanes lanes x 16 B of K and of V; each lane reduces its K slice exactly as
// the scoring kernels do (same function, same order), so the stored score is
// the one qf_score_keys gives.  Blocks are group-major tiles of incoming rows.
// ---------------------------------------------------------------------------
template <int DT, int HD, int MODE, int U>
__global__ __launch_bounds__(KVX_APPEND_BLOCK) void score_append_kernel(
    const char *__restrict__ k_new, const char *__restrict__ v_new, uint32_t S, uint32_t tiles, uint32_t BH,
    uint32_t H, const float *__restrict__ filt, float sign, int32_t pos_base, uint32_t n_kept, uint32_t budget,
    char *__restrict__ k_cache, char *__restrict__ v_cache, float *__restrict__ s_cache,
    int32_t *__restrict__ pos_cache, float *__restrict__ s_new) {
    using R = Row<DT, HD>;
    constexpr int kRowsPerLoad = 64 / R::kLanes;
    constexpr int kRowsPerWave = kRowsPerLoad * U;
    const uint32_t g = blockIdx.x / tiles;
    const uint32_t tile = blockIdx.x - g * tiles;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t sub = lane / R::kLanes, part = lane % R::kLanes;
    const uint32_t r0 = tile * (KVX_APPEND_BLOCK / 64) * kRowsPerWave + (threadIdx.x >> 6) * kRowsPerWave + sub;
    const size_t in0 = (size_t)g * S, out0 = (size_t)g * budget + n_kept;
    float f[R::kElemsPerLane];
    if constexpr (MODE == KVX_SCORE_PROJ) load_filter_slice<DT, HD>(filt, g / BH, g % H, H, part, f);
    uint4 kr[U], vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t r = r0 + u * kRowsPerLoad;
        const size_t off = (in0 + r) * R::kBytes + part * 16;
        kr[u] = r < S ? ld16<true>(k_new + off) : make_uint4(0, 0, 0, 0);
        vr[u] = r < S ? ld16<true>(v_new + off) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t r = r0 + u * kRowsPerLoad;
        const float acc = row_partial<DT, HD, MODE>(kr[u], f);
        if (r < S) {
            const size_t off = (out0 + r) * R::kBytes + part * 16;
            st16<true>(k_cache + off, kr[u]);
            st16<true>(v_cache + off, vr[u]);
            if (part == 0) {
                const float sc = finish_score(MODE, acc, sign);
                s_cache[out0 + r] = sc;
                pos_cache[out0 + r] = pos_base + (int32_t)r;
                if (s_new) s_new[in0 + r] = sc;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Step 4: gather.  Output rows j in [j0, n_out) of every group; blocks are
// numbered group-major.  Each row is kLanes lanes x 16 B for K and the same for
// V; the lane with part == 0 also moves the score and the position.
// keep_idx == nullptr means the identity (nothing evicted).
// ---------------------------------------------------------------------------
template <int DT, int HD, int U>
__global__ __launch_bounds__(KVX_GATHER_BLOCK) void gather_kernel(
    const char *__restrict__ k_kept, const char *__restrict__ v_kept,
    const float *__restrict__ s_kept, const int32_t *__restrict__ pos_kept,
    const char *__restrict__ k_new, const char *__restrict__ v_new,
    const float *__restrict__ s_new, int32_t pos_base, const int32_t *__restrict__ keep_idx,
    int n_kept, int S, int budget, int j0, int n_out, int blocks_per_group, char *__restrict__ k_out,
    char *__restrict__ v_out, float *__restrict__ s_out, int32_t *__restrict__ pos_out, int32_t *chk) {
    using R = Row<DT, HD>;
    constexpr int kRowsPerPass = KVX_GATHER_BLOCK / R::kLanes;
    const int g = blockIdx.x / blocks_per_group;
    const int b = blockIdx.x - g * blocks_per_group;
    const int part = threadIdx.x % R::kLanes;
    const int sub = threadIdx.x / R::kLanes;
    const int jb = j0 + b * (kRowsPerPass * U);
    const size_t cache_row0 = (size_t)g * budget;
    const size_t new_row0 = (size_t)g * S;

    uint4 kr[U], vr[U];
    int src[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int j = jb + u * kRowsPerPass + sub;
        src[u] = -1;
        if (j < n_out) {
            int r = keep_idx ? keep_idx[cache_row0 + j] : j;
            if constexpr (kCheck) {
                if (part == 0 && (unsigned)r >= (unsigned)(n_kept + S)) check_record(chk, KVX_CHECK_RANGE, g, j, r);
                if (part == 0 && keep_idx && j > 0 && keep_idx[cache_row0 + j - 1] >= r)
                    check_record(chk, KVX_CHECK_ORDER, g, j, r);
            }
            if ((unsigned)r >= (unsigned)(n_kept + S)) r = 0;  // keep a corrupt index in bounds
            src[u] = r;
            const size_t off = r < n_kept ? (cache_row0 + r) * R::kBytes
                                          : (new_row0 + (r - n_kept)) * R::kBytes;
            const char *kb = r < n_kept ? k_kept : k_new;
            const char *vb = r < n_kept ? v_kept : v_new;
            kr[u] = ld16<KVX_GATHER_NT_LOAD>(kb + off + part * 16);
            vr[u] = ld16<KVX_GATHER_NT_LOAD>(vb + off + part * 16);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int j = jb + u * kRowsPerPass + sub;
        if (j < n_out) {
            const size_t off = (cache_row0 + j) * R::kBytes + part * 16;
            st16<KVX_GATHER_NT_STORE>(k_out + off, kr[u]);
            st16<KVX_GATHER_NT_STORE>(v_out + off, vr[u]);
            if (part == 0) {
                const int r = src[u];
                s_out[cache_row0 + j] = r < n_kept ? s_kept[cache_row0 + r] : s_new[new_row0 + (r - n_kept)];
                pos_out[cache_row0 + j] = r < n_kept ? pos_kept[cache_row0 + r] : pos_base + (r - n_kept);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Decode: one incoming row per group, in place.  One workgroup per group
// (KVX_DECODE_BLOCK threads).  The victim is the candidate with the smallest key, the higher row on
// equal keys (the last row in the general (key desc, row asc) order).  Rows
// after it move down one row in chunks of C rows: every thread loads its part
// of the chunk, waits for its loads to land, the workgroup meets at a barrier,
// then the chunk is stored one row lower.  A chunk only writes rows below the
// next chunk's sources, so chunk-by-chunk order makes the shift race-free.
// ---------------------------------------------------------------------------
template <int DT, int HD, int U>
__global__ __launch_bounds__(KVX_DECODE_BLOCK) void evict_one_kernel(
    char *__restrict__ k_cache, char *__restrict__ v_cache, float *__restrict__ s_cache,
    int32_t *__restrict__ pos_cache, const char *__restrict__ k_new, const char *__restrict__ v_new,
    const float *__restrict__ s_new, int32_t pos_base, int n_kept, int budget, int n_sink,
    int recent, int keep_low) {
    using R = Row<DT, HD>;
    constexpr int kSlots = 2 * R::kLanes;          // K lanes then V lanes of one row
    constexpr int NB = KVX_DECODE_BLOCK;
    constexpr int kRowsPerPass = NB / kSlots;
    constexpr int C = kRowsPerPass * U;            // rows per chunk
    static_assert(C <= NB, "one thread moves each chunk row's score and position");
    const int g = blockIdx.x;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    char *kc = k_cache + (size_t)g * budget * R::kBytes;
    char *vc = v_cache + (size_t)g * budget * R::kBytes;
    float *sc = s_cache + (size_t)g * budget;
    int32_t *pc = pos_cache + (size_t)g * budget;

    int dst_new = n_kept;
    if (n_kept >= budget) {
        const int n_total = budget + 1;
        const int lo = n_sink, hi = n_total - recent;
        uint64_t best = ~0ull;
        for (int r = lo + t; r < hi; r += NB) {
            const float s = r < budget ? sc[r] : s_new[g];
            const uint64_t kk = ((uint64_t)select_key(s, keep_low) << 32) |
                                (uint64_t)(0xFFFFFFFFu - (uint32_t)r);
            best = kk < best ? kk : best;
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const uint32_t lo32 = __shfl_xor((uint32_t)best, off);
            const uint32_t hi32 = __shfl_xor((uint32_t)(best >> 32), off);
            const uint64_t o = ((uint64_t)hi32 << 32) | lo32;
            best = o < best ? o : best;
        }
        __shared__ uint64_t wbest[NB / 64];
        if (lane == 0) wbest[w] = best;
        __syncthreads();
        best = wbest[0];
#pragma unroll
        for (int i = 1; i < NB / 64; ++i) best = wbest[i] < best ? wbest[i] : best;
        const int victim = __builtin_amdgcn_readfirstlane((int)(0xFFFFFFFFu - (uint32_t)best));
        if (victim >= budget) return;  // the incoming row is the one dropped

        // The first half of the waves moves K rows, the second half V rows, so
        // the row base is uniform per wave and lives in a scalar buffer
        // resource that is rebuilt per chunk; every lane keeps constant offsets.  The
        // resource of a chunk covers only rows up to budget - 1 of the group:
        // loads beyond it return zeros and stores beyond it are dropped, so
        // the body needs no clamping.  Sources past the last row therefore
        // put zeros on row budget - 1, which the incoming row overwrites.
        constexpr int kHalfThreads = NB / 2;
        constexpr int kRowsPerHalfPass = kHalfThreads / R::kLanes;
        static_assert(kRowsPerHalfPass == kRowsPerPass && kHalfThreads % 64 == 0, "K and V halves of whole waves");
        const int half = __builtin_amdgcn_readfirstlane(t / kHalfThreads);
        const int tt = t % kHalfThreads;
        const int part = tt % R::kLanes;
        const int sub = tt / R::kLanes;
        char *base = half ? vc : kc;
        constexpr int kAux = KVX_DECODE_NT ? 2 : 0;  // slc: the non-temporal hint
        constexpr int kDw3 = 0x00020000;             // raw buffer, 32-bit data format
        struct Chunk {
            u32x4 d[U];
            uint32_t sv, pv;
        };
        const int lo_off = sub * R::kBytes + part * 16;
        const int srow = (t % C) * 4;
        auto rsrc = [&](void *p, int64_t bytes) {
            return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)(uint32_t)(bytes > 0 ? bytes : 0), kDw3);
        };
        auto load = [&](Chunk &ch, int c0) {
            const auto r = rsrc(base + (size_t)c0 * R::kBytes, (int64_t)(budget - c0) * R::kBytes);
#pragma unroll
            for (int u = 0; u < U; ++u)
                ch.d[u] = __builtin_amdgcn_raw_buffer_load_b128(r, lo_off + u * kRowsPerPass * R::kBytes, 0, kAux);
            const auto rs = rsrc(sc + c0, (int64_t)(budget - c0) * 4);
            const auto rp = rsrc(pc + c0, (int64_t)(budget - c0) * 4);
            ch.sv = __builtin_amdgcn_raw_buffer_load_b32(rs, srow, 0, 0);
            ch.pv = __builtin_amdgcn_raw_buffer_load_b32(rp, srow, 0, 0);
        };
        auto landed = [&](Chunk &ch) {
#pragma unroll
            for (int u = 0; u < U; ++u) asm volatile("" ::"v"(ch.d[u].x), "v"(ch.d[u].y), "v"(ch.d[u].z), "v"(ch.d[u].w));
            asm volatile("" ::"v"(ch.sv), "v"(ch.pv));
        };
        auto store = [&](const Chunk &ch, int c0) {
            const auto r = rsrc(base + (size_t)(c0 - 1) * R::kBytes, (int64_t)(budget - c0 + 1) * R::kBytes);
#pragma unroll
            for (int u = 0; u < U; ++u)
                __builtin_amdgcn_raw_buffer_store_b128(ch.d[u], r, lo_off + u * kRowsPerPass * R::kBytes, 0, kAux);
            // every thread stores (threads t and t + C hold the same row's values)
            const auto rs = rsrc(sc + c0 - 1, (int64_t)(budget - c0 + 1) * 4);
            const auto rp = rsrc(pc + c0 - 1, (int64_t)(budget - c0 + 1) * 4);
            __builtin_amdgcn_raw_buffer_store_b32(ch.sv, rs, srow, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(ch.pv, rp, srow, 0, 0);
        };
        // Software pipeline: the next chunk's loads are in flight while this
        // chunk waits, meets the barrier and is stored.  The next chunk's
        // sources lie above every row this chunk writes (except row budget - 1,
        // whose value is discarded), and every thread has its loads
        // of this chunk back before the barrier, so no row is overwritten
        // before it has been read.  The first chunk is peeled so that every
        // wait in the loop sees the same operations in flight after its chunk
        // (the previous chunk's stores and the next chunk's loads) and waits
        // for its own loads only.
        Chunk a, b;
        const int c0 = victim + 1;
        int c1 = c0 + C;
        load(a, c0);
        load(b, c1);
        landed(a);
        __syncthreads();
        store(a, c0);
        while (c1 < budget) {
            const int c2 = c1 + C;
            load(a, c2);
            landed(b);
            __syncthreads();
            store(b, c1);
            if (c2 >= budget) break;
            const int c3 = c2 + C;
            load(b, c3);
            landed(a);
            __syncthreads();
            store(a, c2);
            c1 = c3;
        }
        // Every store (including the discarded ones on row budget - 1) must be
        // complete before the incoming row is written there.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        dst_new = budget - 1;
    }
    if (t < kSlots) {
        const int half = t / R::kLanes, part = t % R::kLanes;
        const char *src = (half ? v_new : k_new) + (size_t)g * R::kBytes + part * 16;
        char *dst = (half ? vc : kc) + (size_t)dst_new * R::kBytes + part * 16;
        st16(dst, ld16(src));
    }
    if (t == 0) {
        sc[dst_new] = s_new[g];
        pc[dst_new] = pos_base;
    }
}

// ---------------------------------------------------------------------------
// Host-side validation shared by the entry points.
// ---------------------------------------------------------------------------
int check_params(const kvx_evict_params &p) {
    if (p.budget < 1) return set_error(KVX_EINVAL, "params: budget must be >= 1 (got %lld)", (long long)p.budget);
    if (p.n_sink < 0 || p.recent < 0)
        return set_error(KVX_EINVAL, "params: n_sink and recent must be >= 0");
    if (p.n_sink + p.recent >= p.budget)
        return set_error(KVX_EINVAL, "params: n_sink + recent (%lld) must be below budget (%lld)",
                         (long long)(p.n_sink + p.recent), (long long)p.budget);
    if (p.keep != KVX_KEEP_HIGH && p.keep != KVX_KEEP_LOW)
        return set_error(KVX_EINVAL, "params: keep must be KVX_KEEP_HIGH or KVX_KEEP_LOW (got %d)", (int)p.keep);
    if (p.budget > KVX_MAX_BUDGET)
        return set_error(KVX_ERANGE, "params: budget %lld exceeds KVX_MAX_BUDGET (%d)",
                         (long long)p.budget, KVX_MAX_BUDGET);
    return KVX_OK;
}

int validate_select_sizes(const kvx_shape &shape, int64_t n_kept, int64_t S, const kvx_evict_params &p,
                          int64_t *G) {
    int rc = check_shape(shape, G);
    if (rc) return rc;
    if ((rc = check_params(p))) return rc;
    if (S < 0) return set_error(KVX_EINVAL, "S must be >= 0 (got %lld)", (long long)S);
    if (n_kept < 0 || n_kept > p.budget)
        return set_error(KVX_EINVAL, "n_kept must be in [0, budget] (got %lld, budget %lld)",
                         (long long)n_kept, (long long)p.budget);
    if (n_kept + S > KVX_MAX_TOTAL)
        return set_error(KVX_ERANGE, "n_kept + S = %lld exceeds KVX_MAX_TOTAL (%d)",
                         (long long)(n_kept + S), KVX_MAX_TOTAL);
    return KVX_OK;
}

template <int DT, int HD, int MODE>
int launch_score_mode(const void *k_new, int64_t G, const kvx_shape &sh, int64_t S, const float *filters,
                      float sign, float *s_new, bool cache_keys, hipStream_t st) {
    constexpr int U = KVX_SCORE_U;
    constexpr int kRowsPerBlock = (KVX_SCORE_BLOCK / 64) * (64 / Row<DT, HD>::kLanes) * U;
    const uint32_t BH = (uint32_t)(sh.B * sh.H), H = (uint32_t)sh.H;
    if (S >= kRowsPerBlock / 2) {
        const uint32_t tiles = (uint32_t)((S + kRowsPerBlock - 1) / kRowsPerBlock);
        if ((int64_t)tiles * G > INT32_MAX) return set_error(KVX_ERANGE, "qf_score_keys: grid too large");
        if (cache_keys)
            score_tile_kernel<DT, HD, MODE, U, false><<<(uint32_t)(tiles * G), KVX_SCORE_BLOCK, 0, st>>>(
                (const char *)k_new, (uint32_t)S, tiles, BH, H, filters, sign, s_new);
        else
            score_tile_kernel<DT, HD, MODE, U, true><<<(uint32_t)(tiles * G), KVX_SCORE_BLOCK, 0, st>>>(
                (const char *)k_new, (uint32_t)S, tiles, BH, H, filters, sign, s_new);
    } else {
        const uint32_t n_rows = (uint32_t)(G * S);
        const uint32_t blocks = (n_rows + kRowsPerBlock - 1) / kRowsPerBlock;
        if (cache_keys)
            score_flat_kernel<DT, HD, MODE, U, false><<<blocks, KVX_SCORE_BLOCK, 0, st>>>(
                (const char *)k_new, n_rows, (uint32_t)S, BH, H, filters, sign, s_new);
        else
            score_flat_kernel<DT, HD, MODE, U, true><<<blocks, KVX_SCORE_BLOCK, 0, st>>>(
                (const char *)k_new, n_rows, (uint32_t)S, BH, H, filters, sign, s_new);
    }
    return check_launch("qf_score_keys");
}

template <int DT, int HD>
int launch_score(const void *k_new, int64_t G, const kvx_shape &sh, int64_t S, int32_t mode,
                 const float *filters, int32_t sign, float *s_new, bool cache_keys, hipStream_t st) {
    if (mode == KVX_SCORE_L2)
        return launch_score_mode<DT, HD, KVX_SCORE_L2>(k_new, G, sh, S, filters, 1.0f, s_new, cache_keys, st);
    return launch_score_mode<DT, HD, KVX_SCORE_PROJ>(k_new, G, sh, S, filters, (float)sign, s_new, cache_keys,
                                                     st);
}

template <int DT, int HD>
int launch_gather(const void *k_kept, const void *v_kept, const float *s_kept, const int32_t *pos_kept,
                  const void *k_new, const void *v_new, const float *s_new, int32_t pos_base,
                  const int32_t *keep_idx, int64_t G, int n_kept, int S, int budget, int j0, int n_out,
                  void *k_out, void *v_out, float *s_out, int32_t *pos_out, hipStream_t st) {
    constexpr int U = KVX_GATHER_U;
    constexpr int kRowsPerBlock = (KVX_GATHER_BLOCK / Row<DT, HD>::kLanes) * U;
    const int rows = n_out - j0;
    if (rows <= 0 || G == 0) return KVX_OK;
    const int bpg = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
    const int64_t blocks = G * bpg;
    if (blocks > INT32_MAX) return set_error(KVX_ERANGE, "kv_compact_gather: grid too large");
    gather_kernel<DT, HD, U><<<(uint32_t)blocks, KVX_GATHER_BLOCK, 0, st>>>(
        (const char *)k_kept, (const char *)v_kept, s_kept, pos_kept, (const char *)k_new,
        (const char *)v_new, s_new, pos_base, keep_idx, n_kept, S, budget, j0, n_out, bpg,
        (char *)k_out, (char *)v_out, s_out, pos_out, check_word());
    return check_launch("kv_compact_gather");
}

template <int DT, int HD, int MODE>
int launch_score_append(const void *k_new, const void *v_new, int64_t G, const kvx_shape &sh, int64_t S,
                        const float *filters, float sign, int32_t pos_base, int64_t n_kept, int64_t budget,
                        void *k_cache, void *v_cache, float *s_cache, int32_t *pos_cache, float *s_new,
                        hipStream_t st) {
    constexpr int U = KVX_APPEND_U;
    constexpr int kRowsPerBlock = (KVX_APPEND_BLOCK / 64) * (64 / Row<DT, HD>::kLanes) * U;
    const uint32_t tiles = (uint32_t)((S + kRowsPerBlock - 1) / kRowsPerBlock);
    if ((int64_t)tiles * G > INT32_MAX) return set_error(KVX_ERANGE, "kv_score_append: grid too large");
    score_append_kernel<DT, HD, MODE, U><<<(uint32_t)(tiles * G), KVX_APPEND_BLOCK, 0, st>>>(
        (const char *)k_new, (const char *)v_new, (uint32_t)S, tiles, (uint32_t)(sh.B * sh.H), (uint32_t)sh.H,
        filters, sign, pos_base, (uint32_t)n_kept, (uint32_t)budget, (char *)k_cache, (char *)v_cache, s_cache,
        pos_cache, s_new);
    return check_launch("kv_score_append");
}

// One workgroup of NT threads per group with the keys in registers: M keys
// per thread, the smallest power of two covering n_total (one when nothing is
// evicted: the identity needs no keys).
template <int NT>
int select_in_registers(const float *s_kept, const float *s_new, int64_t G, int64_t n_kept, int64_t S,
                        const kvx_evict_params &p, int32_t *keep_idx, int32_t *chk, hipStream_t st, const char *what) {
    const int64_t n_total = n_kept + S;
    const int a = (int)n_kept, b = (int)S, bud = (int)p.budget, ns = (int)p.n_sink, rc2 = (int)p.recent;
    const int kl = p.keep == KVX_KEEP_LOW;
    const uint32_t grid = (uint32_t)G;
    if (n_total <= NT || n_total <= p.budget)
        select_kernel<1, NT><<<grid, NT, 0, st>>>(s_kept, s_new, a, b, bud, ns, rc2, kl, keep_idx, chk);
    else if (n_total <= 2 * NT)
        select_kernel<2, NT><<<grid, NT, 0, st>>>(s_kept, s_new, a, b, bud, ns, rc2, kl, keep_idx, chk);
    else if (n_total <= 4 * NT)
        select_kernel<4, NT><<<grid, NT, 0, st>>>(s_kept, s_new, a, b, bud, ns, rc2, kl, keep_idx, chk);
    else if (n_total <= 8 * NT)
        select_kernel<8, NT><<<grid, NT, 0, st>>>(s_kept, s_new, a, b, bud, ns, rc2, kl, keep_idx, chk);
    else if (n_total <= 16 * NT)
        select_kernel<16, NT><<<grid, NT, 0, st>>>(s_kept, s_new, a, b, bud, ns, rc2, kl, keep_idx, chk);
    else
        select_kernel<32, NT><<<grid, NT, 0, st>>>(s_kept, s_new, a, b, bud, ns, rc2, kl, keep_idx, chk);
    return check_launch(what);
}

// Selection launches after validation.  `ws` is the multi-block selection's
// workspace (nullptr when it selects on chip).
int launch_select(const float *s_kept, const float *s_new, int64_t G, int64_t n_kept, int64_t S,
                  const kvx_evict_params &p, int32_t *keep_idx, uint32_t *ws, hipStream_t st, const char *what) {
    const int64_t n_total = n_kept + S;
    const int a = (int)n_kept, b = (int)S, bud = (int)p.budget, ns = (int)p.n_sink, rc2 = (int)p.recent;
    const int kl = p.keep == KVX_KEEP_LOW;
    const uint32_t grid = (uint32_t)G;
    int32_t *chk = check_word();
    constexpr int NT = KVX_SELECT_NT;
    static_assert(NT == 1024, "the on-chip bounds assume 1024-thread selection blocks");
    static_assert(KVX_ONCHIP_TOTAL > 32 * NT, "streaming selection above the register-held keys");
    if (ws == nullptr && n_total > 32 * NT) {  // keys streamed from memory at every pass
        select_stream_kernel<8, NT><<<grid, NT, 0, st>>>(s_kept, s_new, a, b, bud, ns, rc2, kl, keep_idx, chk);
        return check_launch(what);
    }
    if (ws == nullptr) {
        constexpr int NS = KVX_SELECT_SMALL_NT;
        static_assert(NS >= 128 && NS <= NT && NT % NS == 0, "small selection blocks of 2 to 16 waves");
        if (NS < NT && n_total <= 32 * NS)
            return select_in_registers<NS>(s_kept, s_new, G, n_kept, S, p, keep_idx, chk, st, what);
        return select_in_registers<NT>(s_kept, s_new, G, n_kept, S, p, keep_idx, chk, st, what);
    }
    const int W = (int)((n_total + MB_ROWS - 1) / MB_ROWS);
    if (G * W > INT32_MAX) return set_error(KVX_ERANGE, "%s: grid too large", what);
    const MbArgs args{s_kept, s_new, a, b, bud, ns, rc2, kl, W, ws, chk};
    mb_init_kernel<<<grid, 256, 0, st>>>(ws, W, bud);  // clears the histograms and state it reuses
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        mb_hist_kernel<<<(uint32_t)(G * W), MB_NT, 0, st>>>(args, shift);
        mb_pick_kernel<<<grid, 64, 0, st>>>(ws, W, shift);
    }
    mb_count_kernel<<<(uint32_t)(G * W), MB_NT, 0, st>>>(args);
    mb_write_kernel<<<(uint32_t)(G * W), MB_NT, 0, st>>>(args, keep_idx);
    return check_launch(what);
}

// Bytes of device workspace the multi-block selection needs (0 on chip).
int64_t select_workspace_bytes(int64_t G, int64_t n_total, int64_t budget) {
    if (n_total <= KVX_ONCHIP_TOTAL || n_total <= budget) return 0;
    const int64_t W = (n_total + MB_ROWS - 1) / MB_ROWS;
    return G * (int64_t)mb_words((int)W) * 4;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint32_t *g_scratch_ptr[kMaxDevices];  // per device, looked up on its first use

// Device address of `scratch` on the current device (the one `stream` must
// belong to), looked up once per device with that device current.
int scratch_address(void *stream, uint32_t **out, const char *what) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return set_error(KVX_EDEVICE, "%s: no usable current device (%d)", what, dev);
    if (stream != nullptr) {
        hipDevice_t sd = -1;
        if (hipStreamGetDevice((hipStream_t)stream, &sd) != hipSuccess)
            return set_error(KVX_EINVAL, "%s: not a valid stream", what);
        if (sd != dev)
            return set_error(KVX_EINVAL, "%s: the stream belongs to device %d but device %d is current", what,
                             (int)sd, dev);
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return set_error(KVX_EDEVICE, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s", what, dev,
                             hipGetErrorString(e));
        g_scratch_ptr[dev] = (uint32_t *)p;
    }
    *out = g_scratch_ptr[dev];
    return KVX_OK;
}

}  // namespace
}  // namespace kvx

using namespace kvx;

extern "C" {

KVX_API int qf_score_keys(const void *k_new, kvx_shape shape, int64_t S, int32_t mode,
                          const float *filters, int32_t sign, float *s_new, void *stream) {
    clear_error();
    int64_t G = 0;
    int rc = check_shape(shape, &G);
    if (rc) return rc;
    if (S < 0) return set_error(KVX_EINVAL, "qf_score_keys: S must be >= 0");
    const bool cache_keys = (mode & KVX_SCORE_CACHE_KEYS) != 0;
    if (cache_keys) mode &= ~KVX_SCORE_CACHE_KEYS;
    if (mode != KVX_SCORE_L2 && mode != KVX_SCORE_PROJ)
        return set_error(KVX_EINVAL,
                         "qf_score_keys: mode must be KVX_SCORE_L2 or KVX_SCORE_PROJ, optionally | "
                         "KVX_SCORE_CACHE_KEYS (got %d)", (int)mode);
    if (mode == KVX_SCORE_PROJ && sign != 1 && sign != -1)
        return set_error(KVX_EINVAL, "qf_score_keys: sign must be +1 or -1 (got %d)", (int)sign);
    if (mode == KVX_SCORE_PROJ && filters == nullptr)
        return set_error(KVX_EINVAL, "qf_score_keys: projection needs filters");
    if (G == 0 || S == 0) return KVX_OK;
    if (G * S >= ((int64_t)1 << 31)) return set_error(KVX_ERANGE, "qf_score_keys: G*S must be below 2^31");
    if (!k_new || !s_new) return set_error(KVX_EINVAL, "qf_score_keys: NULL buffer");
    hipStream_t st = (hipStream_t)stream;
    return dispatch_row(shape, false, [&](auto dt, auto hd) {
        return launch_score<decltype(dt)::value, decltype(hd)::value>(k_new, G, shape, S, mode, filters, sign,
                                                                       s_new, cache_keys, st);
    });
}

KVX_API int kv_evict_workspace_size(kvx_shape shape, int64_t n_kept, int64_t S, kvx_evict_params p,
                                    size_t *bytes) {
    clear_error();
    int64_t G = 0;
    int rc = validate_select_sizes(shape, n_kept, S, p, &G);
    if (rc) return rc;
    if (!bytes) return set_error(KVX_EINVAL, "kv_evict_workspace_size: NULL output");
    *bytes = (size_t)select_workspace_bytes(G, n_kept + S, p.budget);
    return KVX_OK;
}

KVX_API int kv_evict_topk(const float *s_kept, const float *s_new, kvx_shape shape, int64_t n_kept,
                          int64_t S, kvx_evict_params p, int32_t *keep_idx, void *ws, size_t ws_bytes,
                          void *stream) {
    clear_error();
    int64_t G = 0;
    int rc = validate_select_sizes(shape, n_kept, S, p, &G);
    if (rc) return rc;
    const int64_t n_total = n_kept + S;
    if (G == 0 || n_total == 0) return KVX_OK;
    if (!keep_idx || (n_kept > 0 && !s_kept) || (S > 0 && !s_new))
        return set_error(KVX_EINVAL, "kv_evict_topk: NULL buffer");
    const int64_t need = select_workspace_bytes(G, n_total, p.budget);
    if (need > 0 && (ws == nullptr || (int64_t)ws_bytes < need))
        return set_error(KVX_EINVAL, "kv_evict_topk: n_total %lld needs a workspace of %lld bytes (got %zu)",
                         (long long)n_total, (long long)need, ws ? ws_bytes : (size_t)0);
    return launch_select(s_kept, s_new, G, n_kept, S, p, keep_idx, need > 0 ? (uint32_t *)ws : nullptr,
                         (hipStream_t)stream, "kv_evict_topk");
}

KVX_API int kv_evict_topk_noalloc(const float *s_kept, const float *s_new, kvx_shape shape, int64_t n_kept,
                                  int64_t S, kvx_evict_params p, int32_t *keep_idx, void *stream) {
    clear_error();
    int64_t G = 0;
    int rc = validate_select_sizes(shape, n_kept, S, p, &G);
    if (rc) return rc;
    const int64_t n_total = n_kept + S;
    if (G == 0 || n_total == 0) return KVX_OK;
    if (!keep_idx || (n_kept > 0 && !s_kept) || (S > 0 && !s_new))
        return set_error(KVX_EINVAL, "kv_evict_topk_noalloc: NULL buffer");
    const int64_t need = select_workspace_bytes(G, n_total, p.budget);
    if (need > KVX_NOALLOC_SCRATCH_BYTES)
        return set_error(KVX_ERANGE,
                         "kv_evict_topk_noalloc: %lld groups selecting over %lld rows need %lld bytes of scratch; "
                         "the static scratch holds %d (use kv_evict_topk with a workspace)",
                         (long long)G, (long long)n_total, (long long)need, KVX_NOALLOC_SCRATCH_BYTES);
    uint32_t *scr = nullptr;
    if (need > 0 && (rc = scratch_address(stream, &scr, "kv_evict_topk_noalloc"))) return rc;
    return launch_select(s_kept, s_new, G, n_kept, S, p, keep_idx, scr, (hipStream_t)stream,
                         "kv_evict_topk_noalloc");
}

KVX_API int kvx_check_status_word(int32_t *status) {
    clear_error();
    if (!kCheck && status != nullptr)
        return set_error(KVX_EINVAL, "kvx_check_status_word: this library was built without KVX_CHECK");
    g_check_word.store(status, std::memory_order_relaxed);
    return KVX_OK;
}

KVX_API int kv_score_append(const void *k_new, const void *v_new, kvx_shape shape, int64_t S, int32_t mode,
                            const float *filters, int32_t sign, int64_t pos_base, int64_t n_kept,
                            kvx_evict_params p, void *k_cache, void *v_cache, float *s_cache, int32_t *pos_cache,
                            float *s_new, void *stream) {
    clear_error();
    int64_t G = 0;
    int rc = validate_select_sizes(shape, n_kept, S, p, &G);
    if (rc) return rc;
    mode &= ~KVX_SCORE_CACHE_KEYS;  // the keys are read once here either way
    if (mode != KVX_SCORE_L2 && mode != KVX_SCORE_PROJ)
        return set_error(KVX_EINVAL, "kv_score_append: mode must be KVX_SCORE_L2 or KVX_SCORE_PROJ (got %d)",
                         (int)mode);
    if (mode == KVX_SCORE_PROJ && sign != 1 && sign != -1)
        return set_error(KVX_EINVAL, "kv_score_append: sign must be +1 or -1 (got %d)", (int)sign);
    if (mode == KVX_SCORE_PROJ && filters == nullptr)
        return set_error(KVX_EINVAL, "kv_score_append: projection needs filters");
    if (n_kept + S > p.budget)
        return set_error(KVX_EINVAL,
                         "kv_score_append: n_kept + S = %lld exceeds the budget %lld (a call that evicts needs "
                         "kv_evict_topk and kv_compact_gather)", (long long)(n_kept + S), (long long)p.budget);
    if (pos_base < 0 || pos_base + S > INT32_MAX)
        return set_error(KVX_ERANGE, "kv_score_append: positions must fit int32 (pos_base %lld, S %lld)",
                         (long long)pos_base, (long long)S);
    if (G == 0 || S == 0) return KVX_OK;
    if (G * S >= ((int64_t)1 << 31)) return set_error(KVX_ERANGE, "kv_score_append: G*S must be below 2^31");
    if (!k_new || !v_new || !k_cache || !v_cache || !s_cache || !pos_cache)
        return set_error(KVX_EINVAL, "kv_score_append: NULL buffer");
    if (k_new == k_cache || v_new == v_cache || k_new == v_cache || v_new == k_cache)
        return set_error(KVX_EINVAL, "kv_score_append: the incoming rows must not be the cache buffers");
    hipStream_t st = (hipStream_t)stream;
    return dispatch_row(shape, false, [&](auto dt, auto hd) {
        constexpr int DT = decltype(dt)::value, HD = decltype(hd)::value;
        if (mode == KVX_SCORE_L2)
            return launch_score_append<DT, HD, KVX_SCORE_L2>(k_new, v_new, G, shape, S, filters, 1.0f,
                                                             (int32_t)pos_base, n_kept, p.budget, k_cache, v_cache,
                                                             s_cache, pos_cache, s_new, st);
        return launch_score_append<DT, HD, KVX_SCORE_PROJ>(k_new, v_new, G, shape, S, filters, (float)sign,
                                                           (int32_t)pos_base, n_kept, p.budget, k_cache, v_cache,
                                                           s_cache, pos_cache, s_new, st);
    });
}

KVX_API int kv_compact_gather(const void *k_kept, const void *v_kept, const float *s_kept,
                              const int32_t *pos_kept, const void *k_new, const void *v_new,
                              const float *s_new, int64_t pos_base, const int32_t *keep_idx,
                              kvx_shape shape, int64_t n_kept, int64_t S, kvx_evict_params p,
                              void *k_out, void *v_out, float *s_out, int32_t *pos_out, void *stream) {
    clear_error();
    int64_t G = 0;
    int rc = validate_select_sizes(shape, n_kept, S, p, &G);
    if (rc) return rc;
    const int64_t n_total = n_kept + S;
    const bool evict = n_total > p.budget;
    const int n_out = (int)(evict ? p.budget : n_total);
    if (pos_base < 0 || pos_base + S > INT32_MAX)
        return set_error(KVX_ERANGE, "kv_compact_gather: positions must fit int32 (pos_base %lld, S %lld)",
                         (long long)pos_base, (long long)S);
    if (G == 0 || n_out == 0) return KVX_OK;
    if (!k_out || !v_out || !s_out || !pos_out) return set_error(KVX_EINVAL, "kv_compact_gather: NULL output");
    if (n_kept > 0 && (!k_kept || !v_kept || !s_kept || !pos_kept))
        return set_error(KVX_EINVAL, "kv_compact_gather: NULL kept buffer");
    if (S > 0 && (!k_new || !v_new || !s_new)) return set_error(KVX_EINVAL, "kv_compact_gather: NULL incoming buffer");
    if (evict && !keep_idx) return set_error(KVX_EINVAL, "kv_compact_gather: keep_idx is required when evicting");
    const int n_alias = (k_out == k_kept) + (v_out == v_kept) + ((const void *)s_out == (const void *)s_kept) +
                        ((const void *)pos_out == (const void *)pos_kept);
    if (n_alias != 0 && n_alias != 4)
        return set_error(KVX_EINVAL, "kv_compact_gather: outputs must alias all four kept buffers or none");
    if (n_alias == 4 && evict)
        return set_error(KVX_EINVAL, "kv_compact_gather: in-place compaction is only allowed without eviction");
    const int j0 = n_alias == 4 ? (int)n_kept : 0;  // in place: only the incoming rows move
    const int32_t *idx = evict ? keep_idx : nullptr;
    hipStream_t st = (hipStream_t)stream;
    return dispatch_row(shape, true, [&](auto dt, auto hd) {
        return launch_gather<decltype(dt)::value, decltype(hd)::value>(
            k_kept, v_kept, s_kept, pos_kept, k_new, v_new, s_new, (int32_t)pos_base, idx, G, (int)n_kept, (int)S,
            (int)p.budget, j0, n_out, k_out, v_out, s_out, pos_out, st);
    });
}

KVX_API int kv_evict_one_inplace(void *k_cache, void *v_cache, float *s_cache, int32_t *pos_cache,
                                 const void *k_new, const void *v_new, const float *s_new, int64_t pos_base,
                                 kvx_shape shape, int64_t n_kept, kvx_evict_params p, void *stream) {
    clear_error();
    int64_t G = 0;
    int rc = validate_select_sizes(shape, n_kept, 1, p, &G);
    if (rc) return rc;
    if (pos_base < 0 || pos_base >= INT32_MAX)
        return set_error(KVX_ERANGE, "kv_evict_one_inplace: position must fit int32");
    if (G == 0) return KVX_OK;
    if (!k_cache || !v_cache || !s_cache || !pos_cache || !k_new || !v_new || !s_new)
        return set_error(KVX_EINVAL, "kv_evict_one_inplace: NULL buffer");
    hipStream_t st = (hipStream_t)stream;
    if (G > INT32_MAX) return set_error(KVX_ERANGE, "kv_evict_one_inplace: too many groups");
    const int kl = p.keep == KVX_KEEP_LOW;
    dispatch_row(shape, true, [&](auto dt, auto hd) {
        evict_one_kernel<decltype(dt)::value, decltype(hd)::value, KVX_DECODE_U>
            <<<(uint32_t)G, KVX_DECODE_BLOCK, 0, st>>>((char *)k_cache, (char *)v_cache, s_cache, pos_cache,
                                                       (const char *)k_new, (const char *)v_new, s_new,
                                                       (int32_t)pos_base, (int)n_kept, (int)p.budget,
                                                       (int)p.n_sink, (int)p.recent, kl);
        return 0;
    });
    return check_launch("kv_evict_one_inplace");
}

}  // extern "C"
