/*
 * kvevict.h -- C ABI of the MI355X (gfx950) query-free KV-cache eviction step.
 *
 * The step, per (layer, batch, KV head) group, as the pages define it:
 *   1. score every incoming key once, at insertion: its L2 norm, or its
 *      projection onto a frozen per-head filter times a sign
 *      ("L2Norm — Intrinsic Key-Norm Eviction", "How it works" step 1;
 *       "Q-Filters — Query-Agnostic Projection Eviction", "How it works" step 3);
 *   2. append the incoming rows after the kept rows (same sections, step 1/2);
 *   3. when the result holds more rows than the budget, keep the budget best in
 *      one top-k with the first n_sink rows and the last `recent` rows forced to
 *      survive, ties going to the lower row (Q-Filters page, "How it works"
 *      step 4 and "Metal kernels", the tie paragraph);
 *   4. compact the survivors in temporal order, keeping their absolute
 *      positions and their K/V bytes unchanged (Q-Filters page, "Adaptation
 *      notes").
 *
 * Conventions for every entry point below
 *   - Return value: KVX_OK (0) or a negative KVX_E* code.  On error a message is
 *     available from kvx_last_error() (thread-local, valid until the next call
 *     on the same thread).  Nothing throws across the ABI.
 *   - Device entry points (qf_score_keys, kv_evict_topk, kv_compact_gather,
 *     kv_evict_one_inplace) take device pointers owned by the caller, validate
 *     every size argument before enqueueing anything, enqueue their kernels on
 *     `stream` (a hipStream_t; NULL = the default stream) and return without
 *     synchronising.  They never allocate device memory.  A launch failure
 *     returns KVX_EDEVICE.  Pointers must be device memory large enough for the
 *     layouts stated; the library cannot check that.
 *   - Host entry points (qf_filters_*, kvx_stats) take host memory and run
 *     synchronously on the calling thread (qf_filters_from_* may use a few
 *     worker threads internally).
 *   - Groups: g = (l*B + b)*H + h for layer l, batch b, KV head h;
 *     G = L*B*H.  Every group in one call holds the same number of kept rows
 *     (the budget is uniform across heads, Q-Filters page, "Adaptation notes").
 *   - Cache buffers (kept and output) have a per-group capacity of exactly
 *     `budget` rows:  K/V [G, budget, D], scores [G, budget] float32,
 *     positions [G, budget] int32; rows [0, n_kept) are valid, in temporal
 *     order.  Incoming buffers have S rows per group: K/V [G, S, D],
 *     scores [G, S].  All row-major and contiguous.
 *   - Element types: KVX_BF16 (raw bfloat16), KVX_F16 or KVX_F32 for K/V rows;
 *     head dim D of 64, 128 or 256 (rows are D elements).
 */
#ifndef KVEVICT_H
#define KVEVICT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVX_API __attribute__((visibility("default")))

/* Status codes. */
#define KVX_OK 0
#define KVX_EINVAL -1    /* an argument violates a stated rule             */
#define KVX_ERANGE -2    /* a size exceeds a bound of this implementation  */
#define KVX_EDEVICE -3   /* a HIP call or kernel launch failed              */
#define KVX_EIO -4       /* a file could not be read, written or parsed     */
#define KVX_EMISMATCH -5 /* an artifact does not match what the caller asked */

/* Element types of K/V rows. */
#define KVX_F32 0
#define KVX_BF16 1
#define KVX_F16 2  /* IEEE binary16 (the Metal kernels' key type, Q-Filters page, "Metal kernels") */

/* Scorers. */
#define KVX_SCORE_L2 0   /* s = ||k||_2                       */
#define KVX_SCORE_PROJ 1 /* s = sign * (k . f[l][h])          */
#define KVX_SCORE_CACHE_KEYS 0x100 /* or-ed into a mode: read the keys with
                                      cache-allocating loads (see qf_score_keys) */

/* Ranking direction. */
#define KVX_KEEP_HIGH 0  /* keep the highest scores (projection; L2 ablation) */
#define KVX_KEEP_LOW 1   /* keep the lowest scores (L2 norm, paper rule)      */

/* Bounds of this implementation. */
#define KVX_HEAD_DIM 128     /* the head dim of every workload here; D may also be 64 or 256 */
#define KVX_MAX_BUDGET (1 << 21)   /* largest budget accepted                          */
#define KVX_MAX_TOTAL (1 << 22)    /* largest n_kept + S that one selection handles     */
#define KVX_ONCHIP_TOTAL 262144    /* up to this n_total the selection needs no workspace */
#define KVX_NOALLOC_SCRATCH_BYTES (8 << 20) /* static device scratch of kv_evict_topk_noalloc */

typedef struct {
    int64_t L, B, H; /* layers, batch, KV heads: G = L*B*H groups            */
    int64_t D;       /* head dim: 64, 128 or 256                             */
    int32_t dtype;   /* KVX_BF16, KVX_F16 or KVX_F32                         */
} kvx_shape;

typedef struct {
    int64_t budget; /* rows kept per group, sinks included (Q-Filters page, "Usage") */
    int64_t n_sink; /* leading rows never evicted                                    */
    int64_t recent; /* trailing rows of the concatenation never evicted              */
    int32_t keep;   /* KVX_KEEP_HIGH or KVX_KEEP_LOW                                 */
} kvx_evict_params;
/* Rules, checked by every call that takes params: budget >= 1, n_sink >= 0,
 * recent >= 0, n_sink + recent < budget (Q-Filters page, "Evidence", fallback
 * list: a violation raises at build time), budget <= KVX_MAX_BUDGET.         */

typedef struct {
    int64_t kept_bytes;      /* K+V bytes currently retained, all groups          */
    int64_t full_seq_bytes;  /* K+V bytes if every seen token were kept            */
    double compression_ratio; /* full_seq_bytes / kept_bytes (0 when nothing kept) */
    int64_t tokens_seen;     /* absolute tokens absorbed (the true offset)          */
    int64_t tokens_kept;     /* rows kept per group                                  */
    int64_t filter_bytes;    /* frozen filters counted in full: L*H*D*4 (projection) */
} kvx_stats_t;

/* Thread-local message of the last failed call on this thread ("" if none). */
KVX_API const char *kvx_last_error(void);

/* ABI version of this library (incremented on incompatible changes). */
KVX_API int kvx_abi_version(void);

/*
 * qf_score_keys -- step 1: one score per incoming row.
 *   k_new    device [G, S, D] K rows (shape.dtype), widened exactly to float32
 *   S        incoming rows per group (S == 0: nothing is launched)
 *   mode     KVX_SCORE_L2: s = ||k||_2   (L2Norm page, "How it works" step 1)
 *            KVX_SCORE_PROJ: s = sign * sum_d k_d f[l][h][d]
 *                             (Q-Filters page, "How it works" step 3)
 *   filters  device [L, H, D] float32 frozen filters, group (l, b, h) uses
 *            filters[l][h]; NULL allowed only for L2.  Per-group filters
 *            [L*B, H, D] are passed by describing the shape as L' = L*B, B' = 1.
 *   sign     +1 or -1 (projection only; ignored for L2)
 *   s_new    device [G, S] float32 output
 * mode | KVX_SCORE_CACHE_KEYS reads the keys with cache-allocating loads
 * instead of streaming ones.  It pays when the block's keys fit the 256 MB
 * last-level cache and the compaction that follows will re-read a good share
 * of them (the surviving new rows); the scores are the same either way.
 * Scores accumulate in float32 in a fixed order per row (independent of S and
 * of the launch), and a -0 result is written as +0.  Keys must be finite.
 * Errors: KVX_EINVAL (bad mode/sign/dtype/D, NULL pointer), KVX_ERANGE
 * (G*S >= 2^31), KVX_EDEVICE.
 */
KVX_API int qf_score_keys(const void *k_new, kvx_shape shape, int64_t S, int32_t mode,
                          const float *filters, int32_t sign, float *s_new, void *stream);

/*
 * kv_evict_workspace_size -- bytes of device workspace kv_evict_topk needs for
 * these sizes (implementation-defined; the pages define no workspace): 0 when
 * n_kept + S <= KVX_ONCHIP_TOTAL (one workgroup per group selects: up to
 * 32768 rows with every key in registers, beyond that reading the scores
 * again at each radix pass) or when nothing is evicted; otherwise
 * G * (260 + 2 * ceil(n_total / 16384)) * 4 bytes for the multi-block
 * selection's histograms, state and block counts.  The caller allocates it;
 * kv_evict_topk initialises it itself on the stream (no memset needed), and
 * calls that overlap on one workspace race.  Errors: as kv_evict_topk's
 * validation.
 */
KVX_API int kv_evict_workspace_size(kvx_shape shape, int64_t n_kept, int64_t S,
                                    kvx_evict_params p, size_t *bytes);

/*
 * kv_score_append -- steps 1-4 of a call that evicts nothing (n_kept + S <=
 * budget): every incoming row is kept (L2Norm page, "How it works"; Q-Filters
 * page, "How it works" step 4: eviction only when over budget), so the rows
 * are scored and appended in one pass and each key is read once.  The result
 * is bit for bit that of qf_score_keys followed by the in-place
 * kv_compact_gather: rows n_kept .. n_kept + S - 1 of every group receive the
 * incoming K and V bytes, the score (same fixed-order float32 sum, -0 stored
 * as +0) and the position pos_base + i.
 *   k_new, v_new   device [G, S, D] of shape.dtype; must not be the cache buffers
 *   mode, filters, sign   as qf_score_keys (KVX_SCORE_CACHE_KEYS is accepted
 *                  and has no effect); shape describes the filters' layout as
 *                  there, and the cache's groups are the same G
 *   *_cache        device cache buffers [G, budget, *] with n_kept valid rows
 *   s_new          device [G, S] float32 copy of the scores, or NULL
 * Errors: KVX_EINVAL (n_kept + S > budget: such a call evicts and needs
 * kv_evict_topk and kv_compact_gather; bad mode/sign, NULL, aliasing),
 * KVX_ERANGE, KVX_EDEVICE.
 */
KVX_API int kv_score_append(const void *k_new, const void *v_new, kvx_shape shape, int64_t S, int32_t mode,
                            const float *filters, int32_t sign, int64_t pos_base, int64_t n_kept,
                            kvx_evict_params p, void *k_cache, void *v_cache, float *s_cache, int32_t *pos_cache,
                            float *s_new, void *stream);

/*
 * kv_evict_topk -- steps 2-3: which rows of the concatenation survive.
 *   s_kept   device [G, budget] stored scores of the n_kept kept rows
 *   s_new    device [G, S] scores of the incoming rows (from qf_score_keys)
 *   n_kept   0 <= n_kept <= budget;  n_total = n_kept + S <= KVX_MAX_TOTAL
 *   keep_idx device [G, budget] int32 output: the kept rows of the
 *            concatenation (row r < n_kept is kept row r, row r >= n_kept is
 *            incoming row r - n_kept), strictly ascending, min(n_total, budget)
 *            of them per group.
 *   ws       device workspace of at least kv_evict_workspace_size bytes
 *            (may be NULL when that is 0); KVX_EINVAL if missing or too small
 * When n_total <= budget nothing is evicted and keep_idx is 0..n_total-1.
 * Otherwise the protected rows (r < n_sink, r >= n_total - recent) are kept,
 * and the other budget - n_sink - recent slots go to the best rows: highest
 * score for KVX_KEEP_HIGH, lowest for KVX_KEEP_LOW, equal scores (with -0 ==
 * +0) going to the lower row.  Scores must be finite.
 * Errors: KVX_EINVAL, KVX_ERANGE (budget or n_total above the bounds),
 * KVX_EDEVICE.
 */
KVX_API int kv_evict_topk(const float *s_kept, const float *s_new, kvx_shape shape,
                          int64_t n_kept, int64_t S, kvx_evict_params p, int32_t *keep_idx,
                          void *ws, size_t ws_bytes, void *stream);

/*
 * kv_evict_topk_noalloc -- kv_evict_topk for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, rules, output and errors as
 * kv_evict_topk, without the workspace: where kv_evict_workspace_size would
 * be non-zero, the selection uses a static device array of
 * KVX_NOALLOC_SCRATCH_BYTES (8 MiB) that the library holds on every GPU it
 * runs on until the process ends, and sizes whose workspace would exceed it
 * return KVX_ERANGE before anything is enqueued.  Nothing is allocated or
 * freed by this call.  The array is cleared by a fill kernel on `stream` at
 * the start of each call that uses it; every call on one GPU shares it, so
 * calls that overlap on one GPU (other streams, other host threads) race.
 * `stream` must belong to the current device (KVX_EINVAL otherwise).
 */
KVX_API int kv_evict_topk_noalloc(const float *s_kept, const float *s_new, kvx_shape shape, int64_t n_kept,
                                  int64_t S, kvx_evict_params p, int32_t *keep_idx, void *stream);

/*
 * Checked build.  A library compiled with -DKVX_CHECK (libkvevict_check.so)
 * verifies the index lists of the selection and the compaction as it runs:
 * the selection keeps exactly min(n_total, budget) rows and writes every one
 * to a slot below the budget; every keep_idx entry the compaction reads lies
 * in [0, n_kept + S) and is above the one before it.  The first violation is
 * recorded in four device int32 words {code, group, row, value}; later ones
 * are dropped.  Codes: */
#define KVX_CHECK_SLOT 1  /* the selection produced a slot >= budget (value = slot)  */
#define KVX_CHECK_RANGE 2 /* keep_idx[row] outside [0, n_kept + S) (value = index)   */
#define KVX_CHECK_ORDER 3 /* keep_idx[row] <= keep_idx[row - 1] (value = index)      */
#define KVX_CHECK_COUNT 4 /* the selection kept a number of rows != budget (value)   */
/*
 * kvx_check_status_word -- where the checked build records violations: device
 * memory of 4 int32 that the caller zeroes and reads after synchronising (the
 * library never clears it; NULL stops the recording).  One setting per
 * process, read at each launch.  The normal build does no checking and
 * returns KVX_EINVAL for a non-NULL pointer.  Errors: KVX_EINVAL.
 */
KVX_API int kvx_check_status_word(int32_t *status);

/*
 * kv_compact_gather -- step 4: copy the survivors in temporal order.
 *   *_kept   device cache buffers holding n_kept rows per group (capacity budget)
 *   k_new, v_new, s_new  device incoming rows [G, S, *]
 *   pos_base absolute position of incoming row 0 (= tokens seen before this
 *            block, the true offset; Q-Filters page, "RoPE positions had to be
 *            fixed first"); incoming row i gets position pos_base + i
 *   keep_idx from kv_evict_topk for the same (n_kept, S, p); not read, and may
 *            be NULL, when n_kept + S <= budget
 *   *_out    device cache buffers [G, budget, *] receiving min(n_total, budget)
 *            rows per group: out[j] = concat[keep_idx[j]] for K, V (bit copies),
 *            score (the stored score, never a protection mark) and position.
 * Aliasing: the outputs must not overlap the inputs, except that when
 * n_kept + S <= budget all four outputs may be the kept buffers themselves
 * (then the incoming rows are appended in place and nothing else moves).
 * keep_idx is not validated by the normal build: an entry outside
 * [0, n_kept + S) is read as row 0 (no access leaves the buffers, but the
 * result is wrong and the call still returns KVX_OK), and a list that is not
 * strictly ascending gives rows out of temporal order.  The checked build
 * records both (kvx_check_status_word).
 * Errors: KVX_EINVAL (including a partial alias), KVX_ERANGE, KVX_EDEVICE.
 */
KVX_API int kv_compact_gather(const void *k_kept, const void *v_kept, const float *s_kept,
                              const int32_t *pos_kept, const void *k_new, const void *v_new,
                              const float *s_new, int64_t pos_base, const int32_t *keep_idx,
                              kvx_shape shape, int64_t n_kept, int64_t S, kvx_evict_params p,
                              void *k_out, void *v_out, float *s_out, int32_t *pos_out,
                              void *stream);

/*
 * kv_evict_one_inplace -- steps 2-4 for a single incoming row (S = 1), done in
 * place on the cache buffers (decode): the argmin-then-shift pattern of the
 * pages' other Metal eviction kernels (Q-Filters page, "Metal kernels"), with
 * the ranking and protection of the general step (same page, "How it works"
 * step 4).
 *   *_cache  device cache buffers [G, budget, *] with n_kept valid rows
 *   k_new, v_new  device [G, 1, D];  s_new device [G] (from qf_score_keys)
 *   pos_base position of the incoming row
 * If n_kept < budget the row is appended at row n_kept.  Otherwise
 * (n_kept == budget) exactly one row of the budget + 1 is dropped: the
 * unprotected row ranked last (lowest key; of equal keys the higher row),
 * which is what the general rule gives for S = 1.  Rows after it move down by
 * one, in order, and the incoming row lands at row budget - 1 unless it was the
 * one dropped (possible only when recent == 0).  The kept set is then
 * n = min(n_kept + 1, budget) rows.
 * Calls that overlap on the same buffers race.
 * Errors: KVX_EINVAL, KVX_ERANGE, KVX_EDEVICE.
 */
KVX_API int kv_evict_one_inplace(void *k_cache, void *v_cache, float *s_cache,
                                 int32_t *pos_cache, const void *k_new, const void *v_new,
                                 const float *s_new, int64_t pos_base, kvx_shape shape,
                                 int64_t n_kept, kvx_evict_params p, void *stream);

/*
 * qf_filters_load -- read a calibration artifact (Q-Filters page, "Calibrated"
 * and "Usage"): an uncompressed .npz holding `filters` float32 [L, H_kv, D],
 * `model_id` (string), `version` (int64, must be 1), `n_samples` (int64) and
 * `dataset` (string).
 *   expect_model_id  when not NULL, must equal the stored model_id
 *   L, H_kv, D       the layout the caller's model has
 *   out              host [L, H_kv, D] float32
 *   n_samples_out    optional (may be NULL)
 * Every member's CRC-32 is checked, and offsets and sizes that point outside
 * the file are refused before anything is read through them.
 * Errors: KVX_EIO (missing file, bad zip/npy, checksum mismatch, missing field,
 * wrong dtype), KVX_EMISMATCH (version, model id, layer count, head layout or
 * D differ).
 */
KVX_API int qf_filters_load(const char *path, const char *expect_model_id, int64_t L,
                            int64_t H_kv, int64_t D, float *out, int64_t *n_samples_out);

/* qf_filters_save -- write an artifact in the format qf_filters_load reads
 * (version 1).  Errors: KVX_EINVAL, KVX_EIO. */
KVX_API int qf_filters_save(const char *path, const float *filters, int64_t L, int64_t H_kv,
                            int64_t D, const char *model_id, int64_t n_samples,
                            const char *dataset);

/*
 * qf_filters_from_queries -- calibrated filters of one layer (Q-Filters page,
 * "Calibrated — the paper's actual mechanism"): for each query head, the top
 * right singular vector v1 of its activations Q_h [N, D] without mean
 * centring, with the sign of 1^T u1 (sgn(0) taken as +1); then the query heads
 * of each group (contiguous: head h -> KV head h / (H_q / H_kv)) are averaged
 * and renormalised onto their KV head.
 *   q    host [H_q, N, D] float32;  out host [H_kv, D] float32 (unit norm)
 * Errors: KVX_EINVAL (H_q not a multiple of H_kv, sizes, a head whose top two
 * singular values coincide, a zero matrix or a zero group mean).
 */
KVX_API int qf_filters_from_queries(const float *q, int64_t H_q, int64_t N, int64_t D,
                                    int64_t H_kv, float *out);

/*
 * qf_filters_from_keys -- key-SVD fallback filters (Q-Filters page, "Two
 * filter sources" and "Key-SVD fallback"): for each of G groups, the top right
 * singular vector of the group's first n keys after subtracting their column
 * means, signed so that its largest-magnitude entry is positive.
 *   k           host keys, group g's row i at k + (g*group_stride + i)*D
 *               elements, of `dtype`
 *   out         host [G, D] float32 (unit norm)
 * Errors: KVX_EINVAL (sizes, non-finite keys, degenerate spectrum).
 */
KVX_API int qf_filters_from_keys(const void *k, int32_t dtype, int64_t G, int64_t n,
                                 int64_t group_stride, int64_t D, float *out);

/*
 * kv_passthrough_append -- the fallback's pre-calibration passthrough
 * (Q-Filters page, "How it works" step 2): until the key-SVD filter exists no
 * row can be scored, so every row is kept, even over budget.  Copies the n_held
 * held rows and then the S new rows of each group into the output, and writes
 * their positions (row o gets position o: the passthrough only ever holds the
 * stream's first tokens).
 *   k_held, v_held  device [G, cap_held, D] of `shape.dtype`, n_held valid rows
 *                   (may be NULL when n_held == 0)
 *   k_new, v_new    device [G, S, D]
 *   k_out, v_out    device [G, cap_out, D];  pos_out device [G, cap_out] int32
 * Needs n_held <= cap_held and n_held + S <= cap_out.  When the outputs are the
 * held buffers themselves (same pointers, cap_out == cap_held) only the new
 * rows (and their positions) are written; any other overlap of an output with
 * an input is rejected.  Asynchronous on `stream`.
 * Errors: KVX_EINVAL (sizes, NULL, overlap), KVX_ERANGE, KVX_EDEVICE.
 */
KVX_API int kv_passthrough_append(const void *k_held, const void *v_held, int64_t n_held, int64_t cap_held,
                                  const void *k_new, const void *v_new, int64_t S, kvx_shape shape, void *k_out,
                                  void *v_out, int32_t *pos_out, int64_t cap_out, void *stream);

/*
 * qf_filters_from_keys_device -- the key-SVD fallback filter of
 * qf_filters_from_keys, computed on the device and batched over G groups (one
 * workgroup each; Q-Filters page, "Key-SVD fallback"): the column means of each
 * group's first n keys are subtracted, the centred Gram matrix is accumulated in
 * fp64 and its top eigenvector found by fp64 power iteration, stopped when no
 * entry moves by 1e-14 on two successive steps; the entry of largest magnitude
 * is made positive (lowest index on ties).
 *   k        device keys of `dtype`; group g's row i at row g*group_stride + i
 *   n        keys per group, 2 <= n <= KVX_MAX_TOTAL, group_stride >= n
 *   D        64 or 128 (256 is KVX_ERANGE here; qf_filters_from_keys covers it)
 *   out      device [G, D] float32, unit norm
 *   status   device [G] int32: 0 converged; 1 still moving after max_iter steps
 *            (top two eigenvalues too close to separate); 2 the centred keys
 *            are all zero
 * Asynchronous on `stream`; read `status` after synchronising.
 * Errors: KVX_EINVAL, KVX_ERANGE, KVX_EDEVICE.
 */
KVX_API int qf_filters_from_keys_device(const void *k, int32_t dtype, int64_t G, int64_t n, int64_t group_stride,
                                        int64_t D, float *out, int32_t *status, int32_t max_iter, void *stream);

/*
 * qf_filters_from_queries_device -- query-SVD calibration on the device,
 * batched over layers (Q-Filters page, "Calibrated — the paper's actual
 * mechanism"): per query head, the top right singular vector v1 of its raw (not
 * mean-centred) activations Q [N, D], signed by sgn(1^T u1) (the sign of
 * (column sums of Q) . v1, +1 at zero); the H_q / H_kv filters of the query
 * heads that share a KV head (contiguous: query head h -> KV head
 * h / (H_q / H_kv)) are averaged and renormalised.  fp64 Gram matrix and power
 * iteration, as qf_filters_from_keys_device; one workgroup per (layer, KV head).
 *   q        device [L, H_q, N, D] of `dtype` (activations of calibration text)
 *   out      device [L, H_kv, D] float32, unit norm: the filters qf_score_keys reads
 *   status   device [L, H_kv] int32: 0 ok; 1 a query head's top singular value
 *            is not separated (or no convergence in max_iter steps); 2 a query
 *            head's activations are all zero; 3 the group's mean filter is zero
 * Asynchronous on `stream`; read `status` after synchronising.
 * Errors: KVX_EINVAL (H_q not a multiple of H_kv, sizes, NULL), KVX_ERANGE
 * (D = 256; qf_filters_from_queries covers it on the host), KVX_EDEVICE.
 */
KVX_API int qf_filters_from_queries_device(const void *q, int32_t dtype, int64_t L, int64_t H_q, int64_t N,
                                           int64_t D, int64_t H_kv, float *out, int32_t *status, int32_t max_iter,
                                           void *stream);

/*
 * kvx_stats -- byte accounting of a cache (Q-Filters page, "How it works",
 * last paragraph; L2Norm page, "How it works"): K+V bytes kept and the bytes a
 * full cache of tokens_seen rows would take, their ratio, and the filter bytes
 * when a projection scorer is used.  Errors: KVX_EINVAL.
 */
KVX_API int kvx_stats(kvx_shape shape, int64_t tokens_seen, int64_t tokens_kept, int32_t mode,
                      kvx_stats_t *out);

#ifdef __cplusplus
}
#endif

#endif /* KVEVICT_H */
