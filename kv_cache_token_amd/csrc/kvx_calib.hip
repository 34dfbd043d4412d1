// The filter side of "Q-Filters — Query-Agnostic Projection Eviction" on the
// device: the key-SVD fallback's pre-calibration passthrough, and filter
// estimation (the dominant direction of a set of rows, batched over groups)
// for the page's two filter sources:
//
// * "Key-SVD fallback": the top right singular vector of a group's keys after
//   subtracting their column means, signed so that its largest-magnitude entry
//   is positive (after centring, the sum of the left singular vector is
//   identically zero, so that sum cannot fix the sign);
// * "Calibrated — the paper's actual mechanism": per query head the top right
//   singular vector v1 of the raw (not centred) query activations, signed by
//   the sign of the sum of the left singular vector u1 = Q v1 / sigma1, i.e. of
//   (column sums of Q) . v1, with +1 for an exact zero; under grouped-query
//   attention the filters of the query heads sharing a KV head are averaged
//   and renormalised.
//
// Both are the top eigenvector of a Gram matrix C = X^T X (X centred or raw),
// a dense fp64 contraction, done on the matrix cores (v_mfma_f64_16x16x4f64).
// One workgroup per group, one wave per 64 x 64 quadrant of C held as 16
// accumulator tiles of 16 x 16: a pass over the rows for the fp64 column sums,
// a pass that stages chunks of rows (centred when asked) in LDS as fp64 and
// feeds them four rows at a time to the tiles, then power iteration with C
// held in the tiles, and a check that the top eigenvalue is separated: first a
// bound from the Frobenius norm (on C, then on C^2), else a bounded second
// iteration on the complement of the found vector.  While the iteration is
// slow (top two eigenvalues close), C is squared in place every
// KVX_SQUARE_EVERY steps (C staged in LDS, the product again on the matrix
// cores; up to 2^10-th powers, rescaled by a power of two): the eigenvectors
// stay, the ratio of the top two eigenvalues is squared.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "kvevict.h"
#include "kvx_common.h"
#include "kvx_rows.h"

namespace kvx {
namespace {

// ---------------------------------------------------------------------------
// Pre-calibration passthrough ("Q-Filters — Query-Agnostic Projection
// Eviction", "How it works" step 2): before the fallback filter exists every
// row is kept.  out[g, o] = held[g, o] for o < n_held, new[g, o - n_held] after
// that, positions o (the passthrough only happens from token 0).  When the
// output is the held buffer itself only the new rows are written (streaming
// hints: the rows are not read again soon).
// ---------------------------------------------------------------------------
template <int DT, int HD>
__global__ __launch_bounds__(256) void append_rows_kernel(const char *__restrict__ k_held,
                                                          const char *__restrict__ v_held, int64_t cap_held,
                                                          int64_t n_held, const char *__restrict__ k_new,
                                                          const char *__restrict__ v_new, int64_t S, char *k_out,
                                                          char *v_out, int32_t *pos_out, int64_t cap_out,
                                                          int64_t first, int64_t G) {
    using R = Row<DT, HD>;
    const int64_t rows = n_held + S - first;  // rows written per group
    const int64_t total = G * rows * R::kLanes;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int part = (int)(e % R::kLanes);
        const int64_t gr = e / R::kLanes, g = gr / rows, o = first + gr % rows;
        const char *ks, *vs;
        if (o < n_held) {
            ks = k_held + ((size_t)g * cap_held + o) * R::kBytes;
            vs = v_held + ((size_t)g * cap_held + o) * R::kBytes;
        } else {
            ks = k_new + ((size_t)g * S + (o - n_held)) * R::kBytes;
            vs = v_new + ((size_t)g * S + (o - n_held)) * R::kBytes;
        }
        const size_t od = ((size_t)g * cap_out + o) * R::kBytes + part * 16;
        const uint4 kx = ld16<true>(ks + part * 16), vx = ld16<true>(vs + part * 16);
        st16<true>(k_out + od, kx);
        st16<true>(v_out + od, vx);
        if (part == 0) pos_out[(size_t)g * cap_out + o] = (int32_t)o;
    }
}

enum { DIR_CENTRED_KEYS = 0, DIR_RAW_QUERIES = 1 };

#ifndef KVX_SQUARE_EVERY
#define KVX_SQUARE_EVERY 8
#endif

template <int HD>
struct DirLayout {
    static constexpr int QW = HD / 64;     // quadrants of C per side
    static constexpr int NT = 64 * QW * QW;  // one wave per quadrant: 64 threads for HD 64, 256 for HD 128
    static constexpr int CH = HD;          // staged rows per chunk: an HD x HD fp64 square of LDS
    static constexpr int S = HD + 1;       // LDS row stride in doubles of C (column reads hit distinct banks)
    // Staged rows: column c at c + c / 8 (a gap after every 8 columns, so that
    // the 16 lanes of a row, each writing its 8 consecutive columns, hit
    // distinct banks), rows SP doubles apart
    static constexpr int SP = HD + HD / 8 + 1;
    static constexpr int SQUARE_EVERY = KVX_SQUARE_EVERY;  // power steps between squarings of C
    static constexpr int MAX_SQUARINGS = 10;
    static_assert(QW == 1 || QW == 2, "the device estimator covers head dims 64 and 128");
};

// C is symmetric, so the Gram pass accumulates only its 16 x 16 tiles (i, j)
// with i <= j (36 of 64 at head dim 128), spread evenly over the waves.  A
// pattern names the wave's operand slots (each holds the rows' entries of one
// 16-column block) and, per tile, the two slots it multiplies.  Head dim 64
// (one wave): the upper triangle of the 4 x 4 tiles.  Head dim 128: a wave of
// a diagonal quadrant takes that quadrant's upper triangle except its tile
// (1, 1); the two other waves split the off-diagonal quadrant by tile rows and
// each takes one of the two tiles left over.
struct GramUpper {  // slots: the quadrant's four column blocks
    static constexpr int kSlots = 4, kTiles = 10;
    static constexpr int ta[kTiles] = {0, 0, 0, 0, 1, 1, 1, 2, 2, 3};
    static constexpr int tb[kTiles] = {0, 1, 2, 3, 1, 2, 3, 2, 3, 3};
};
struct GramDiag {  // as GramUpper without tile (1, 1)
    static constexpr int kSlots = 4, kTiles = 9;
    static constexpr int ta[kTiles] = {0, 0, 0, 0, 1, 1, 2, 2, 3};
    static constexpr int tb[kTiles] = {0, 1, 2, 3, 2, 3, 2, 3, 3};
};
struct GramOff {  // slots: two row blocks, column blocks 4-7, a diagonal quadrant's block 1
    static constexpr int kSlots = 7, kTiles = 9;
    static constexpr int ta[kTiles] = {0, 0, 0, 0, 1, 1, 1, 1, 6};
    static constexpr int tb[kTiles] = {2, 3, 4, 5, 2, 3, 4, 5, 6};
};

typedef double f64x4 __attribute__((ext_vector_type(4)));

// One 16 x 16 x 4 fp64 matrix-core product: lane l gives A[l % 16][l / 16] and
// B[l / 16][l % 16]; element q of the result holds D[l / 16 + 4q][l % 16].
__device__ __forceinline__ f64x4 mfma16x16x4(double a, double b, f64x4 c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// x of another lane by a DPP move of its two 32-bit halves (CTRL: a quad
// permute or a row rotation; every lane reads a valid source).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
    const unsigned long long u = (unsigned long long)__double_as_longlong(x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xf, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xf, 0xf, false);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
__device__ __forceinline__ double readlane_f64(double x, int lane) {
    const unsigned long long u = (unsigned long long)__double_as_longlong(x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
// op over the 64 lanes of a wave, the result in every lane: pairs and quads
// by quad permutes, the four quads of a row by rotating the row by 4 and 8
// lanes, the four rows by reading one lane of each (all on the vector unit's
// lane network, no LDS round trips).
template <class Op>
__device__ __forceinline__ double wave_reduce_f64(double s, Op op) {
    s = op(s, dpp_f64<0xB1>(s));   // quad_perm [1, 0, 3, 2]
    s = op(s, dpp_f64<0x4E>(s));   // quad_perm [2, 3, 0, 1]
    s = op(s, dpp_f64<0x124>(s));  // row_ror:4
    s = op(s, dpp_f64<0x128>(s));  // row_ror:8
    return op(op(readlane_f64(s, 0), readlane_f64(s, 16)), op(readlane_f64(s, 32), readlane_f64(s, 48)));
}

__device__ __forceinline__ double shfl_xor_f64(double x, int off) {
    const unsigned long long u = (unsigned long long)__double_as_longlong(x);
    const uint32_t lo = __shfl_xor((uint32_t)u, off), hi = __shfl_xor((uint32_t)(u >> 32), off);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// Group g owns r heads; head q's n rows start at row (g*r + q)*stride of x.
// MODE DIR_CENTRED_KEYS (r = 1): out[g] = the signed fallback direction.
// MODE DIR_RAW_QUERIES: out[g] = the renormalised mean of the r signed query
// filters.  status[g]: 0 ok; 1 a head's top eigenvalue not separated (or not
// converged in max_iter steps); 2 a head's Gram matrix is zero; 3 the mean of
// the group's filters is zero.
template <int DT, int HD, int MODE>
__global__ __launch_bounds__(DirLayout<HD>::NT) void top_direction_kernel(
    const char *__restrict__ x, int64_t stride, int r, int64_t n, float *__restrict__ out,
    int32_t *__restrict__ status, int max_iter) {
    using L = DirLayout<HD>;
    using R = Row<DT, HD>;
    constexpr int NT = L::NT, CH = L::CH, S = L::S, SP = L::SP, E = R::kElemsPerLane, SLOTS = NT / R::kLanes;
    static_assert(CH * SP >= HD * S, "C fits the staging buffer");
    static_assert(SLOTS >= 1 && NT % R::kLanes == 0, "a workgroup covers whole rows");
    static_assert(SLOTS <= CH, "the column partial sums fit the staging buffer");
    __shared__ double xd[CH * SP];  // staged rows, or C; first the column partial sums
    // ypb: quadrant column sums of a mat-vec, two buffers used in turn by the
    // power iteration (the other mat-vecs use the first); vw: each wave's copy
    // of the power iteration's iterate
    __shared__ double cs[HD], mu[HD], v[HD], y[HD], w[HD], acc[HD], ypb[2][L::QW][HD], vw[NT / 64][HD],
        lam[2], red[NT / 64],
        fr[NT / 64];
    __shared__ int flag;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int lr = lane & 15, lk = lane >> 4;
    const int R0 = (wv / L::QW) * 64, C0 = (wv % L::QW) * 64;  // this wave's quadrant of C
    const int64_t g = blockIdx.x;

    // C[R0 + 16a + lk + 4q][C0 + 16b + lr] = Cm[a][b][q]
    f64x4 Cm[4][4];
    auto zero_c = [&]() {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) Cm[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};
    };
    // y = C x, as C^T x (C is symmetric): each lane sums its 16 entries of a
    // column, the four lanes of a column meet by two shuffles, and each
    // quadrant's column sums go to ypb[0] (ends with a barrier); wave 0 then adds
    // the quadrants of a column band (gather_y)
    auto matvec = [&](const double *xv) __attribute__((always_inline)) {
        double p[4] = {0.0, 0.0, 0.0, 0.0};  // p[b]: part of y[C0 + 16b + lr]
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const double xi = xv[R0 + 16 * a + lk + 4 * q];
#pragma unroll
                for (int b = 0; b < 4; ++b) p[b] = __builtin_fma(Cm[a][b][q], xi, p[b]);
            }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            p[b] += shfl_xor_f64(p[b], 16);
            p[b] += shfl_xor_f64(p[b], 32);
        }
        if (lk == 0)
#pragma unroll
            for (int b = 0; b < 4; ++b) ypb[0][wv / L::QW][C0 + 16 * b + lr] = p[b];
        __syncthreads();
    };
    auto gather_y = [&]() {  // wave 0
        for (int i = lane; i < HD; i += 64) {
            double s = ypb[0][0][i];
#pragma unroll
            for (int h = 1; h < L::QW; ++h) s += ypb[0][h][i];
            y[i] = s;
        }
    };
    // wave-0 reductions and vector updates over HD-long LDS vectors
    auto wsum = [&](double s) { return wave_reduce_f64(s, [](double a, double b) { return a + b; }); };
    auto wmax = [&](double s) { return wave_reduce_f64(s, [](double a, double b) { return fmax(a, b); }); };
    auto wdot = [&](const double *a, const double *b) {
        double s = 0.0;
        for (int i = lane; i < HD; i += 64) s += a[i] * b[i];
        return wsum(s);
    };
    // xv <- yv / |yv| (after removing the component along `away` when given);
    // returns 2 for a zero yv, 1 when no entry of xv moved by 1e-14, else 0
    auto renorm = [&](double *xv, double *yv, const double *away) {
        if (away) {
            const double d = wdot(away, yv);
            for (int i = lane; i < HD; i += 64) yv[i] -= d * away[i];
        }
        const double ss = wdot(yv, yv);
        const double inv = ss > 0.0 ? 1.0 / sqrt(ss) : 0.0;
        double dmax = 0.0;
        for (int i = lane; i < HD; i += 64) {
            const double nv = yv[i] * inv;
            dmax = fmax(dmax, fabs(nv - xv[i]));
            xv[i] = nv;
        }
        dmax = wmax(dmax);
        return !(ss > 0.0) ? 2 : (dmax < 1e-14 ? 1 : 0);
    };
    // a fixed, generic start vector
    auto start_value = [](int i, uint32_t salt) {
        const uint32_t h = ((uint32_t)(i + 1) ^ salt) * 2654435761u;
        return ((h >> 31) ? -1.0 : 1.0) * (0.5 + (double)((h >> 8) & 0xFFFF) / 65536.0);
    };
    auto start = [&](double *xv, uint32_t salt) {
        for (int i = t; i < HD; i += NT) xv[i] = start_value(i, salt);
    };
    // One power step on this wave's copy of the iterate: the mat-vec's
    // quadrant sums go to ypb[k] and meet after one barrier; then every wave
    // adds them and normalises by itself (the same operations on the same
    // values, so every copy stays equal and every wave returns the same
    // verdict: 2 for a zero result, 1 when no entry moved by 1e-14, else 0).
    // With the two buffers used in turn one barrier per step suffices: a wave
    // rewrites ypb[k] only after the next step's barrier, which every wave
    // passes after its reads of ypb[k].
    auto power_step = [&](int k) __attribute__((always_inline)) {
        double *xv = vw[wv];
        double p[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const double xi = xv[R0 + 16 * a + lk + 4 * q];
#pragma unroll
                for (int b = 0; b < 4; ++b) p[b] = __builtin_fma(Cm[a][b][q], xi, p[b]);
            }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            p[b] += shfl_xor_f64(p[b], 16);
            p[b] += shfl_xor_f64(p[b], 32);
        }
        if (lk == 0)
#pragma unroll
            for (int b = 0; b < 4; ++b) ypb[k][wv / L::QW][C0 + 16 * b + lr] = p[b];
        __syncthreads();
        constexpr int J = HD / 64;
        double yv[J], ss = 0.0;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int i = lane + 64 * j;
            double s = ypb[k][0][i];
#pragma unroll
            for (int h = 1; h < L::QW; ++h) s += ypb[k][h][i];
            yv[j] = s;
            ss += s * s;
        }
        ss = wsum(ss);
        const double inv = ss > 0.0 ? 1.0 / sqrt(ss) : 0.0;
        double dmax = 0.0;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int i = lane + 64 * j;
            const double nv = yv[j] * inv;
            dmax = fmax(dmax, fabs(nv - xv[i]));
            xv[i] = nv;
        }
        dmax = wmax(dmax);
        return !(ss > 0.0) ? 2 : (dmax < 1e-14 ? 1 : 0);
    };

    // This wave's Gram pattern and the 16-column block of each operand slot
    // (off the diagonal, wave 1 takes rows 0-31 and tile (1, 1), wave 2 rows
    // 32-63 and tile (5, 5)).
    const bool diag = R0 == C0;
    int blk[GramOff::kSlots];
#pragma unroll
    for (int sl = 0; sl < GramOff::kSlots; ++sl)
        blk[sl] = diag ? R0 / 16 + min(sl, 3)
                       : (sl < 2 ? 2 * (wv - 1) + sl : (sl < 6 ? 2 + sl : (wv == 1 ? 1 : 5)));
    // Gram steps 0 .. steps-1 of the staged chunk (rows 4s .. 4s+3): slot
    // operands X[k][16 blk + lr] (at column 18 blk + lr + lr / 8 of the staged
    // layout) of the next step are read from LDS before this step's products
    // are issued (two operand sets used in turn), so the matrix cores do not
    // wait for them
    auto gram_steps = [&](auto pattern, int steps) __attribute__((always_inline)) {
        using P = decltype(pattern);
        double o0[P::kSlots], o1[P::kSlots];
        auto operands = [&](int st, double *o) {
            const int k = 4 * st + lk;
#pragma unroll
            for (int sl = 0; sl < P::kSlots; ++sl) o[sl] = xd[k * SP + 18 * blk[sl] + lr + (lr >> 3)];
        };
        auto products = [&](const double *o) {
#pragma unroll
            for (int u = 0; u < P::kTiles; ++u)
                Cm[u / 4][u % 4] = mfma16x16x4(o[P::ta[u]], o[P::tb[u]], Cm[u / 4][u % 4]);
        };
        // the next set is read even past the last step (a repeat of the last
        // one, unused), so the loads do not depend on the step count; the
        // scheduling barriers keep each set's loads ahead of the other set's
        // products, so every product waits only for operands read a step
        // earlier
        operands(0, o0);
        for (int st = 0; st < steps; st += 2) {
            operands(min(st + 1, steps - 1), o1);
            __builtin_amdgcn_sched_barrier(0);
            products(o0);
            __builtin_amdgcn_sched_barrier(0);
            operands(min(st + 2, steps - 1), o0);
            __builtin_amdgcn_sched_barrier(0);
            if (st + 1 < steps) products(o1);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto gram_to_lds = [&](auto pattern) __attribute__((always_inline)) {
        using P = decltype(pattern);
#pragma unroll
        for (int u = 0; u < P::kTiles; ++u) {
            const int bi = blk[P::ta[u]], bj = blk[P::tb[u]];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int i = 16 * bi + lk + 4 * q, j = 16 * bj + lr;
                xd[i * S + j] = Cm[u / 4][u % 4][q];
                if (bi != bj) xd[j * S + i] = Cm[u / 4][u % 4][q];
            }
        }
    };

    // every wave's quadrant of C from xd (row stride S); ends with a barrier
    auto quadrant_from_lds = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int q = 0; q < 4; ++q) Cm[a][b][q] = xd[(R0 + 16 * a + lk + 4 * q) * S + C0 + 16 * b + lr];
        __syncthreads();
    };
    // the upper tiles in Cm to their places in xd and the mirrored ones, then
    // every wave's quadrant back into Cm; begins and ends with a barrier
    auto symmetric_c = [&]() __attribute__((always_inline)) {
        __syncthreads();  // the products have read xd
        if constexpr (L::QW == 1)
            gram_to_lds(GramUpper{});
        else if (diag)
            gram_to_lds(GramDiag{});
        else
            gram_to_lds(GramOff{});
        __syncthreads();
        quadrant_from_lds();
    };
    // C <- C C / 2^e, e the exponent of the largest entry of C C.  C is
    // symmetric, so C C = C^T C is the Gram matrix of C's rows: C goes to xd
    // in the staged-row layout and the Gram pass's products make the upper
    // tiles.  Ends with a barrier.
    auto square = [&]() __attribute__((always_inline)) {
        __syncthreads();  // nobody reads xd any more
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = C0 + 16 * b + lr;
                    xd[(R0 + 16 * a + lk + 4 * q) * SP + c + (c >> 3)] = Cm[a][b][q];
                }
        __syncthreads();
        zero_c();
        if constexpr (L::QW == 1)
            gram_steps(GramUpper{}, HD / 4);
        else if (diag)
            gram_steps(GramDiag{}, HD / 4);
        else
            gram_steps(GramOff{}, HD / 4);
        symmetric_c();
        double m = 0.0;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int q = 0; q < 4; ++q) m = fmax(m, fabs(Cm[a][b][q]));
        m = wmax(m);
        if (lane == 0) red[t / 64] = m;
        __syncthreads();
        double mx = 0.0;
        for (int i = 0; i < NT / 64; ++i) mx = fmax(mx, red[i]);
        const double scale = mx > 0.0 ? ldexp(1.0, -ilogb(mx)) : 1.0;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) Cm[a][b] *= scale;
        __syncthreads();  // red and xd are free again
    };

    for (int i = t; i < HD; i += NT) acc[i] = 0.0;
    int worst = 0;
    for (int q = 0; q < r; ++q) {
        const char *xg = x + (size_t)(g * r + q) * stride * R::kBytes;
        // Column sums (their mean centres the keys; their dot with v signs a
        // query filter).  Thread (slot, part) always covers the same 16-byte
        // column slice `part`; its rows are summed in registers and the slots
        // meet in LDS.  Centred keys need the means before the Gram pass, so
        // they take a pass of their own; raw queries sum while staging.
        constexpr int kPer = CH * R::kLanes / NT;  // staged loads per thread per chunk
        const int part = t % R::kLanes, slot = t / R::kLanes;
        double csum[E];
#pragma unroll
        for (int e = 0; e < E; ++e) csum[e] = 0.0;
        auto reduce_sums = [&]() {
            __syncthreads();  // xd is free
#pragma unroll
            for (int e = 0; e < E; ++e) xd[slot * HD + part * E + e] = csum[e];
            __syncthreads();
            for (int c = t; c < HD; c += NT) {
                double s = 0.0;
                for (int j = 0; j < SLOTS; ++j) s += xd[j * HD + c];
                cs[c] = s;
                mu[c] = s / (double)n;  // a division, so that n equal rows centre to exact zeros
            }
            __syncthreads();
        };
        if constexpr (MODE == DIR_CENTRED_KEYS) {
            // kLoads rows in flight per thread; rows past n read row n - 1 and add nothing
            constexpr int kLoads = 8;
            for (int64_t row0 = slot; row0 < n; row0 += (int64_t)SLOTS * kLoads) {
                uint4 raw[kLoads];
#pragma unroll
                for (int u = 0; u < kLoads; ++u) {
                    const int64_t row = min(row0 + (int64_t)u * SLOTS, n - 1);
                    raw[u] = ld16(xg + (size_t)row * R::kBytes + part * 16);
                }
#pragma unroll
                for (int u = 0; u < kLoads; ++u) {
                    if (row0 + (int64_t)u * SLOTS >= n) break;
                    float f[E];
                    widen<DT>(raw[u], f);
#pragma unroll
                    for (int e = 0; e < E; ++e) csum[e] += (double)f[e];
                }
            }
            reduce_sums();
        }
        // Gram matrix of the (centred) rows: A = X^T and B = X, four rows a
        // step, upper tiles only (GramUpper / GramDiag / GramOff) accumulated
        // in the first entries of Cm.  The loads of chunk c + 1 are in flight
        // while chunk c is on the matrix cores; rows past a chunk read its last
        // row and are not used.
        zero_c();
        uint4 raw[kPer];
        auto fetch = [&](int64_t base) {
            const int rows = (int)min((int64_t)CH, n - base);
#pragma unroll
            for (int u = 0; u < kPer; ++u) {
                const int rr = min((t + u * NT) / R::kLanes, rows - 1);
                raw[u] = ld16(xg + (size_t)(base + rr) * R::kBytes + part * 16);
            }
        };
        fetch(0);
        for (int64_t base = 0; base < n; base += CH) {
            const int rows = (int)min((int64_t)CH, n - base);
            __syncthreads();  // the previous chunk's products have read xd
#pragma unroll
            for (int u = 0; u < kPer; ++u) {
                const int rr = (t + u * NT) / R::kLanes;
                if (rr >= rows) {  // past the chunk's end: zeros, so that steps need no bound checks
#pragma unroll
                    for (int k = 0; k < E; ++k) {
                        const int c = part * E + k;
                        xd[rr * SP + c + (c >> 3)] = 0.0;
                    }
                    continue;
                }
                float f[E];
                widen<DT>(raw[u], f);
#pragma unroll
                for (int k = 0; k < E; ++k) {
                    const int c = part * E + k;
                    if constexpr (MODE == DIR_CENTRED_KEYS) {
                        xd[rr * SP + c + (c >> 3)] = (double)f[k] - mu[c];
                    } else {
                        xd[rr * SP + c + (c >> 3)] = (double)f[k];
                        csum[k] += (double)f[k];
                    }
                }
            }
            if (base + CH < n) fetch(base + CH);
            __syncthreads();
            // steps of four rows (the last one padded with the zero rows); the
            // operands of the next step are read from LDS before this step's
            // products are issued, so the matrix cores do not wait for them
            const int steps = (rows + 3) >> 2;
            if constexpr (L::QW == 1)
                gram_steps(GramUpper{}, steps);
            else if (diag)
                gram_steps(GramDiag{}, steps);
            else
                gram_steps(GramOff{}, steps);
        }
        // C from the upper tiles: each tile to its place in xd and, off the
        // diagonal, its transpose to the mirrored place; then every wave loads
        // its whole quadrant into Cm
        symmetric_c();
        if constexpr (MODE == DIR_RAW_QUERIES) reduce_sums();  // begins with a barrier
        __syncthreads();

        // power iteration (power_step: every wave on its own copy of the
        // iterate, every wave taking the same decisions)
        for (int i = lane; i < HD; i += 64) vw[wv][i] = start_value(i, 0u);
        int calm = 0, it = 0, f = 0, squarings = 0;
        double power = 1.0;  // C now holds the original C to this power
        for (; it < max_iter; ++it) {
            f = power_step(it & 1);
            if (f == 2) break;
            calm = f == 1 ? calm + 1 : 0;
            if (calm >= 2) break;
            if ((it + 1) % L::SQUARE_EVERY == 0 && squarings < L::MAX_SQUARINGS) {
                square();
                ++squarings;
                power *= 2.0;
                calm = 0;
            }
        }
        if (wv == 0)
            for (int i = lane; i < HD; i += 64) v[i] = vw[0][i];
        __syncthreads();
        int st = f == 2 ? 2 : (calm >= 2 ? 0 : 1);
        double fro_all = 0.0;  // |C|_F^2 of the current C, summed over the workgroup
        if (st == 0) {
            // Separation check: equal top eigenvalues (lambda2 >= lambda1 (1 -
            // 1e-9)) are reported as status 1; on the p-th power of C that is a
            // ratio of 1 - p 1e-9.  lambda1 is the Rayleigh quotient of v.  C is a
            // Gram matrix (symmetric, positive semi-definite), so lambda2^2 <=
            // sum_{i>=2} lambda_i^2 = |C|_F^2 - lambda1^2: when that is below
            // the tie threshold the separation is certified at once.  If not,
            // and the same bound on C^2 can still pass (by Cauchy-Schwarz it
            // cannot once (sum_{i>=2} lambda_i^2)^2 / (D - 1) reaches lambda1^4),
            // C is squared and the bound tried again.  Otherwise lambda2 is
            // approached from below by power iteration on the complement of v (w
            // kept orthogonal to v), for at most kSepSteps steps: a tie whose
            // eigenvalues stand clear of the rest shows within a few steps; top
            // eigenvalues that are close but not tied have already kept the main
            // iteration from converging.
            bool certified = false;
            for (int round = 0; round < 2 && !certified; ++round) {
                if (round == 1) {
                    const double l1 = lam[0], rest = fro_all - l1 * l1;
                    const double lim2 = l1 * l1 * (1.0 - 2e-9 * power);
                    if (!(rest * rest < (double)(HD - 1) * lim2 * lim2)) break;  // C^2 cannot pass either
                    square();
                    power *= 2.0;
                }
                matvec(v);
                if (t < 64) {
                    gather_y();
                    const double l1 = wdot(v, y);
                    if (lane == 0) lam[0] = l1;
                }
                double fro = 0.0;  // this lane's part of |C|_F^2
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int b = 0; b < 4; ++b)
#pragma unroll
                        for (int qq = 0; qq < 4; ++qq) fro = __builtin_fma(Cm[a][b][qq], Cm[a][b][qq], fro);
                fro = wsum(fro);
                if (lane == 0) fr[wv] = fro;
                __syncthreads();
                fro_all = 0.0;
                for (int i = 0; i < NT / 64; ++i) fro_all += fr[i];
                const double l1 = lam[0], lim = l1 * (1.0 - 1e-9 * power);
                certified = l1 > 0.0 && fro_all - l1 * l1 < lim * lim;
                __syncthreads();  // fr and lam are read before they are written again
            }
            start(w, 0x9E3779B9u);
            __syncthreads();
            if (t < 64 && !certified) renorm(w, w, v);  // orthogonalise and normalise the start
            __syncthreads();
            int calm2 = 0;
            constexpr int kSepSteps = 48;
            for (int it2 = 0; it2 < (certified ? 0 : kSepSteps); ++it2) {
                matvec(w);
                if (t < 64) {
                    gather_y();
                    const double l2 = wdot(w, y);
                    const int rc = renorm(w, y, v);
                    if (lane == 0) {
                        lam[1] = l2;
                        flag = rc;
                    }
                }
                __syncthreads();
                const int f2 = flag;
                const bool tied = lam[1] >= lam[0] * (1.0 - 1e-9 * power);
                if (tied) {
                    st = 1;
                    break;
                }
                if (f2 == 2) break;  // nothing outside v: rank one
                calm2 = f2 == 1 ? calm2 + 1 : 0;
                if (calm2 >= 2) break;
            }
        }
        worst = max(worst, st);
        // sign, then accumulate the signed unit vector
        if (t < 64) {
            double sg;
            if constexpr (MODE == DIR_CENTRED_KEYS) {
                // the entry of largest magnitude positive, lowest index on ties
                double best = -1.0;
                int bi = HD;
                for (int i = lane; i < HD; i += 64) {
                    const double m = fabs(v[i]);
                    if (m > best) {
                        best = m;
                        bi = i;
                    }
                }
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) {
                    const double ob = shfl_xor_f64(best, off);
                    const int oi = __shfl_xor(bi, off);
                    if (ob > best || (ob == best && oi < bi)) {
                        best = ob;
                        bi = oi;
                    }
                }
                sg = v[bi] > 0.0 ? 1.0 : -1.0;
            } else {
                sg = wdot(cs, v) >= 0.0 ? 1.0 : -1.0;  // sgn(1^T u1), +1 at zero
            }
            for (int i = lane; i < HD; i += 64) acc[i] += sg * v[i];
        }
        __syncthreads();
    }
    if (t < 64) {
        if constexpr (MODE == DIR_CENTRED_KEYS) {
            for (int i = lane; i < HD; i += 64) out[(size_t)g * HD + i] = (float)acc[i];
        } else {
            for (int i = lane; i < HD; i += 64) acc[i] *= 1.0 / (double)r;
            const double nrm = sqrt(wdot(acc, acc));
            if (nrm == 0.0 && worst == 0) worst = 3;
            const double inv = nrm > 0.0 ? 1.0 / nrm : 0.0;
            for (int i = lane; i < HD; i += 64) out[(size_t)g * HD + i] = (float)(acc[i] * inv);
        }
        if (lane == 0) status[g] = worst;
    }
}

template <int MODE>
int launch_direction(const char *what, const void *x, int32_t dtype, int64_t groups, int64_t r, int64_t n,
                     int64_t stride, int64_t D, float *out, int32_t *status, int32_t max_iter, void *stream) {
    if (D != 64 && D != 128)
        return set_error(KVX_ERANGE, "%s: head dim %lld (64 or 128 on the device)", what, (long long)D);
    if (dtype != KVX_BF16 && dtype != KVX_F16 && dtype != KVX_F32)
        return set_error(KVX_EINVAL, "%s: bad dtype %d", what, (int)dtype);
    if (groups == 0) return KVX_OK;
    if (!x || !out || !status) return set_error(KVX_EINVAL, "%s: NULL buffer", what);
    if (groups > INT32_MAX) return set_error(KVX_ERANGE, "%s: too many groups", what);
    const kvx_shape sh{1, 1, 1, D, dtype};
    hipStream_t st = (hipStream_t)stream;
    dispatch_row(sh, false, [&](auto dt, auto hd) {
        constexpr int HD = decltype(hd)::value;
        if constexpr (HD <= 128)
            top_direction_kernel<decltype(dt)::value, HD, MODE><<<(uint32_t)groups, DirLayout<HD>::NT, 0, st>>>(
                (const char *)x, stride, (int)r, n, out, status, (int)max_iter);
        return 0;
    });
    return check_launch(what);
}

}  // namespace
}  // namespace kvx

using namespace kvx;

extern "C" {

KVX_API int kv_passthrough_append(const void *k_held, const void *v_held, int64_t n_held, int64_t cap_held,
                                  const void *k_new, const void *v_new, int64_t S, kvx_shape shape, void *k_out,
                                  void *v_out, int32_t *pos_out, int64_t cap_out, void *stream) {
    clear_error();
    int64_t G = 0;
    int rc = check_shape(shape, &G);
    if (rc) return rc;
    if (n_held < 0 || S < 0 || cap_held < 0 || cap_out < 0 || n_held > cap_held || n_held + S > cap_out)
        return set_error(KVX_EINVAL, "kv_passthrough_append: need 0 <= n_held <= cap_held and n_held + S <= cap_out "
                         "(n_held %lld, cap_held %lld, S %lld, cap_out %lld)", (long long)n_held, (long long)cap_held,
                         (long long)S, (long long)cap_out);
    if (n_held + S > INT32_MAX) return set_error(KVX_ERANGE, "kv_passthrough_append: positions beyond int32");
    if (G == 0 || n_held + S == 0) return KVX_OK;
    if (!k_out || !v_out || !pos_out || (S > 0 && (!k_new || !v_new)) || (n_held > 0 && (!k_held || !v_held)))
        return set_error(KVX_EINVAL, "kv_passthrough_append: NULL buffer");
    const size_t row = (size_t)shape.D * (shape.dtype == KVX_F32 ? 4 : 2);
    const bool alias = k_out == k_held && v_out == v_held && cap_out == cap_held;
    auto overlap = [](const void *a, size_t na, const void *b, size_t nb) {
        const char *x = (const char *)a, *y = (const char *)b;
        return a && b && na && nb && x < y + nb && y < x + na;
    };
    const size_t out_b = (size_t)G * cap_out * row, held_b = (size_t)G * cap_held * row,
                 new_b = (size_t)G * S * row;
    if (!alias && n_held > 0 &&
        (overlap(k_out, out_b, k_held, held_b) || overlap(k_out, out_b, v_held, held_b) ||
         overlap(v_out, out_b, k_held, held_b) || overlap(v_out, out_b, v_held, held_b)))
        return set_error(KVX_EINVAL, "kv_passthrough_append: output overlaps the held rows without being them");
    if (overlap(k_out, out_b, k_new, new_b) || overlap(k_out, out_b, v_new, new_b) ||
        overlap(v_out, out_b, k_new, new_b) || overlap(v_out, out_b, v_new, new_b) ||
        overlap(k_out, out_b, v_out, out_b))
        return set_error(KVX_EINVAL, "kv_passthrough_append: output overlaps the new rows or itself");
    const int64_t first = alias ? n_held : 0;
    const int64_t lanes = G * (n_held + S - first) * (int64_t)(row / 16);
    if (lanes == 0) return KVX_OK;
    const uint32_t grid = (uint32_t)std::min<int64_t>((lanes + 255) / 256, 65536);
    hipStream_t st = (hipStream_t)stream;
    dispatch_row(shape, true, [&](auto dt, auto hd) {
        append_rows_kernel<decltype(dt)::value, decltype(hd)::value><<<grid, 256, 0, st>>>(
            (const char *)k_held, (const char *)v_held, cap_held, n_held, (const char *)k_new, (const char *)v_new,
            S, (char *)k_out, (char *)v_out, pos_out, cap_out, first, G);
        return 0;
    });
    return check_launch("kv_passthrough_append");
}

KVX_API int qf_filters_from_keys_device(const void *k, int32_t dtype, int64_t G, int64_t n, int64_t group_stride,
                                        int64_t D, float *out, int32_t *status, int32_t max_iter, void *stream) {
    clear_error();
    if (G < 0 || n < 2 || n > KVX_MAX_TOTAL || group_stride < n || max_iter < 1)
        return set_error(KVX_EINVAL, "qf_filters_from_keys_device: need G >= 0, 2 <= n <= %d, group_stride >= n, "
                         "max_iter >= 1 (n %lld, group_stride %lld, max_iter %d)", KVX_MAX_TOTAL, (long long)n,
                         (long long)group_stride, (int)max_iter);
    return launch_direction<DIR_CENTRED_KEYS>("qf_filters_from_keys_device", k, dtype, G, 1, n, group_stride, D, out,
                                              status, max_iter, stream);
}

KVX_API int qf_filters_from_queries_device(const void *q, int32_t dtype, int64_t L, int64_t H_q, int64_t N,
                                           int64_t D, int64_t H_kv, float *out, int32_t *status, int32_t max_iter,
                                           void *stream) {
    clear_error();
    if (L < 0 || H_q < 1 || H_kv < 1 || H_q % H_kv || N < 1 || N > KVX_MAX_TOTAL || max_iter < 1)
        return set_error(KVX_EINVAL, "qf_filters_from_queries_device: need L >= 0, H_q a multiple of H_kv >= 1, "
                         "1 <= N <= %d, max_iter >= 1 (L %lld, H_q %lld, H_kv %lld, N %lld)", KVX_MAX_TOTAL,
                         (long long)L, (long long)H_q, (long long)H_kv, (long long)N);
    if (L > INT32_MAX / H_kv) return set_error(KVX_ERANGE, "qf_filters_from_queries_device: too many groups");
    return launch_direction<DIR_RAW_QUERIES>("qf_filters_from_queries_device", q, dtype, L * H_kv, H_q / H_kv, N, N,
                                             D, out, status, max_iter, stream);
}

}  // extern "C"
