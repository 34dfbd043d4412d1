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
// Both are the top eigenvector of a Gram matrix C = X^T X (X centred or raw).
// One workgroup per group: a pass over the rows for the fp64 column sums, a
// pass that stages chunks of rows (centred when asked) in LDS as fp64 and
// accumulates C in 8 x 8 fp64 register tiles, then power iteration with C held
// in registers, and a bounded second iteration on the complement of the found
// vector that checks that the top eigenvalue is separated.  When the iteration
// is slow (top two eigenvalues close), C is squared in place every 32 steps (up
// to 2^10-th powers, rescaled by a power of two): the eigenvectors stay, the
// ratio of the top two eigenvalues is squared.
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

template <int HD>
struct DirLayout {
    static constexpr int T = 8;            // Gram tile edge per thread
    static constexpr int TPR = HD / T;     // threads along one tile row
    static constexpr int NT = TPR * TPR;   // 64 threads for HD 64, 256 for HD 128
    static constexpr int CH = HD;          // staged rows per chunk: an HD x HD fp64 square of LDS
    static constexpr int SQUARE_EVERY = 32;  // power steps between squarings of C
    static constexpr int MAX_SQUARINGS = 10;
    static_assert(NT >= 64 && NT <= 256, "the device estimator covers head dims 64 and 128");
};

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
    constexpr int NT = L::NT, TPR = L::TPR, CH = L::CH, E = R::kElemsPerLane, SLOTS = NT / R::kLanes;
    static_assert(SLOTS >= 1 && NT % R::kLanes == 0, "a workgroup covers whole rows");
    static_assert(SLOTS <= CH, "the column partial sums fit the staging buffer");
    __shared__ double xd[CH * HD];  // staged rows, or C while it is squared; first the column partial sums
    __shared__ double cs[HD], v[HD], y[HD], w[HD], acc[HD], lam[2], red[NT / 64];
    __shared__ int flag;
    const int t = threadIdx.x, lane = t & 63;
    const int64_t g = blockIdx.x;
    const int tr = t / TPR, tc = t % TPR, r0 = tr * L::T, c0 = tc * L::T;

    // y = C x over the register tiles (x, y in LDS); ends with a barrier
    double C[L::T][L::T];
    auto matvec = [&](const double *xv, double *yv) {
        double p[L::T];
#pragma unroll
        for (int i = 0; i < L::T; ++i) {
            double s = 0.0;
#pragma unroll
            for (int j = 0; j < L::T; ++j) s = __builtin_fma(C[i][j], xv[c0 + j], s);
            p[i] = s;
        }
#pragma unroll
        for (int off = TPR / 2; off > 0; off >>= 1)
#pragma unroll
            for (int i = 0; i < L::T; ++i) p[i] += shfl_xor_f64(p[i], off);
        if (tc == 0)
#pragma unroll
            for (int i = 0; i < L::T; ++i) yv[r0 + i] = p[i];
        __syncthreads();
    };
    // wave-0 reductions and vector updates over HD-long LDS vectors
    auto wsum = [&](double s) {
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) s += shfl_xor_f64(s, off);
        return s;
    };
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
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) dmax = fmax(dmax, shfl_xor_f64(dmax, off));
        return !(ss > 0.0) ? 2 : (dmax < 1e-14 ? 1 : 0);
    };
    // C <- C C / 2^e (C symmetric: row k of C is column k), e the exponent of
    // the largest entry of C C; ends with a barrier
    auto square = [&]() {
        __syncthreads();  // nobody reads xd any more
#pragma unroll
        for (int i = 0; i < L::T; ++i)
#pragma unroll
            for (int j = 0; j < L::T; ++j) xd[(r0 + i) * HD + c0 + j] = C[i][j];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < L::T; ++i)
#pragma unroll
            for (int j = 0; j < L::T; ++j) C[i][j] = 0.0;
        for (int k = 0; k < HD; ++k) {
            double a[L::T], b[L::T];
#pragma unroll
            for (int i = 0; i < L::T; ++i) {
                a[i] = xd[k * HD + r0 + i];
                b[i] = xd[k * HD + c0 + i];
            }
#pragma unroll
            for (int i = 0; i < L::T; ++i)
#pragma unroll
                for (int j = 0; j < L::T; ++j) C[i][j] = __builtin_fma(a[i], b[j], C[i][j]);
        }
        double m = 0.0;
#pragma unroll
        for (int i = 0; i < L::T; ++i)
#pragma unroll
            for (int j = 0; j < L::T; ++j) m = fmax(m, fabs(C[i][j]));
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) m = fmax(m, shfl_xor_f64(m, off));
        if (lane == 0) red[t / 64] = m;
        __syncthreads();
        double mx = 0.0;
        for (int i = 0; i < NT / 64; ++i) mx = fmax(mx, red[i]);
        const double scale = mx > 0.0 ? ldexp(1.0, -ilogb(mx)) : 1.0;
#pragma unroll
        for (int i = 0; i < L::T; ++i)
#pragma unroll
            for (int j = 0; j < L::T; ++j) C[i][j] *= scale;
        __syncthreads();  // red and xd are free again
    };
    // a fixed, generic start vector
    auto start = [&](double *xv, uint32_t salt) {
        for (int i = t; i < HD; i += NT) {
            const uint32_t h = ((uint32_t)(i + 1) ^ salt) * 2654435761u;
            xv[i] = ((h >> 31) ? -1.0 : 1.0) * (0.5 + (double)((h >> 8) & 0xFFFF) / 65536.0);
        }
    };

    for (int i = t; i < HD; i += NT) acc[i] = 0.0;
    int worst = 0;
    for (int q = 0; q < r; ++q) {
        const char *xg = x + (size_t)(g * r + q) * stride * R::kBytes;
        // column sums: thread (slot, part) sums rows slot, slot + SLOTS, ...
        {
            const int part = t % R::kLanes, slot = t / R::kLanes;
            double a[E];
#pragma unroll
            for (int e = 0; e < E; ++e) a[e] = 0.0;
            for (int64_t row = slot; row < n; row += SLOTS) {
                float f[E];
                widen<DT>(ld16(xg + (size_t)row * R::kBytes + part * 16), f);
#pragma unroll
                for (int e = 0; e < E; ++e) a[e] += (double)f[e];
            }
            __syncthreads();  // the previous head is done with xd
#pragma unroll
            for (int e = 0; e < E; ++e) xd[slot * HD + part * E + e] = a[e];
            __syncthreads();
            for (int c = t; c < HD; c += NT) {
                double s = 0.0;
                for (int j = 0; j < SLOTS; ++j) s += xd[j * HD + c];
                cs[c] = s;
            }
            __syncthreads();
        }
        // Gram matrix of the (centred) rows, tile (r0.., c0..) of 8 x 8 per thread
#pragma unroll
        for (int i = 0; i < L::T; ++i)
#pragma unroll
            for (int j = 0; j < L::T; ++j) C[i][j] = 0.0;
        const double inv_n = 1.0 / (double)n;
        for (int64_t base = 0; base < n; base += CH) {
            const int rows = (int)min((int64_t)CH, n - base);
            for (int e = t; e < rows * R::kLanes; e += NT) {
                const int rr = e / R::kLanes, part = e % R::kLanes;
                float f[E];
                widen<DT>(ld16(xg + (size_t)(base + rr) * R::kBytes + part * 16), f);
#pragma unroll
                for (int k = 0; k < E; ++k) {
                    const int c = part * E + k;
                    xd[rr * HD + c] = MODE == DIR_CENTRED_KEYS ? (double)f[k] - cs[c] * inv_n : (double)f[k];
                }
            }
            __syncthreads();
            for (int rr = 0; rr < rows; ++rr) {
                double a[L::T], b[L::T];
#pragma unroll
                for (int i = 0; i < L::T; ++i) {
                    a[i] = xd[rr * HD + r0 + i];
                    b[i] = xd[rr * HD + c0 + i];
                }
#pragma unroll
                for (int i = 0; i < L::T; ++i)
#pragma unroll
                    for (int j = 0; j < L::T; ++j) C[i][j] = __builtin_fma(a[i], b[j], C[i][j]);
            }
            __syncthreads();
        }

        // power iteration; `flag` carries wave 0's verdict to the workgroup
        start(v, 0u);
        __syncthreads();
        int calm = 0, it = 0, f = 0, squarings = 0;
        double power = 1.0;  // C now holds the original C to this power
        for (; it < max_iter; ++it) {
            matvec(v, y);
            if (t < 64) {
                const int rc = renorm(v, y, nullptr);
                if (lane == 0) flag = rc;
            }
            __syncthreads();
            f = flag;
            __syncthreads();  // every thread has read flag before wave 0 rewrites it
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
        int st = f == 2 ? 2 : (calm >= 2 ? 0 : 1);
        if (st == 0) {
            // Separation check: lambda1 is the Rayleigh quotient of v; lambda2 is
            // approached from below by power iteration on the complement of v
            // (w kept orthogonal to v), for at most as many steps again.  Equal
            // top eigenvalues (lambda2 >= lambda1 (1 - 1e-9)) are reported as
            // status 1; on the p-th power of C that is a ratio of 1 - p 1e-9.
            matvec(v, y);
            if (t < 64) {
                const double l1 = wdot(v, y);
                if (lane == 0) lam[0] = l1;
            }
            start(w, 0x9E3779B9u);
            __syncthreads();
            if (t < 64) renorm(w, w, v);  // orthogonalise and normalise the start
            __syncthreads();
            int calm2 = 0;
            for (int it2 = 0; it2 < it + 64; ++it2) {
                matvec(w, y);
                if (t < 64) {
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
                __syncthreads();
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
