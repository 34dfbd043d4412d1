// Row-level device helpers and launch plumbing shared by the library's HIP
// translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kvevict.h"
#include "kvx_common.h"

namespace kvx {
namespace {

// A K/V row of HD elements of type DT, read 16 bytes per lane.
template <int DT, int HD>
struct Row {
    static constexpr int kElemBytes = DT == KVX_F32 ? 4 : 2;
    static constexpr int kBytes = HD * kElemBytes;    // e.g. 256 B for a bf16 row of 128
    static constexpr int kLanes = kBytes / 16;        // lanes covering one row, 16 B each
    static constexpr int kElemsPerLane = 16 / kElemBytes;
    static_assert(kLanes >= 1 && kLanes <= 64 && (kLanes & (kLanes - 1)) == 0,
                  "a row spans a power-of-two number of lanes of one wave");
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 to_uint4(u32x4 v) { return make_uint4(v.x, v.y, v.z, v.w); }

template <bool NT = false>
__device__ __forceinline__ uint4 ld16(const char *p) {
    if constexpr (NT)
        return to_uint4(__builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p)));
    else
        return to_uint4(*reinterpret_cast<const u32x4 *>(p));
}
template <bool NT = false>
__device__ __forceinline__ void st16(char *p, uint4 v) {
    const u32x4 w = {v.x, v.y, v.z, v.w};
    if constexpr (NT)
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(p));
    else
        *reinterpret_cast<u32x4 *>(p) = w;
}

// Widen the 16 bytes a lane holds to float32 (exact for every element type).
template <int DT>
__device__ __forceinline__ void widen(uint4 r, float *x) {
    if constexpr (DT == KVX_F16) {
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = (float)__builtin_bit_cast(_Float16, (unsigned short)(w[i] & 0xFFFFu));
            x[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (unsigned short)(w[i] >> 16));
        }
    } else if constexpr (DT == KVX_BF16) {
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(w[i] << 16);           // element 2i   (low half)
            x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);  // element 2i+1 (high half)
        }
    } else {
        x[0] = __uint_as_float(r.x);
        x[1] = __uint_as_float(r.y);
        x[2] = __uint_as_float(r.z);
        x[3] = __uint_as_float(r.w);
    }
}

// Validates a shape (sizes, head dim, element type) and returns its group count.
inline int check_shape(const kvx_shape &sh, int64_t *G) {
    if (sh.L < 0 || sh.B < 0 || sh.H < 0)
        return set_error(KVX_EINVAL, "shape: L, B, H must be >= 0 (got %lld, %lld, %lld)",
                         (long long)sh.L, (long long)sh.B, (long long)sh.H);
    if (sh.D != 64 && sh.D != 128 && sh.D != 256)
        return set_error(KVX_EINVAL, "shape: D must be 64, 128 or 256 (got %lld)", (long long)sh.D);
    if (sh.dtype != KVX_BF16 && sh.dtype != KVX_F32 && sh.dtype != KVX_F16)
        return set_error(KVX_EINVAL, "shape: dtype must be KVX_BF16, KVX_F16 or KVX_F32 (got %d)", (int)sh.dtype);
    if (sh.L > INT32_MAX || sh.B > INT32_MAX || sh.H > INT32_MAX ||
        (sh.L > 0 && sh.B > 0 && sh.H > 0 && sh.L * sh.B > INT32_MAX / sh.H))
        return set_error(KVX_ERANGE, "shape: L*B*H must be below 2^31");
    *G = sh.L * sh.B * sh.H;
    return KVX_OK;
}

// Launch status of the last kernel on this thread, as a library status.
inline int check_launch(const char *what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return set_error(KVX_EDEVICE, "%s: launch failed: %s", what, hipGetErrorString(e));
    return KVX_OK;
}

// Calls f(DT, HD) with compile-time constants for the shape's element type and
// head dim.  `copy_only` maps fp16 onto bf16 (same row bytes) for kernels that
// only move rows.
template <class F>
int dispatch_row(const kvx_shape &sh, bool copy_only, F &&f) {
    using bf = std::integral_constant<int, KVX_BF16>;
    using hf = std::integral_constant<int, KVX_F16>;
    using fp = std::integral_constant<int, KVX_F32>;
    auto by_d = [&](auto dt) -> int {
        switch (sh.D) {
            case 64: return f(dt, std::integral_constant<int, 64>{});
            case 128: return f(dt, std::integral_constant<int, 128>{});
            default: return f(dt, std::integral_constant<int, 256>{});
        }
    };
    if (sh.dtype == KVX_F32) return by_d(fp{});
    if (sh.dtype == KVX_F16 && !copy_only) return by_d(hf{});
    return by_d(bf{});
}

}  // namespace
}  // namespace kvx
