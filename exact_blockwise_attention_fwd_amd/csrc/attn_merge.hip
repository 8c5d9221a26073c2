// Merge of two partial attention results over disjoint key sets:
//     M = max(lse_a, lse_b), w_x = exp(lse_x - M), O = (w_a O_a + w_b O_b) / (w_a + w_b),
//     lse = M + ln(w_a + w_b), and (0, -inf) when both parts are empty.
// This is the associative combination of per-fragment statistics in the "ATTENTION2D" explainer
// (sections 2 and 3), with the rescale rule of "FlashAttention by hand" (paragraph on rescaling).
//
// The merge streams rows * d elements and is bound by HBM bandwidth; the weights are computed per vector
// from the two lse values (cheap next to the memory traffic).  Two kernels:
//  - rows_kernel, for d a multiple of 4 up to 256 with vector-aligned buffers: every row belongs to one
//    wave, a power-of-two group of lanes per row, one 4-element vector per lane; each lane keeps U rows in
//    flight.  Streams larger than twice the 256 MB Infinity Cache use non-temporal loads and stores,
//    smaller ones plain ones (measured: each is 8-16 % faster on its side of that size).
//  - merge_kernel, for any other d or alignment: a workgroup processes whole rows at a time.
// In-place use (O == O_a, lse == lse_a) is safe in both: every output vector is written by the lane that
// read it.  In rows_kernel a row's lse is read by the lanes of one wave in one load instruction and
// written by one of them with a value computed from that load, so after every read of it; merge_kernel
// writes a row's lse only after a workgroup barrier that follows every read of it.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "attn_internal.h"

namespace attn {
namespace {

constexpr int M_THREADS = 256;

__device__ __forceinline__ float bf16_to_f32(uint16_t x) { return __uint_as_float((unsigned)x << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    __bf16 b = (__bf16)f;   // round to nearest even
    return __builtin_bit_cast(uint16_t, b);
}

template <bool IN_BF16, int VEC>
__device__ __forceinline__ void load_vec(const void* p, size_t idx, float (&x)[VEC]) {
    if constexpr (IN_BF16) {
        const uint16_t* s = static_cast<const uint16_t*>(p) + idx;
        if constexpr (VEC == 4) {
            const uint2 u = *reinterpret_cast<const uint2*>(s);
            x[0] = __uint_as_float(u.x << 16); x[1] = __uint_as_float(u.x & 0xffff0000u);
            x[2] = __uint_as_float(u.y << 16); x[3] = __uint_as_float(u.y & 0xffff0000u);
        } else {
            for (int e = 0; e < VEC; ++e) x[e] = bf16_to_f32(s[e]);
        }
    } else {
        const float* s = static_cast<const float*>(p) + idx;
        if constexpr (VEC == 4) {
            const float4 u = *reinterpret_cast<const float4*>(s);
            x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
        } else {
            for (int e = 0; e < VEC; ++e) x[e] = s[e];
        }
    }
}

template <bool OUT_BF16, int VEC>
__device__ __forceinline__ void store_vec(void* p, size_t idx, const float (&x)[VEC]) {
    if constexpr (OUT_BF16) {
        uint16_t* s = static_cast<uint16_t*>(p) + idx;
        if constexpr (VEC == 4) {
            uint2 u;
            u.x = (unsigned)f32_to_bf16(x[0]) | ((unsigned)f32_to_bf16(x[1]) << 16);
            u.y = (unsigned)f32_to_bf16(x[2]) | ((unsigned)f32_to_bf16(x[3]) << 16);
            *reinterpret_cast<uint2*>(s) = u;
        } else {
            for (int e = 0; e < VEC; ++e) s[e] = f32_to_bf16(x[e]);
        }
    } else {
        float* s = static_cast<float*>(p) + idx;
        if constexpr (VEC == 4) {
            *reinterpret_cast<float4*>(s) = make_float4(x[0], x[1], x[2], x[3]);
        } else {
            for (int e = 0; e < VEC; ++e) s[e] = x[e];
        }
    }
}

template <bool IN_BF16, bool OUT_BF16, int VEC>
__global__ __launch_bounds__(M_THREADS) void merge_kernel(MergeArgs a, int vpr, int rows_per_iter) {
    const int tid = threadIdx.x;
    const long long step = (long long)gridDim.x * rows_per_iter;
    for (long long rb = (long long)blockIdx.x * rows_per_iter; rb < a.rows; rb += step) {
        // this workgroup owns rows [rb, rb + rows_per_iter)
        float my_la = -INFINITY, my_lb = -INFINITY;
        const bool writes_lse = tid < rows_per_iter && rb + tid < a.rows;
        if (writes_lse) {
            my_la = a.lse_a[rb + tid];
            my_lb = a.lse_b[rb + tid];
        }
        for (int v = tid; v < rows_per_iter * vpr; v += M_THREADS) {
            const long long row = rb + v / vpr;
            if (row >= a.rows) break;
            const int c0 = (v % vpr) * VEC;
            const float la = a.lse_a[row], lb = a.lse_b[row];
            const float big = fmaxf(la, lb);
            float wa = 0.f, wb = 0.f;
            if (big != -INFINITY) {
                wa = expf(la - big);
                wb = expf(lb - big);
                const float inv = 1.f / (wa + wb);
                wa *= inv;
                wb *= inv;
            }
            const size_t idx = (size_t)row * a.d + c0;
            float x[VEC], y[VEC];
            load_vec<IN_BF16, VEC>(a.o_a, idx, x);
            load_vec<IN_BF16, VEC>(a.o_b, idx, y);
#pragma unroll
            for (int e = 0; e < VEC; ++e) x[e] = wa * x[e] + wb * y[e];
            store_vec<OUT_BF16, VEC>(a.o, idx, x);
        }
        __syncthreads();   // every read of these rows' lse precedes the writes below
        if (writes_lse) {
            const float big = fmaxf(my_la, my_lb);
            a.lse[rb + tid] = big == -INFINITY ? -INFINITY
                                               : big + logf(expf(my_la - big) + expf(my_lb - big));
        }
    }
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

template <bool IN_BF16, bool NT>
__device__ __forceinline__ f32x4 load4(const void* base, size_t idx) {
    if constexpr (IN_BF16) {
        const u32x2* p = reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(base) + idx);
        u32x2 u;
        if constexpr (NT) u = __builtin_nontemporal_load(p);
        else u = *p;
        return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xffff0000u)};
    } else {
        const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + idx);
        if constexpr (NT) return __builtin_nontemporal_load(p);
        else return *p;
    }
}

template <bool OUT_BF16, bool NT>
__device__ __forceinline__ void store4(void* base, size_t idx, f32x4 x) {
    if constexpr (OUT_BF16) {
        u32x2 u;
        u.x = (unsigned)f32_to_bf16(x.x) | ((unsigned)f32_to_bf16(x.y) << 16);
        u.y = (unsigned)f32_to_bf16(x.z) | ((unsigned)f32_to_bf16(x.w) << 16);
        u32x2* p = reinterpret_cast<u32x2*>(static_cast<uint16_t*>(base) + idx);
        if constexpr (NT) __builtin_nontemporal_store(u, p);
        else *p = u;
    } else {
        f32x4* p = reinterpret_cast<f32x4*>(static_cast<float*>(base) + idx);
        if constexpr (NT) __builtin_nontemporal_store(x, p);
        else *p = x;
    }
}

// Lane l of a wave handles column vector (l mod 2^lpr_log2) of row (l >> lpr_log2) of each of its U row
// groups; wave group g covers rows [g*U*rpw, (g+1)*U*rpw) with rpw = 64 >> lpr_log2 rows per group.
template <bool IN_BF16, bool OUT_BF16, int U, bool NT>
__global__ __launch_bounds__(M_THREADS) void rows_kernel(MergeArgs a, int lpr_log2, long long groups) {
    const int lane = threadIdx.x & 63;
    const int rpw = 64 >> lpr_log2;
    const int r = lane >> lpr_log2, c = lane & ((1 << lpr_log2) - 1);
    const bool col_ok = 4 * c < a.d;
    const long long waves = (long long)gridDim.x * (M_THREADS / 64);
    for (long long g = (long long)blockIdx.x * (M_THREADS / 64) + (threadIdx.x >> 6); g < groups; g += waves) {
        const long long row0 = g * U * rpw + r;
        float la[U], lb[U];
        f32x4 x[U], y[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {   // every load of the U rows is issued before any arithmetic
            const long long row = row0 + (long long)u * rpw;
            la[u] = lb[u] = -INFINITY;
            x[u] = y[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (row < a.rows) {
                la[u] = a.lse_a[row];
                lb[u] = a.lse_b[row];
                if (col_ok) {
                    const size_t idx = (size_t)row * a.d + 4 * c;
                    x[u] = load4<IN_BF16, NT>(a.o_a, idx);
                    y[u] = load4<IN_BF16, NT>(a.o_b, idx);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const long long row = row0 + (long long)u * rpw;
            if (row >= a.rows) continue;
            const float big = fmaxf(la[u], lb[u]);
            float wa = 0.f, wb = 0.f;
            if (big != -INFINITY) {
                wa = expf(la[u] - big);
                wb = expf(lb[u] - big);
                const float inv = 1.f / (wa + wb);
                wa *= inv;
                wb *= inv;
            }
            if (col_ok) store4<OUT_BF16, NT>(a.o, (size_t)row * a.d + 4 * c, wa * x[u] + wb * y[u]);
            if (c == 0)
                a.lse[row] = big == -INFINITY ? -INFINITY : big + logf(expf(la[u] - big) + expf(lb[u] - big));
        }
    }
}

template <bool IN_BF16, bool OUT_BF16, int U, bool NT>
hipError_t launch_rows(const MergeArgs& a, int lpr_log2, hipStream_t s) {
    const long long per_group = (long long)U * (64 >> lpr_log2);
    const long long groups = (a.rows + per_group - 1) / per_group;
    long long blocks = (groups + M_THREADS / 64 - 1) / (M_THREADS / 64);
    if (blocks > (1LL << 20)) blocks = 1LL << 20;   // beyond that the waves loop over their groups
    hipLaunchKernelGGL((rows_kernel<IN_BF16, OUT_BF16, U, NT>), dim3((unsigned)blocks), dim3(M_THREADS), 0, s, a,
                       lpr_log2, groups);
    return hipGetLastError();
}

template <bool IN_BF16, bool OUT_BF16>
hipError_t launch_t(const MergeArgs& a, hipStream_t s) {
    const size_t in_align = IN_BF16 ? 8 : 16, out_align = OUT_BF16 ? 8 : 16;
    const bool aligned = ((uintptr_t)a.o_a % in_align) == 0 && ((uintptr_t)a.o_b % in_align) == 0 &&
                         ((uintptr_t)a.o % out_align) == 0;
    if (aligned && a.d % 4 == 0 && a.d <= 256) {
        int lpr_log2 = 0;
        while ((4 << lpr_log2) < a.d) ++lpr_log2;
        const double bytes = (double)a.rows * (a.d * (2.0 * (IN_BF16 ? 2 : 4) + (OUT_BF16 ? 2 : 4)) + 12.0);
        if (bytes > 512.0 * 1024 * 1024) return launch_rows<IN_BF16, OUT_BF16, 2, true>(a, lpr_log2, s);
        return launch_rows<IN_BF16, OUT_BF16, 1, false>(a, lpr_log2, s);
    }
    const bool vec4 = (a.d % 4) == 0 && aligned;
    const int vpr = vec4 ? a.d / 4 : a.d;
    const int rows_per_iter = vpr >= M_THREADS ? 1 : M_THREADS / vpr;
    long long blocks = (a.rows + rows_per_iter - 1) / rows_per_iter;
    if (blocks > 256 * 64) blocks = 256 * 64;   // grid-stride beyond 64 workgroups per CU
    if (blocks < 1) blocks = 1;
    if (vec4)
        hipLaunchKernelGGL((merge_kernel<IN_BF16, OUT_BF16, 4>), dim3((unsigned)blocks), dim3(M_THREADS), 0, s, a,
                           vpr, rows_per_iter);
    else
        hipLaunchKernelGGL((merge_kernel<IN_BF16, OUT_BF16, 1>), dim3((unsigned)blocks), dim3(M_THREADS), 0, s, a,
                           vpr, rows_per_iter);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
    if (a.in_bf16) return a.out_bf16 ? launch_t<true, true>(a, s) : launch_t<true, false>(a, s);
    return a.out_bf16 ? launch_t<false, true>(a, s) : launch_t<false, false>(a, s);
}

}  // namespace attn
