// Merge of two partial attention results over disjoint key sets:
//     M = max(lse_a, lse_b), w_x = exp(lse_x - M), O = (w_a O_a + w_b O_b) / (w_a + w_b),
//     lse = M + ln(w_a + w_b), and (0, -inf) when both parts are empty.
// This is the associative combination of per-fragment statistics in the "ATTENTION2D" explainer
// (sections 2 and 3), with the rescale rule of "FlashAttention by hand" (paragraph on rescaling).
//
// The kernel streams rows * d elements and is bound by HBM bandwidth: 16-byte loads and stores where
// the head dimension allows, a workgroup processes whole rows at a time, and the weights are computed per
// vector from the two lse values (cheap next to the memory traffic).  In-place use (O == O_a, lse ==
// lse_a) is safe: every output vector is written by the thread that read it, and a row's lse is written
// only after a workgroup barrier that follows every read of that row's lse.
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

template <bool IN_BF16, bool OUT_BF16>
hipError_t launch_t(const MergeArgs& a, hipStream_t s) {
    const bool vec4 = (a.d % 4) == 0;
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
