// Exact attention forward for fp32 Q/K/V (any head dimension 1..256), fp32 throughout.
//
// Same algorithm as the bf16 kernel ("FlashAttention by hand": key/value tiles streamed through on-chip
// memory, running max, running denominator, rescale on a new max, one final division), written for
// exactness rather than speed: no fp32 matrix cores (gfx950 has no xf32 MFMA and the fp32 path only serves
// small problems) and accurate expf/logf.  Dot products, scaled logits and the running max are kept in
// fp64, so that the rounding of an fp32 dot product (which grows with the logit magnitude) does not reach
// the softmax weights; weights, the denominator and the output accumulate in fp32.  A workgroup owns 64
// query rows; four lanes share a row, each holding a quarter of the head dimension in float4 chunks, and
// K/V tiles of 32 keys are staged in LDS with zero padding.
#include <hip/hip_runtime.h>
#include <math.h>

#include "attn_internal.h"

namespace attn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int F_THREADS = 256;
constexpr int F_ROWS = F_THREADS / 4;   // query rows per workgroup
constexpr int F_TKV = 32;               // keys per tile

template <int DMAX>
__global__ __launch_bounds__(F_THREADS) void fwd_f32_kernel(FwdArgs a, int num_qt) {
    constexpr int NCH = DMAX / 16;      // float4 chunks per lane
    __shared__ f32x4 ks[F_TKV][DMAX / 4];
    __shared__ f32x4 vs[F_TKV][DMAX / 4];

    const int bh = blockIdx.x / num_qt;
    const int qt = blockIdx.x % num_qt;
    const int tid = threadIdx.x;
    const int r = tid & 3;                       // quarter of the head dimension
    const int qi = qt * F_ROWS + (tid >> 2);     // this lane group's query
    const bool q_ok = qi < a.n_q;
    const int d = a.d;

    const float* qh = static_cast<const float*>(a.q) + (size_t)bh * a.q_head_stride;
    const float* kh = static_cast<const float*>(a.k) + (size_t)bh * a.kv_head_stride;
    const float* vh = static_cast<const float*>(a.v) + (size_t)bh * a.kv_head_stride;

    // chunk i of this lane covers head-dim elements 16*i + 4*r + (0..3)
    f32x4 q[NCH], acc[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int cc = 16 * i + 4 * r + e;
            q[i][e] = (q_ok && cc < d) ? qh[(size_t)qi * d + cc] : 0.f;
        }
    }

    const int q_last = min(qt * F_ROWS + F_ROWS, a.n_q) - 1;
    const int kv_end = a.causal ? max(0, min(a.n_kv, q_last + a.offset + 1)) : a.n_kv;
    const int lim = a.causal ? min(a.n_kv - 1, qi + a.offset) : a.n_kv - 1;   // last key visible to qi

    double m = -INFINITY;
    float l = 0.f;
    for (int kt = 0; kt < kv_end; kt += F_TKV) {
        __syncthreads();
        for (int idx = tid; idx < F_TKV * DMAX; idx += F_THREADS) {
            const int row = idx / DMAX, cc = idx % DMAX, key = kt + row;
            const bool ok = key < a.n_kv && cc < d;
            ks[row][cc / 4][cc % 4] = ok ? kh[(size_t)key * d + cc] : 0.f;
            vs[row][cc / 4][cc % 4] = ok ? vh[(size_t)key * d + cc] : 0.f;
        }
        __syncthreads();

        double s[F_TKV];
        double mt = -INFINITY;
#pragma unroll
        for (int j = 0; j < F_TKV; ++j) {
            double part = 0.0;
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const f32x4 k4 = ks[j][4 * i + r];
                part = fma((double)q[i][0], (double)k4[0], part);
                part = fma((double)q[i][1], (double)k4[1], part);
                part = fma((double)q[i][2], (double)k4[2], part);
                part = fma((double)q[i][3], (double)k4[3], part);
            }
            part += __shfl_xor(part, 1, 64);
            part += __shfl_xor(part, 2, 64);
            s[j] = (kt + j <= lim) ? part * (double)a.scale : -INFINITY;
            mt = fmax(mt, s[j]);
        }
        const double m_new = fmax(m, mt);
        if (m_new == -INFINITY) continue;        // nothing visible yet for this row
        const float alpha = m == -INFINITY ? 0.f : expf((float)(m - m_new));
        l *= alpha;
#pragma unroll
        for (int i = 0; i < NCH; ++i) acc[i] *= alpha;
#pragma unroll
        for (int j = 0; j < F_TKV; ++j) {
            const float p = expf((float)(s[j] - m_new));   // exp(-inf) = 0 for masked keys
            l += p;
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const f32x4 v4 = vs[j][4 * i + r];
                acc[i][0] = fmaf(p, v4[0], acc[i][0]);
                acc[i][1] = fmaf(p, v4[1], acc[i][1]);
                acc[i][2] = fmaf(p, v4[2], acc[i][2]);
                acc[i][3] = fmaf(p, v4[3], acc[i][3]);
            }
        }
        m = m_new;
    }

    if (!q_ok) return;
    // O = acc / l and lse = m + ln(l) (or (0, -inf)); when the launch accumulates, folded into the running
    // partial with the two-term merge of the (O, lse) merge kernel
    const float lb = l > 0.f ? (float)(m + (double)logf(l)) : -INFINITY;
    float cb = l > 0.f ? 1.f / l : 0.f, ca = 0.f, lse = lb;
    const float* op = nullptr;
    if (a.o_prev) {
        const float la = a.lse_prev[(size_t)bh * a.n_q + qi];
        const float big = fmaxf(la, lb);
        if (big != -INFINITY) {
            const float wa = expf(la - big), wb = expf(lb - big);
            const float inv = 1.f / (wa + wb);
            ca = wa * inv;
            cb *= wb * inv;
            lse = big + logf(wa + wb);
        } else {
            cb = 0.f;
            lse = -INFINITY;
        }
        op = a.o_prev + (size_t)bh * a.q_head_stride + (size_t)qi * d;
    }
    float* oh = static_cast<float*>(a.o) + (size_t)bh * a.q_head_stride + (size_t)qi * d;
#pragma unroll
    for (int i = 0; i < NCH; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int cc = 16 * i + 4 * r + e;
            if (cc < d) oh[cc] = acc[i][e] * cb + (op ? ca * op[cc] : 0.f);
        }
    if (r == 0) a.lse[(size_t)bh * a.n_q + qi] = lse;
}

template <int DMAX>
hipError_t launch_t(const FwdArgs& a, hipStream_t s) {
    const int num_qt = (a.n_q + F_ROWS - 1) / F_ROWS;
    const long long grid = (long long)num_qt * a.bh;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fwd_f32_kernel<DMAX>, dim3((unsigned)grid), dim3(F_THREADS), 0, s, a, num_qt);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s) {
    if (a.d <= 32) return launch_t<32>(a, s);
    if (a.d <= 64) return launch_t<64>(a, s);
    if (a.d <= 128) return launch_t<128>(a, s);
    if (a.d <= 256) return launch_t<256>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace attn
