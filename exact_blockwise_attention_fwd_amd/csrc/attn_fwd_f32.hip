// Exact attention forward for fp32 Q/K/V (any head dimension 1..256), fp32 throughout.
//
// Same algorithm as the bf16 kernel ("FlashAttention by hand": key/value tiles streamed through on-chip
// memory, running max, running denominator, rescale on a new max, one final division), written for
// exactness: no fp32 matrix cores (gfx950 has no xf32 MFMA) and accurate expf/logf.  Dot products, scaled
// logits and the running max are kept in fp64, so that the rounding of an fp32 dot product (which grows
// with the logit magnitude) does not reach the softmax weights; weights, the denominator and the output
// accumulate in fp32, per key tile first and then across tiles.
//
// The problems this path serves are small, so the kernel is built for latency:
//  * LPR lanes share a query row (4, 8 or 16), each holding DMAX/LPR head-dim elements in float4 chunks;
//    a workgroup of 256 lanes owns 256/LPR rows.  The launch takes the fewest lanes per row (at least 8 from
//    d = 128 up) that still give two workgroups per CU, so small launches spread over the chip with short
//    per-lane dot products.
//  * K/V tiles of 32 keys (16 at d > 128, which keeps LDS at 64 KiB) are double-buffered in LDS, zero padded
//    past d and past the last key.  The global loads of tile t+1 are issued into registers before tile t is
//    computed and land in the other buffer after it, so load latency hides under the arithmetic; one
//    barrier per tile.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include "attn_internal.h"

namespace attn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int F_THREADS = 256;

template <int DMAX, int LPR>
__global__ __launch_bounds__(F_THREADS) void fwd_f32_kernel(FwdArgs a, int num_qt, int vec_loads) {
    constexpr int F_TKV = DMAX > 128 ? 16 : 32;    // keys per tile
    constexpr int ROWS = F_THREADS / LPR;          // query rows per workgroup
    constexpr int NCH = DMAX / (4 * LPR);          // float4 chunks per lane
    constexpr int C4 = DMAX / 4;                   // float4 chunks per K/V row in LDS
    constexpr int LOADS = F_TKV * C4 / F_THREADS;  // float4 chunks of one tile each thread loads, per tensor
    constexpr int SUB = F_TKV;                     // keys whose weights are summed apart before joining the row's sums
    static_assert(NCH >= 1 && LOADS >= 1 && F_TKV * C4 % F_THREADS == 0, "tile split");
    __shared__ f32x4 ks[2][F_TKV][C4];
    __shared__ f32x4 vs[2][F_TKV][C4];

    const int bh = blockIdx.x / num_qt;
    const int qt = blockIdx.x % num_qt;
    const int tid = threadIdx.x;
    const int r = tid % LPR;                     // which chunks of the head dimension
    const int qi = qt * ROWS + tid / LPR;        // this lane group's query
    const bool q_ok = qi < a.n_q;
    const int d = a.d;

    const float* qh = static_cast<const float*>(a.q) + (size_t)bh * a.q_head_stride;
    const float* kh = static_cast<const float*>(a.k) + (size_t)bh * a.kv_head_stride;
    const float* vh = static_cast<const float*>(a.v) + (size_t)bh * a.kv_head_stride;

    // chunk i of this lane covers head-dim elements 4*(LPR*i + r) + (0..3)
    f32x4 q[NCH], acc[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int cc = 4 * (LPR * i + r) + e;
            q[i][e] = (q_ok && cc < d) ? qh[(size_t)qi * d + cc] : 0.f;
        }
    }

    const int q_last = min(qt * ROWS + ROWS, a.n_q) - 1;
    const int kv_end = a.causal ? max(0, min(a.n_kv, q_last + a.offset + 1)) : a.n_kv;
    const int lim = a.causal ? min(a.n_kv - 1, qi + a.offset) : a.n_kv - 1;   // last key visible to qi
    const int ntiles = (kv_end + F_TKV - 1) / F_TKV;

    // tile loads: thread tid fetches float4 chunks tid + F_THREADS*u (u < LOADS) of the tile, i.e. key
    // row c / C4 and elements 4*(c % C4) .. +3, with zeros past d and past the last key
    f32x4 kr[LOADS], vr[LOADS];
    auto fetch = [&](int t) {
#pragma unroll
        for (int u = 0; u < LOADS; ++u) {
            const int c = tid + F_THREADS * u, row = c / C4, c0 = 4 * (c % C4), key = t * F_TKV + row;
            kr[u] = vr[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (key < a.n_kv && c0 < d) {
                const size_t off = (size_t)key * d + c0;
                if (vec_loads) {   // d % 4 == 0 and 16-byte aligned rows
                    kr[u] = *reinterpret_cast<const f32x4*>(kh + off);
                    vr[u] = *reinterpret_cast<const f32x4*>(vh + off);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (c0 + e < d) {
                            kr[u][e] = kh[off + e];
                            vr[u][e] = vh[off + e];
                        }
                }
            }
        }
    };
    auto stash = [&](int b) {
#pragma unroll
        for (int u = 0; u < LOADS; ++u) {
            const int c = tid + F_THREADS * u;
            ks[b][c / C4][c % C4] = kr[u];
            vs[b][c / C4][c % C4] = vr[u];
        }
    };

    if (ntiles > 0) {
        fetch(0);
        stash(0);
    }
    __syncthreads();

    double m = -INFINITY;
    float l = 0.f;
    for (int t = 0; t < ntiles; ++t) {
        const int b = t & 1;
        if (t + 1 < ntiles) fetch(t + 1);          // in flight while tile t is computed

#pragma unroll
        for (int h0 = 0; h0 < F_TKV; h0 += SUB) {   // keys h0 .. h0+SUB-1 of the tile
            double s[SUB];
            double mt = -INFINITY;
            const int kt = t * F_TKV + h0;
#pragma unroll
            for (int j = 0; j < SUB; ++j) {
                double part = 0.0;
#pragma unroll
                for (int i = 0; i < NCH; ++i) {
                    const f32x4 k4 = ks[b][h0 + j][LPR * i + r];
                    part = fma((double)q[i][0], (double)k4[0], part);
                    part = fma((double)q[i][1], (double)k4[1], part);
                    part = fma((double)q[i][2], (double)k4[2], part);
                    part = fma((double)q[i][3], (double)k4[3], part);
                }
#pragma unroll
                for (int w = 1; w < LPR; w *= 2) part += __shfl_xor(part, w, 64);
                s[j] = (kt + j <= lim) ? part * (double)a.scale : -INFINITY;
                mt = fmax(mt, s[j]);
            }
            const double m_new = fmax(m, mt);
            if (m_new != -INFINITY) {                  // else nothing visible yet for this row
                const float alpha = m == -INFINITY ? 0.f : expf((float)(m - m_new));
                // These keys' weights and weighted rows are summed apart (chains of SUB terms) and join the running
                // sums once, so a row's rounding grows with its count of tiles rather than of keys.
                float lt = 0.f;
                f32x4 at[NCH];
#pragma unroll
                for (int i = 0; i < NCH; ++i) at[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < SUB; ++j) {
                    const float p = expf((float)(s[j] - m_new));   // exp(-inf) = 0 for masked keys
                    lt += p;
#pragma unroll
                    for (int i = 0; i < NCH; ++i) {
                        const f32x4 v4 = vs[b][h0 + j][LPR * i + r];
                        at[i][0] = fmaf(p, v4[0], at[i][0]);
                        at[i][1] = fmaf(p, v4[1], at[i][1]);
                        at[i][2] = fmaf(p, v4[2], at[i][2]);
                        at[i][3] = fmaf(p, v4[3], at[i][3]);
                    }
                }
                l = fmaf(l, alpha, lt);
#pragma unroll
                for (int i = 0; i < NCH; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[i][e] = fmaf(acc[i][e], alpha, at[i][e]);
                m = m_new;
            }
        }
        // Buffer b^1 was last read in iteration t-1, which every wave finished before the barrier that
        // ended it; the barrier below keeps iteration t+1 from reading it before every wave stored it.
        if (t + 1 < ntiles) stash(b ^ 1);
        __syncthreads();
    }

    if (!q_ok) return;
    // O = acc / l and lse = m + ln(l) (or (0, -inf)); when the launch accumulates, folded into the running
    // partial with the two-term merge of the (O, lse) merge kernel.  Every element of the row is read and
    // written by the lane that owns it; the row's lse is read by its LPR lanes (one wave) in one load and
    // written by one of them with a value computed from that load.
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
            const int cc = 4 * (LPR * i + r) + e;
            if (cc < d) oh[cc] = acc[i][e] * cb + (op ? ca * op[cc] : 0.f);
        }
    if (r == 0) a.lse[(size_t)bh * a.n_q + qi] = lse;
}

template <int DMAX, int LPR>
hipError_t launch_t(const FwdArgs& a, int vec_loads, hipStream_t s) {
    constexpr int ROWS = F_THREADS / LPR;
    const int num_qt = (a.n_q + ROWS - 1) / ROWS;
    const long long grid = (long long)num_qt * a.bh;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((fwd_f32_kernel<DMAX, LPR>), dim3((unsigned)grid), dim3(F_THREADS), 0, s, a, num_qt, vec_loads);
    return hipGetLastError();
}

// The fewest lanes per row (4, 8, 16; at most DMAX/4) that still give two workgroups per CU, and at least 8
// from 128 elements up: four lanes per row there need more registers than two waves per SIMD hold (measured
// against four: +124 % at d = 256 on a 4096-row launch; -25 % at d = 128, where four lanes fitted two waves
// before each key tile got its own partial sums).
// ATTN_F32_LANES_PER_ROW=4, 8 or 16 forces one where the head dimension allows it (used by the tests to run
// every shape through each).
template <int DMAX>
hipError_t launch_d(const FwdArgs& a, int vec_loads, hipStream_t s) {
    int lpr = 0;
    if (const char* e = getenv("ATTN_F32_LANES_PER_ROW")) {
        const int v = atoi(e);
        if (v == 4 || v == 8 || (v == 16 && DMAX >= 64)) lpr = v;
    }
    if (lpr == 0) {
        const long long want = 2LL * device_cus();
        auto groups = [&](int l) { return (long long)((a.n_q + F_THREADS / l - 1) / (F_THREADS / l)) * a.bh; };
        lpr = (DMAX <= 64 && groups(4) >= want) ? 4 : (DMAX < 64 || groups(8) >= want) ? 8 : 16;
    }
    if constexpr (DMAX >= 64) {
        if (lpr == 16) return launch_t<DMAX, 16>(a, vec_loads, s);
    }
    if (lpr == 8) return launch_t<DMAX, 8>(a, vec_loads, s);
    return launch_t<DMAX, 4>(a, vec_loads, s);
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s) {
    // float4 loads of K and V rows need every row start 16-byte aligned
    const int vec_loads = (a.d % 4 == 0) && (a.kv_head_stride % 4 == 0) && ((uintptr_t)a.k % 16 == 0) &&
                          ((uintptr_t)a.v % 16 == 0);
    if (a.d <= 32) return launch_d<32>(a, vec_loads, s);
    if (a.d <= 64) return launch_d<64>(a, vec_loads, s);
    if (a.d <= 128) return launch_d<128>(a, vec_loads, s);
    if (a.d <= 256) return launch_d<256>(a, vec_loads, s);
    return hipErrorInvalidValue;
}

}  // namespace attn
