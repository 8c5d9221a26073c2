// Exact attention forward for bf16 Q/K/V on gfx950: bf16 MFMA for Q.K^T and P.V, fp32 online softmax.
//
// The method is the fused, tiled exact attention of "FlashAttention by hand" (paragraphs on fused tiled
// attention, online softmax, the per-tile flow, rescaling and the single final division): key/value tiles
// are staged in on-chip memory (LDS here), every query row keeps a running max m, a running denominator l
// and an unnormalised output, and the score tile never leaves registers.  Causal masking ("HOF SWIFT
// Attention", section 3, Transform stage) is bottom-right aligned; tiles wholly in the future are skipped.
//
// Mapping to CDNA4 (gfx950), designed for this chip rather than taken from the pages' GPU:
//  * A workgroup is 4 wave64s and owns 128 query rows of one (b, h); each wave owns 32 rows.
//  * Everything is computed transposed.  S^T = K Q^T uses v_mfma_f32_32x32x16_bf16 with A = K rows from
//    LDS and B = Q^T held in registers for the whole key loop.  In the 32x32 accumulator layout a lane then
//    holds 16 keys of ONE query (lane l and l^32 share query l%32), so the row max and row sum are in-lane
//    reductions plus one exchange between the two half-waves, and the per-query rescale factor is a
//    per-lane scalar.
//  * The A rows of S^T are read from K with bits 2 and 3 of the row index swapped.  That puts keys
//    16*(j/8) + 8*(l/32) + (j%8) into accumulator element j of lane l, so the fp32 scores of one
//    16-key k-step are 8 consecutive keys per lane: exactly the B operand (P^T) that the P.V MFMA needs,
//    with no cross-lane shuffle, and the matching A operand (V^T) is one 16-byte LDS read.
//  * O^T = V^T P^T accumulates in 32x32 blocks over d; V is transposed while it is staged into LDS
//    (byte permutes in registers, 8-byte LDS writes).
//  * K/V tiles are double-buffered in LDS: the global loads of tile t+1 are in flight while tile t is
//    computed; one workgroup barrier per tile.
//  * LDS rows are XOR-swizzled in 16-byte units so that the MFMA operand reads of 16 consecutive lanes hit
//    distinct banks.
//  * exp is v_exp_f32 (base 2) with scale*log2(e) folded into one FMA per score; the rescale of the
//    output accumulator is skipped, exactly, when no row max of the wave moved.
//  * Workgroup ids are remapped so that consecutive logical tiles (same head, neighbouring query rows,
//    hence the same K/V stream) land on the same XCD and share its L2; causal launches start with the
//    longest query tiles.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "attn_internal.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float LOG2E = 1.4426950408889634f;
constexpr int NXCD = 8;

template <int D>
struct Tile {
    static constexpr int NW = 4;                 // waves per workgroup
    static constexpr int THREADS = 64 * NW;
    static constexpr int BR = 32 * NW;           // query rows per workgroup
    static constexpr int BC = D == 128 ? 64 : 128;  // keys per tile
    static constexpr int NKB = BC / 32;          // 32-key blocks of S^T per tile
    static constexpr int NDB = D / 32;           // 32-row blocks of O^T
    static constexpr int NKS = D / 16;           // k-steps of S^T (over d)
    static constexpr int KROW = 2 * D;           // bytes per K row in LDS
    static constexpr int VROW = 2 * BC;          // bytes per V^T row in LDS
    static constexpr int KBYTES = BC * KROW;
    static constexpr int VBYTES = D * VROW;
    static constexpr int BUF = KBYTES + VBYTES;
    static constexpr int LDS = 2 * BUF;
    static constexpr int KCH = D / 8;            // 16-byte chunks per K row
    static constexpr int VCH = BC / 8;           // 16-byte chunks per V^T row
    static constexpr int K_LOADS = BC * KCH / THREADS;   // 16-byte K loads per thread per tile
    static_assert(BC * KCH % THREADS == 0, "K tile split");
    static_assert((BC / 4) * (D / 8) == THREADS, "V tile split: one 4-key x 8-d block per thread");
};

// bits 2 and 3 of a key slot swapped (an involution)
__device__ __forceinline__ int swap23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

// byte offset of 16-byte chunk c of K row r inside a K tile
template <int D>
__device__ __forceinline__ int k_off(int r, int c) {
    const int rho = swap23(r & 15);
    int phys;
    if constexpr (D == 128) phys = c ^ (rho & 15);
    else phys = c ^ ((rho & 7) ^ ((rho >> 3) & 1));
    return r * Tile<D>::KROW + phys * 16;
}

// byte offset of 16-byte chunk c (8 keys) of V^T row dd (head-dim index) inside a V^T tile
template <int D>
__device__ __forceinline__ int v_off(int dd, int c) {
    int phys;
    if constexpr (Tile<D>::VCH == 8) phys = c ^ ((dd ^ (dd >> 3)) & 7);
    else phys = c ^ (dd & 15);
    return dd * Tile<D>::VROW + phys * 16;
}

__device__ __forceinline__ u32x4 lds_read16(const char* base, int off) {
    return *reinterpret_cast<const u32x4*>(base + off);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
    bf16x2 p = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(unsigned, p);
}

__device__ __forceinline__ float wave_xor32(float x) { return __shfl_xor(x, 32, 64); }

template <int D>
struct Staged {            // one tile's global loads held in registers until written to LDS
    u32x4 k[Tile<D>::K_LOADS];
    u32x4 v[4];
};

template <int D>
__device__ __forceinline__ void load_tile(Staged<D>& st, const uint16_t* kh, const uint16_t* vh, int kt,
                                          int n_kv, int tid) {
    using T = Tile<D>;
#pragma unroll
    for (int i = 0; i < T::K_LOADS; ++i) {
        const int q = tid + T::THREADS * i;
        const int r = q / T::KCH, c = q % T::KCH;
        const int key = kt + r;
        st.k[i] = key < n_kv ? *reinterpret_cast<const u32x4*>(kh + (size_t)key * D + c * 8) : u32x4{0, 0, 0, 0};
    }
    const int kg = tid / (D / 8), dc = tid % (D / 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int key = kt + 4 * kg + i;
        st.v[i] = key < n_kv ? *reinterpret_cast<const u32x4*>(vh + (size_t)key * D + dc * 8) : u32x4{0, 0, 0, 0};
    }
}

template <int D>
__device__ __forceinline__ void store_tile(const Staged<D>& st, char* buf, int tid) {
    using T = Tile<D>;
#pragma unroll
    for (int i = 0; i < T::K_LOADS; ++i) {
        const int q = tid + T::THREADS * i;
        const int r = q / T::KCH, c = q % T::KCH;
        *reinterpret_cast<u32x4*>(buf + k_off<D>(r, c)) = st.k[i];
    }
    // transpose a 4-key x 8-d block: for head-dim element e, the four keys' values become one 8-byte unit
    const int kg = tid / (D / 8), dc = tid % (D / 8);
    char* vt = buf + T::KBYTES;
#pragma unroll
    for (int w = 0; w < 4; ++w) {           // dword w holds head-dim elements 2w, 2w+1
        const unsigned lo_e = __builtin_amdgcn_perm(st.v[1][w], st.v[0][w], 0x05040100u);
        const unsigned hi_e = __builtin_amdgcn_perm(st.v[3][w], st.v[2][w], 0x05040100u);
        const unsigned lo_o = __builtin_amdgcn_perm(st.v[1][w], st.v[0][w], 0x07060302u);
        const unsigned hi_o = __builtin_amdgcn_perm(st.v[3][w], st.v[2][w], 0x07060302u);
        const int d0 = 8 * dc + 2 * w;
        *reinterpret_cast<u32x2*>(vt + v_off<D>(d0, kg >> 1) + 8 * (kg & 1)) = u32x2{lo_e, hi_e};
        *reinterpret_cast<u32x2*>(vt + v_off<D>(d0 + 1, kg >> 1) + 8 * (kg & 1)) = u32x2{lo_o, hi_o};
    }
}

template <int D, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(Tile<D>::THREADS, 2) void fwd_bf16_kernel(FwdArgs a, int num_qt, int total,
                                                                      int per_xcd) {
    using T = Tile<D>;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    // XCD-aware remap: hardware workgroup w runs on XCD w % 8; give each XCD a contiguous logical range
    const int w_hw = blockIdx.x;
    const int logical = (w_hw % NXCD) * per_xcd + w_hw / NXCD;
    if (logical >= total) return;
    const int bh = logical / num_qt;
    int qt = logical % num_qt;
    if (CAUSAL) qt = num_qt - 1 - qt;                // longest query tiles first

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = lane >> 5;                         // half-wave
    const int col = lane & 31;                       // query slot within the wave

    const int q0 = qt * T::BR;
    const int qw0 = q0 + 32 * wave;                  // first query of this wave
    const int qi = qw0 + col;                        // this lane's query
    const bool q_ok = qi < a.n_q;

    const uint16_t* qh = static_cast<const uint16_t*>(a.q) + (size_t)bh * a.q_head_stride;
    const uint16_t* kh = static_cast<const uint16_t*>(a.k) + (size_t)bh * a.kv_head_stride;
    const uint16_t* vh = static_cast<const uint16_t*>(a.v) + (size_t)bh * a.kv_head_stride;

    // keys this workgroup needs: [0, kv_end)
    const int q_last = min(q0 + T::BR, a.n_q) - 1;
    int kv_end = a.n_kv;
    if (CAUSAL) kv_end = max(0, min(a.n_kv, q_last + a.offset + 1));
    const int ntiles = (kv_end + T::BC - 1) / T::BC;

    // per-wave visibility bounds
    const int qw_last = min(qw0 + 31, a.n_q - 1);
    const int wave_key_end = CAUSAL ? min(kv_end, qw_last + a.offset + 1) : kv_end;   // exclusive
    const int wave_full_end = CAUSAL ? min(a.n_kv, qw0 + a.offset + 1) : a.n_kv;      // keys < this: all visible

    // Q^T fragments (B operand): query qi, head-dim elements 16*ks + 8*h .. +7
    // A negative scale negates Q (exact in bf16) so that every exponent is taken against a running max;
    // a zero scale zeroes Q, which gives the same all-zero logits without multiplying -inf by zero.
    const float scale_abs = fabsf(a.scale);
    const unsigned neg = a.scale < 0.f ? 0x80008000u : 0u;
    const unsigned keep = a.scale == 0.f ? 0u : 0xffffffffu;
    bf16x8 qf[T::NKS];
#pragma unroll
    for (int ks = 0; ks < T::NKS; ++ks) {
        u32x4 x = q_ok ? *reinterpret_cast<const u32x4*>(qh + (size_t)qi * D + 16 * ks + 8 * h) : u32x4{0, 0, 0, 0};
        x = (x ^ neg) & keep;
        qf[ks] = as_bf16x8(x);
    }
    const float c = a.scale == 0.f ? LOG2E : scale_abs * LOG2E;   // scale * log2(e), always > 0

    f32x16 acc[T::NDB];
#pragma unroll
    for (int db = 0; db < T::NDB; ++db) acc[db] = f32x16{};
    float m = -INFINITY;   // running max of the raw dot products of this lane's query
    float l = 0.f;         // running denominator, this half-wave's keys only

    Staged<D> st;
    if (ntiles > 0) {
        load_tile<D>(st, kh, vh, 0, a.n_kv, tid);
        store_tile<D>(st, smem, tid);
        if (ntiles > 1) load_tile<D>(st, kh, vh, T::BC, a.n_kv, tid);
    }
    __syncthreads();

    const int kslot = swap23(col);   // K row (within a 32-key block) that feeds A-row `col`

    for (int t = 0; t < ntiles; ++t) {
        const char* buf = smem + (t & 1) * T::BUF;
        const int kt = t * T::BC;
        if (kt < wave_key_end) {
            // ---- S^T = K Q^T for BC keys x 32 queries
            f32x16 s[T::NKB];
#pragma unroll
            for (int kb = 0; kb < T::NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < T::NKS; ++ks) {
#pragma unroll
                for (int kb = 0; kb < T::NKB; ++kb) {
                    const bf16x8 kf = as_bf16x8(lds_read16(buf, k_off<D>(32 * kb + kslot, 2 * ks + h)));
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[kb], 0, 0, 0);
                }
            }
            // ---- mask keys past the end or in the causal future (diagonal / ragged tiles only)
            const bool need_mask = (kt + T::BC > wave_full_end) || (kt + T::BC > a.n_kv);
            if (need_mask) {
                const int lim = CAUSAL ? min(a.n_kv - 1, qi + a.offset) : a.n_kv - 1;   // last visible key
#pragma unroll
                for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int key = kt + 32 * kb + 16 * (j >> 3) + 8 * h + (j & 7);
                        if (key > lim) s[kb][j] = -INFINITY;
                    }
            }
            // ---- running max
            float mt = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j) mt = fmaxf(mt, s[kb][j]);
            mt = fmaxf(mt, wave_xor32(mt));
            const float m_new = fmaxf(m, mt);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float mc = m_use * c;
            // ---- rescale what was accumulated under the old max (skipped when no max moved: alpha == 1)
            const float alpha = __builtin_amdgcn_exp2f(m * c - mc);
            if (__any(m_new > m)) {
#pragma unroll
                for (int db = 0; db < T::NDB; ++db) acc[db] *= alpha;
                l *= alpha;
            }
            m = m_new;
            // ---- probabilities (fp32 sum for l, bf16 for the P.V product)
            u32x4 pf[T::NKB][2];
            float rs = 0.f;
#pragma unroll
            for (int kb = 0; kb < T::NKB; ++kb) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    s[kb][j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][j], c, -mc));
                    rs += s[kb][j];
                }
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int w = 0; w < 4; ++w)
                        pf[kb][ks][w] = pack_bf16(s[kb][8 * ks + 2 * w], s[kb][8 * ks + 2 * w + 1]);
            }
            l += rs;
            // ---- O^T += V^T P^T
            const char* vt = buf + T::KBYTES;
#pragma unroll
            for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int db = 0; db < T::NDB; ++db) {
                        const bf16x8 vf = as_bf16x8(lds_read16(vt, v_off<D>(32 * db + col, 4 * kb + 2 * ks + h)));
                        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, as_bf16x8(pf[kb][ks]), acc[db], 0, 0, 0);
                    }
        }
        if (t + 1 < ntiles) {
            store_tile<D>(st, smem + ((t + 1) & 1) * T::BUF, tid);
            if (t + 2 < ntiles) load_tile<D>(st, kh, vh, (t + 2) * T::BC, a.n_kv, tid);
        }
        __syncthreads();
    }

    // ---- epilogue: one division by the final denominator; lse = scaled max + ln(l)
    const float l_tot = l + wave_xor32(l);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (q_ok) {
        if (OUT_F32) {
            float* oh = static_cast<float*>(a.o) + (size_t)bh * a.q_head_stride + (size_t)qi * D;
#pragma unroll
            for (int db = 0; db < T::NDB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    f32x4 o4 = {acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv, acc[db][4 * g + 2] * inv,
                                acc[db][4 * g + 3] * inv};
                    *reinterpret_cast<f32x4*>(oh + 32 * db + 8 * g + 4 * h) = o4;
                }
        } else {
            uint16_t* oh = static_cast<uint16_t*>(a.o) + (size_t)bh * a.q_head_stride + (size_t)qi * D;
#pragma unroll
            for (int db = 0; db < T::NDB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    u32x2 o2 = {pack_bf16(acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv),
                                pack_bf16(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv)};
                    *reinterpret_cast<u32x2*>(oh + 32 * db + 8 * g + 4 * h) = o2;
                }
        }
        if (h == 0) a.lse[(size_t)bh * a.n_q + qi] = l_tot > 0.f ? m * scale_abs + logf(l_tot) : -INFINITY;
    }
}

template <int D, bool CAUSAL, bool OUT_F32>
hipError_t launch_t(const FwdArgs& a, hipStream_t s) {
    using T = Tile<D>;
    const int num_qt = (a.n_q + T::BR - 1) / T::BR;
    const long long total_ll = (long long)num_qt * a.bh;
    if (total_ll > 0x7fffffffLL - NXCD) return hipErrorInvalidValue;
    const int total = (int)total_ll;
    const int per_xcd = (total + NXCD - 1) / NXCD;
    const int grid = per_xcd * NXCD;
    auto kern = fwd_bf16_kernel<D, CAUSAL, OUT_F32>;
    static bool attr_set = false;   // LDS above 64 KiB needs an explicit opt-in
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, T::LDS);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(T::THREADS), T::LDS, s, a, num_qt, total, per_xcd);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, bool out_f32, hipStream_t s) {
    const bool c = a.causal != 0;
    if (a.d == 128) {
        if (c) return out_f32 ? launch_t<128, true, true>(a, s) : launch_t<128, true, false>(a, s);
        return out_f32 ? launch_t<128, false, true>(a, s) : launch_t<128, false, false>(a, s);
    }
    if (a.d == 64) {
        if (c) return out_f32 ? launch_t<64, true, true>(a, s) : launch_t<64, true, false>(a, s);
        return out_f32 ? launch_t<64, false, true>(a, s) : launch_t<64, false, false>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace attn
