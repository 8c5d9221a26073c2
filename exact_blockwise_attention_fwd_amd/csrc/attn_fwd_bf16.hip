// Exact attention forward for bf16 Q/K/V on gfx950: bf16 MFMA for Q.K^T and P.V, fp32 online softmax.
//
// The method is the fused, tiled exact attention of "FlashAttention by hand" (paragraphs on fused tiled
// attention, online softmax, the per-tile flow, rescaling and the single final division): key/value tiles
// are staged in on-chip memory (LDS here), every query row keeps a running max m, a running denominator l
// and an unnormalised output, and the score tile never leaves registers.  Causal masking ("HOF SWIFT
// Attention", section 3, Transform stage) is bottom-right aligned; tiles wholly in the future are skipped.
//
// Mapping to CDNA4 (gfx950), designed for this chip rather than taken from the pages' GPU:
//  * Every wave owns 32 query rows of one (b, h), and every SIMD runs two waves.  Key tiles are 64 keys
//    for d = 128 and 128 keys for d = 64 (16 KiB of K and of V per tile either way).  Two kernels share
//    the machinery below and differ in their software pipeline: fwd_bf16_kernel (used for d = 64) and
//    fwd_p3_kernel (d = 128), described where each is defined.
//  * Everything is computed transposed.  S^T = K Q^T uses v_mfma_f32_32x32x16_bf16 with A = K rows from
//    LDS and B = Q^T held in registers for the whole key loop.  In the 32x32 accumulator layout a lane then
//    holds 16 keys of ONE query (lane l and l^32 share query l%32), so the row max and row sum are in-lane
//    reductions plus one exchange between the two half-waves, and the per-query rescale factor is a
//    per-lane scalar.
//  * The A rows of S^T are read from K with bits 2 and 3 of the row index swapped.  That puts keys
//    16*(j/8) + 8*(l/32) + (j%8) into accumulator element j of lane l, so the fp32 scores of one 16-key
//    k-step are 8 consecutive keys per lane: exactly the B operand (P^T) that the P.V MFMA needs, with no
//    cross-lane shuffle.
//  * O^T = V^T P^T accumulates in 32x32 blocks over d.  Its A operand (V^T: one head-dim row, 8 keys per
//    lane) comes straight from the row-major V tile through ds_read_b64_tr_b16, the LDS transpose read:
//    within each 16-lane block, lane 4e+s points at 4 head-dim values of key e and lane i receives head-dim
//    value i of keys 0..3, so two such reads give a lane its 8 keys.
//  * K and V tiles move from HBM to LDS with buffer_load_dwordx4 ... lds: no staging registers, no LDS
//    store instructions, and loads past the last key return zeros (the buffer resource's bound).  Each
//    wave instruction fills one contiguous 1 KiB LDS segment in lane order, so the XOR swizzle of the LDS
//    layout is applied by choosing which 16-byte global chunk each lane fetches.
//  * LDS rows are XOR-swizzled in 16-byte units so that the operand reads of each 16-lane block (K rows for
//    S^T, four V rows for the transpose read) hit distinct banks.
//  * exp is v_exp_f32 (base 2) with scale*log2(e) folded into one FMA per score.  The exponent reference
//    need not be the running max: weights are taken against the current reference, and only when a row
//    has no reference yet or some row's weight sum for the tile exceeds 2^64 is the tile redone against
//    its true max (which then becomes the reference, and the output is rescaled once).  Every weight is
//    then at most 2^64, the fp32 sums stay far from overflow, and the single final division by the
//    denominator accumulated against the same reference gives the running-max result up to rounding.
//    The common path therefore has no row max, no rescale factor and no rescale of the accumulators.
//  * Workgroup ids are remapped so that consecutive logical tiles (same head, neighbouring query rows,
//    hence the same K/V stream) land on the same XCD and share its L2; causal launches start with the
//    longest query tiles.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <atomic>
#include <type_traits>

#include "attn_internal.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

constexpr float LOG2E = 1.4426950408889634f;
constexpr float REF_BOUND = 18446744073709551616.0f;   // 2^64: largest weight sum taken against a stale reference
constexpr int NXCD = 8;
constexpr unsigned BUF_RSRC_WORD3 = 0x00020000u;   // raw buffer, 32-bit data format, bounds-checked

template <int D>
struct Tile {
    static constexpr int QB = 1;      // 32-row query blocks per wave
    static constexpr int NW = 4;                     // waves per workgroup
    static constexpr int THREADS = 64 * NW;
    static constexpr int WAVES_PER_SIMD = 2;
    static constexpr int BR = 32 * QB * NW;          // query rows per workgroup
    static constexpr int BC = D == 128 ? 64 : 128;   // keys per tile
    static constexpr int NKB = BC / 32;              // 32-key blocks of S^T per tile
    static constexpr int NDB = D / 32;               // 32-row blocks of O^T
    static constexpr int NKS = D / 16;               // k-steps of S^T (over d)
    static constexpr int ROW = 2 * D;                // bytes per K or V row in LDS
    static constexpr int TILE = BC * ROW;            // bytes of one K (or V) tile
    static constexpr int SEGS = TILE / 1024;         // 1 KiB load segments per tile
    static constexpr int SEGS_PER_WAVE = SEGS / NW;
    static constexpr int RPS = 1024 / ROW;           // rows per segment
    static constexpr int LPR = ROW / 16;             // lanes (16-byte chunks) per row
    static constexpr int L = 2;                      // tiles of lookahead: tile t+L is loaded when iteration t ends
    static constexpr int NK = L, NV = L + 1;         // K and V buffers (V_{t-1} is still read in iteration t)
    static constexpr int LPT = 2 * SEGS_PER_WAVE;
    static constexpr int LDS = (NK + NV) * TILE;
    static_assert(SEGS % NW == 0, "segments split evenly over the waves");
    static_assert(NW * RPS * ROW == 4096, "a wave's load segments are 4 KiB apart");
};

// bits 2 and 3 of a row index swapped (an involution)
__device__ __forceinline__ int swap23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

// XOR applied to the 16-byte chunk index of K row r.  Read side: lane slot rho = swap23(r & 15) reads it.
template <int D>
__device__ __forceinline__ int k_swz(int r) {
    const int rho = swap23(r & 15);
    if constexpr (D == 128) return rho & 15;
    else return (rho & 7) ^ ((rho >> 3) & 1);
}

// XOR applied to the 16-byte chunk index of V row (key) r, chosen for the transpose reads
template <int D>
__device__ __forceinline__ int v_swz(int r) {
    if constexpr (D == 128) return 4 * (r & 3);
    else return 4 * ((r >> 1) & 1);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
    bf16x2 p = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(unsigned, p);
}

__device__ __forceinline__ float wave_xor32(float x) { return __shfl_xor(x, 32, 64); }

// Workgroup barrier ordering LDS accesses only: this wave's LDS reads have returned (lgkmcnt(0)) before it
// arrives.  Tile loads into LDS that are still in flight are not waited for here (a release fence would
// wait for all of them); callers wait with an explicit vmcnt for exactly the loads that must have landed.
// The empty asm statements keep the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// One query row's result from a bf16 kernel: O = acc / l and lse = m*|scale| + ln(l), or (0, -inf) when the
// row saw no key; when the launch accumulates, folded into the running partial with the two-term merge
// (M = max of the two lse, weights exp(lse - M) normalised to sum 1, lse = M + ln of their sum).  Lane h
// of the row's half-wave pair holds head-dim elements 32*db + 8*g + 4*h + (0..3) of acc[db].
template <int NDB, bool OUT_F32>
__device__ __forceinline__ void store_row(const FwdArgs& a, int bh, int qi, int h, const f32x16 (&acc)[NDB],
                                          float l_tot, float m, float scale_abs) {
    constexpr int D = 32 * NDB;
    const float lb = l_tot > 0.f ? m * scale_abs + logf(l_tot) : -INFINITY;
    float cb = l_tot > 0.f ? 1.f / l_tot : 0.f;   // factor on this launch's accumulator
    float ca = 0.f;                               // factor on the previous partial
    float lse = lb;
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
        op = a.o_prev + (size_t)bh * a.q_head_stride + (size_t)qi * D;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int c0 = 32 * db + 8 * g + 4 * h;
            f32x4 o4 = {acc[db][4 * g] * cb, acc[db][4 * g + 1] * cb, acc[db][4 * g + 2] * cb, acc[db][4 * g + 3] * cb};
            if (op) {
                o4 += ca * *reinterpret_cast<const f32x4*>(op + c0);
            }
            if (OUT_F32) {
                float* oh = static_cast<float*>(a.o) + (size_t)bh * a.q_head_stride + (size_t)qi * D;
                *reinterpret_cast<f32x4*>(oh + c0) = o4;
            } else {
                uint16_t* oh = static_cast<uint16_t*>(a.o) + (size_t)bh * a.q_head_stride + (size_t)qi * D;
                const u32x2 o2 = {pack_bf16(o4[0], o4[1]), pack_bf16(o4[2], o4[3])};
                *reinterpret_cast<u32x2*>(oh + c0) = o2;
            }
        }
    if (h == 0) a.lse[(size_t)bh * a.n_q + qi] = lse;
}

// ---- Two-stage pipeline (used for d = 64): workgroups of four waves (128 query rows), two per CU.  K is
// double-buffered and V triple-buffered.  Iteration t computes S(t) and the weights of tile t, and the P.V
// product of tile t-1: the softmax of one tile shares a basic block with the P.V MFMAs of the previous one,
// so the VALU and the matrix cores overlap inside one wave.  After the barrier that ends iteration t, tile
// t+2 is loaded into the buffers of K_t and V_{t-1}; it has a whole iteration to land.
template <int D, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(Tile<D>::THREADS, Tile<D>::WAVES_PER_SIMD) void fwd_bf16_kernel(FwdArgs a, int num_qt,
                                                                                            int total, int per_xcd) {
    using T = Tile<D>;
    constexpr int QB = T::QB;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    lds_char* const lds = (lds_char*)smem;   // all LDS addressing stays in the LDS address space

    // XCD-aware remap: hardware workgroup w runs on XCD w % 8; give each XCD a contiguous logical range
    const int w_hw = blockIdx.x;
    const int logical = (w_hw % NXCD) * per_xcd + w_hw / NXCD;
    if (logical >= total) return;
    const int bh = logical / num_qt;
    int qt = logical % num_qt;
    if (CAUSAL) qt = num_qt - 1 - qt;                // longest query tiles first

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5;                         // half-wave
    const int col = lane & 31;                       // query slot within a 32-row block

    const int q0 = qt * T::BR;
    const int qw0 = q0 + 32 * QB * wave;             // first query of this wave; block qb starts at qw0+32qb

    const uint16_t* qh = static_cast<const uint16_t*>(a.q) + (size_t)bh * a.q_head_stride;
    const uint16_t* kh = static_cast<const uint16_t*>(a.k) + (size_t)bh * a.kv_head_stride;
    const uint16_t* vh = static_cast<const uint16_t*>(a.v) + (size_t)bh * a.kv_head_stride;

    // keys this workgroup needs: [0, kv_end)
    const int q_last = min(q0 + T::BR, a.n_q) - 1;
    int kv_end = a.n_kv;
    if (CAUSAL) kv_end = max(0, min(a.n_kv, q_last + a.offset + 1));
    const int ntiles = (kv_end + T::BC - 1) / T::BC;

    // per-wave visibility bounds (wave-uniform)
    const int qw_last = min(qw0 + 32 * QB - 1, a.n_q - 1);
    const int wave_key_end = qw0 >= a.n_q ? 0 : CAUSAL ? min(kv_end, qw_last + a.offset + 1) : kv_end;
    const int wave_full_end = CAUSAL ? min(a.n_kv, qw0 + a.offset + 1) : a.n_kv;   // keys < this: all visible

    // ---- global -> LDS loads.  Each tile gets buffer resources whose base is the tile's first key and whose
    // bound is the rest of this head's key range, so loads past the last key return zeros; the whole
    // offset is in the per-lane VGPR offset (the scalar offset stays 0).
    const long long kv_bytes = (long long)a.n_kv * T::ROW;
    // this wave fills segments wave, wave+NW, ...; lane L writes row RPS*seg + L/LPR, physical chunk L%LPR.
    // Rows of segment wave+NW*k are those of segment `wave` plus NW*RPS*k (= 4096*k bytes), and the
    // swizzles only look at row bits that this shift leaves alone.
    int k_voff, v_voff;
    {
        const int r0 = T::RPS * wave + lane / T::LPR;
        const int p = lane % T::LPR;
        k_voff = r0 * T::ROW + 16 * (p ^ k_swz<D>(r0));
        v_voff = r0 * T::ROW + 16 * (p ^ v_swz<D>(r0));
    }
    auto issue_tile = [&](int t) {
        lds_char* kbuf = lds + (t % T::NK) * T::TILE;
        lds_char* vbuf = lds + (T::NK + t % T::NV) * T::TILE;
        const long long base = (long long)t * T::TILE;
        const int left = (int)(kv_bytes - base);
        const __amdgpu_buffer_rsrc_t krs =
            __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)kh + base), (short)0, left, BUF_RSRC_WORD3);
        const __amdgpu_buffer_rsrc_t vrs =
            __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)vh + base), (short)0, left, BUF_RSRC_WORD3);
#pragma unroll
        for (int k = 0; k < T::SEGS_PER_WAVE; ++k) {
            const int seg = wave + T::NW * k;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(kbuf + seg * 1024), 16, k_voff, 4096 * k, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(vbuf + seg * 1024), 16, v_voff, 4096 * k, 0, 0);
        }
    };

    // ---- Q^T fragments (B operand): query qw0+32qb+col, head-dim elements 16*ks + 8*h .. +7.
    // A negative scale negates Q (exact in bf16) so that every exponent is taken against a running max;
    // a zero scale zeroes Q, which gives the same all-zero logits without multiplying -inf by zero.
    const float scale_abs = fabsf(a.scale);
    const unsigned neg = a.scale < 0.f ? 0x80008000u : 0u;
    const unsigned keep = a.scale == 0.f ? 0u : 0xffffffffu;
    bf16x8 qf[QB][T::NKS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int qi = qw0 + 32 * qb + col;
#pragma unroll
        for (int ks = 0; ks < T::NKS; ++ks) {
            u32x4 x = qi < a.n_q ? *reinterpret_cast<const u32x4*>(qh + (size_t)qi * D + 16 * ks + 8 * h)
                                 : u32x4{0, 0, 0, 0};
            x = (x ^ neg) & keep;
            qf[qb][ks] = as_bf16x8(x);
        }
    }
    const float c = a.scale == 0.f ? LOG2E : scale_abs * LOG2E;   // scale * log2(e), always > 0

    // ---- per-lane LDS read offsets (the tile buffer and (kb, ks) parts are added as immediates)
    const int kslot = swap23(col);                   // K row (within a 32-key block) feeding A-row `col`
    int k_roff[T::NKS];
#pragma unroll
    for (int ks = 0; ks < T::NKS; ++ks) k_roff[ks] = kslot * T::ROW + 16 * ((2 * ks + h) ^ k_swz<D>(kslot));
    // transpose reads: block b = lane/16 -> half-wave h and head-dim half dp; e = key within a group of
    // four, s4 = which 4 head-dim values of the 16
    int v_roff[T::NDB];
    {
        const int b = lane >> 4, j = lane & 15, e = j >> 2, s4 = j & 3, dp = b & 1;
#pragma unroll
        for (int db = 0; db < T::NDB; ++db) {
            const int chunk = 4 * db + 2 * dp + (s4 >> 1);
            v_roff[db] = (8 * h + e) * T::ROW + 16 * (chunk ^ v_swz<D>(e)) + 8 * (s4 & 1);
        }
    }

    f32x16 acc[QB][T::NDB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int db = 0; db < T::NDB; ++db) acc[qb][db] = f32x16{};
    float m[QB], l[QB];   // exponent reference (running max of raw dot products, may lag) and denominator
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m[qb] = -INFINITY;
        l[qb] = 0.f;      // this half-wave's keys only; the halves are added at the end
    }
    u32x4 p_cur[QB][T::NKB][2];   // bf16 weights of the previous tile, consumed by its P.V one step later

    // Tiles this wave computes: a prefix [0, wave_tiles) of the workgroup's ntiles (causal waves stop early).
    const int wave_tiles = min(ntiles, (wave_key_end + T::BC - 1) / T::BC);

    // One pipelined step at tile t: S(t) = K_t Q^T, the P.V product of tile t-1 (weights from the previous
    // step), then the weights of tile t.  In program order the MFMAs of both products come first and the
    // softmax last, all in one straight-line block: the softmax waits only for S(t) and then issues while
    // the P.V MFMAs run.  An output rescale caused by tile t is applied at the start of the next step, i.e.
    // after P.V(t-1) (old reference) and before P.V(t) (new reference).
    //
    // The exponent reference m is not recomputed from every tile: the weights exp2(s*c - m*c) are taken
    // against the current reference, and only if no reference exists yet or some weight sum exceeds 2^64
    // (a score more than 64 exp2-units above the reference) is the tile redone against its true max.  Every
    // weight is then below 2^64 and the accumulated sums stay far inside fp32 range, so the result equals
    // the running-max formulation up to rounding; the row max drops out of the common path.
    float alpha_prev[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) alpha_prev[qb] = 1.f;
    bool moved_prev = false;
    auto step = [&](auto do_s, auto do_pv, auto masked_c, int t, const lds_char* __restrict__ kbuf,
                    const lds_char* __restrict__ vbuf) {
        constexpr bool DO_S = decltype(do_s)::value, DO_PV = decltype(do_pv)::value;
        constexpr bool MASKED = decltype(masked_c)::value;
        // Per-lane LDS offsets pass through an empty statement here, so that the compiler forms
        // "buffer + offset" once per step and folds the (kb, ks) constants into the instructions' offset
        // fields, instead of hoisting every offset+constant combination out of the loop.
#pragma unroll
        for (int ks = 0; ks < T::NKS; ++ks) __asm__ volatile("" : "+v"(k_roff[ks]));
#pragma unroll
        for (int db = 0; db < T::NDB; ++db) __asm__ volatile("" : "+v"(v_roff[db]));
        const int (&kro)[T::NKS] = k_roff;
        const int (&vro)[T::NDB] = v_roff;
        if (moved_prev) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int db = 0; db < T::NDB; ++db) acc[qb][db] *= alpha_prev[qb];
            moved_prev = false;
        }
        f32x16 s[QB][T::NKB];
        if constexpr (DO_S) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int kb = 0; kb < T::NKB; ++kb) s[qb][kb] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < T::NKS; ++ks) {
#pragma unroll
                for (int kb = 0; kb < T::NKB; ++kb) {
                    const u32x4 kv = *(const lds_u32x4*)(kbuf + kro[ks] + 32 * kb * T::ROW);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
                        s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kv), qf[qb][ks], s[qb][kb], 0, 0, 0);
                }
            }
        }
        if constexpr (DO_PV) {   // O^T += V^T P^T for tile t-1; V^T operand by two transpose reads
#pragma unroll
            for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int db = 0; db < T::NDB; ++db) {
                        const lds_char* p = vbuf + vro[db] + (32 * kb + 16 * ks) * T::ROW;
                        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
                        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * T::ROW));
                        const u32x4 vv = {__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                                          __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]};
#pragma unroll
                        for (int qb = 0; qb < QB; ++qb)
                            acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vv), as_bf16x8(p_cur[qb][kb][ks]),
                                                                              acc[qb][db], 0, 0, 0);
                    }
        }
        if constexpr (DO_S) {
            if constexpr (MASKED) {   // keys past the end or in the causal future
                const int kt = t * T::BC;
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    const int qi = qw0 + 32 * qb + col;
                    const int lim = CAUSAL ? min(a.n_kv - 1, qi + a.offset) : a.n_kv - 1;   // last visible key
#pragma unroll
                    for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
                        for (int j = 0; j < 16; ++j) {
                            const int key = kt + 32 * kb + 16 * (j >> 3) + 8 * h + (j & 7);
                            if (key > lim) s[qb][kb][j] = -INFINITY;
                        }
                }
            }
            u32x4 p_next[QB][T::NKB][2];
            float rs[QB];
            // weights of tile t against reference m (m*c == mc; 0 stands in while no reference exists)
            auto weights = [&](const float (&mc)[QB]) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    rs[qb] = 0.f;
#pragma unroll
                    for (int kb = 0; kb < T::NKB; ++kb) {
                        float e[16];
#pragma unroll
                        for (int j = 0; j < 16; ++j) e[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][kb][j], c, -mc[qb]));
                        float r8[8];   // pairwise row sum (short dependency chains)
#pragma unroll
                        for (int j = 0; j < 8; ++j) r8[j] = e[2 * j] + e[2 * j + 1];
#pragma unroll
                        for (int j = 0; j < 4; ++j) r8[j] = r8[2 * j] + r8[2 * j + 1];
                        rs[qb] += (r8[0] + r8[1]) + (r8[2] + r8[3]);
#pragma unroll
                        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                            for (int w = 0; w < 4; ++w)
                                p_next[qb][kb][ks][w] = pack_bf16(e[8 * ks + 2 * w], e[8 * ks + 2 * w + 1]);
                    }
                }
            };
            float mc[QB];
            bool redo = false;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                mc[qb] = m[qb] == -INFINITY ? 0.f : m[qb] * c;
                redo = redo || m[qb] == -INFINITY;
            }
            weights(mc);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) redo = redo || !(rs[qb] <= REF_BOUND);
            float alpha[QB];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) alpha[qb] = 1.f;
            if (__any(redo)) {
                // rare: the first visible keys, or a score far above the reference.  Move the reference to
                // the running max (for every row of the wave) and recompute the weights.
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    float mt = -INFINITY;
#pragma unroll
                    for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
                        for (int j = 0; j < 16; ++j) mt = fmaxf(mt, s[qb][kb][j]);
                    mt = fmaxf(mt, wave_xor32(mt));
                    const float m_new = fmaxf(m[qb], mt);
                    alpha[qb] = m[qb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m[qb] - m_new) * c);
                    m[qb] = m_new;
                    mc[qb] = m_new == -INFINITY ? 0.f : m_new * c;
                    alpha_prev[qb] = alpha[qb];
                }
                moved_prev = true;
                weights(mc);
            }
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) l[qb] = __builtin_fmaf(l[qb], alpha[qb], rs[qb]);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) p_cur[qb][kb][ks] = p_next[qb][kb][ks];
        }
    };
    using yes = std::integral_constant<bool, true>;
    using no = std::integral_constant<bool, false>;

    // prologue: tiles 0 .. L-1 in flight, tile 0 must have landed (in every wave) before the first step
    for (int t0 = 0; t0 < T::L && t0 < ntiles; ++t0) issue_tile(t0);
    if (ntiles >= T::L) __builtin_amdgcn_s_waitcnt(0x0F70 | ((T::L - 1) * T::LPT));
    else __builtin_amdgcn_s_waitcnt(0x0F70);
    lds_barrier();

    // End of iteration t: this wave's loads of tile t+1 have landed (tiles t+2 .. t+L-1 may still fly) and,
    // after the barrier, every wave's have, and every wave is done with K_t and V_{t-1}; tile t+L is then
    // loaded into their buffers.  All waves run exactly ntiles such barriers, whether or not they still have
    // tiles to compute.
    auto retire = [&](int t) {
        if (t + T::L - 1 < ntiles) __builtin_amdgcn_s_waitcnt(0x0F70 | ((T::L - 2) * T::LPT));
        else __builtin_amdgcn_s_waitcnt(0x0F70);
        lds_barrier();
        if (t + T::L < ntiles) issue_tile(t + T::L);
    };
    auto kbuf_of = [&](int t) { return (const lds_char*)(lds + (t % T::NK) * T::TILE); };
    auto vbuf_of = [&](int t) { return (const lds_char*)(lds + (T::NK + t % T::NV) * T::TILE); };
    // The steady-state iteration gets its buffers as restrict-qualified pointers, distinct from those the
    // loads issued by retire() write (tile t+L), so the compiler does not wait for those loads before
    // reading tile t and t-1 (the explicit vmcnt wait before every barrier is what makes that true).
    auto iterate = [&](int t, const lds_char* __restrict__ kb, const lds_char* __restrict__ vb) {
        step(yes{}, yes{}, no{}, t, kb, vb);
        retire(t);
    };
    // Tiles [0, full_tiles) of this wave need no mask; [full_tiles, wave_tiles) are the diagonal or ragged ones.
    const int full_tiles = min(wave_tiles, wave_full_end / T::BC);
    auto iterate_masked = [&](int t, const lds_char* __restrict__ kb, const lds_char* __restrict__ vb) {
        step(yes{}, yes{}, yes{}, t, kb, vb);
        retire(t);
    };
    int t = 0;
    if (ntiles > 0) {
        if (wave_tiles > 0) {
            if (full_tiles > 0) step(yes{}, no{}, no{}, 0, kbuf_of(0), vbuf_of(T::NV - 1));
            else step(yes{}, no{}, yes{}, 0, kbuf_of(0), vbuf_of(T::NV - 1));
        }
        retire(0);
        for (t = 1; t < full_tiles; ++t) iterate(t, kbuf_of(t), vbuf_of(t - 1));
        for (t = max(t, 1); t < wave_tiles; ++t) iterate_masked(t, kbuf_of(t), vbuf_of(t - 1));
        if (wave_tiles > 0) step(no{}, yes{}, no{}, t, kbuf_of(t), vbuf_of(t - 1));   // P.V of the last tile
        for (t = max(t, 1); t < ntiles; ++t) retire(t);
    }

    // ---- epilogue: one division by the final denominator; lse = scaled reference + ln(l)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int qi = qw0 + 32 * qb + col;
        const float l_tot = l[qb] + wave_xor32(l[qb]);
        if (qi < a.n_q) store_row<T::NDB, OUT_F32>(a, bh, qi, h, acc[qb], l_tot, m[qb], scale_abs);
    }
}

// LDS above the default limit needs an explicit opt-in, once per kernel and device.  Threads that race on
// the first launch may both set the attribute, which is harmless; the flags themselves are atomic.
template <auto KERN>
hipError_t allow_lds(int bytes) {
    static std::atomic<bool> done[64] = {};
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    if (!done[dev].load(std::memory_order_acquire)) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(KERN), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
        if (e != hipSuccess) return e;
        done[dev].store(true, std::memory_order_release);
    }
    return hipSuccess;
}

template <int D, bool CAUSAL, bool OUT_F32>
hipError_t launch_t(const FwdArgs& a, hipStream_t s) {
    using T = Tile<D>;
    const int num_qt = (a.n_q + T::BR - 1) / T::BR;
    const long long total_ll = (long long)num_qt * a.bh;
    if (total_ll > 0x7fffffffLL - NXCD) return hipErrorInvalidValue;
    if ((long long)a.n_kv * T::ROW > 0x7fffffffLL) return hipErrorInvalidValue;   // buffer bound is 31-bit
    const int total = (int)total_ll;
    const int per_xcd = (total + NXCD - 1) / NXCD;
    const int grid = per_xcd * NXCD;
    auto kern = fwd_bf16_kernel<D, CAUSAL, OUT_F32>;
    if (hipError_t e = allow_lds<fwd_bf16_kernel<D, CAUSAL, OUT_F32>>(T::LDS); e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(T::THREADS), T::LDS, s, a, num_qt, total, per_xcd);
    return hipGetLastError();
}

// ---- d = 128: three-stage software pipeline with a fixed interleave.
//
// Step t of a wave computes the softmax of tile t, whose scores S(t) were produced by the previous step,
// next to two batches of MFMAs that do not depend on it:
//   part 1:  P.V of tile t-1 (16 MFMAs, V^T by transpose reads)      with the scaling and exp of tile t's scores
//   part 2:  S(t+1) = K_{t+1} Q^T (16 MFMAs)                          with the row sums and bf16 packs of tile t
// so every VALU instruction of a step has an MFMA of the same step to hide under, and the order (two MFMAs,
// a share of the VALU work, the LDS reads for two MFMAs ahead) is pinned with scheduling fences.  Scores
// and weights need no double buffers: part 1 reads the scores before part 2 overwrites them, and part 2
// writes the new weights after part 1's MFMAs have read the old ones.  The rare redo of a tile (see the
// exponent reference rule in the file header) recomputes its scores from K_t, which stays in LDS until
// the step ends.  Two waves share every SIMD.  A workgroup is either four waves (128 query rows) or eight
// (256 rows: both waves of each SIMD then belong to it and share its K/V tiles, and with one workgroup per
// CU the LDS holds three steps of lead for every load).  K_{t+NK} and V_{t+NV-1} are loaded when step t ends.
template <int NW_>
struct P3 {
    static constexpr int D = 128, NW = NW_, THREADS = 64 * NW, BR = 32 * NW, BC = 64;
    static constexpr int NKB = BC / 32, NDB = D / 32, NKS = D / 16, ROW = 2 * D, TILE = BC * ROW;
    static constexpr int SEGS = TILE / 1024, SEGS_PER_WAVE = SEGS / NW;
    static constexpr int RPS = 1024 / ROW, LPR = ROW / 16;
    static constexpr int L = NW == 8 ? 3 : 1;        // steps of lead for every tile load
    static constexpr int NK = L + 2, NV = L + 1;     // K and V buffers
    static constexpr int LDS = (NK + NV) * TILE;
    static constexpr int WSTRIDE = NW * RPS * ROW;   // bytes between the load segments of one wave
    static_assert(NW == 4 || NW == 8, "four or eight waves per workgroup");
    static_assert(NK + NV >= NW + 1, "the epilogue stages every wave's rows in its own free K/V buffer");
};

template <int NW, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(P3<NW>::THREADS, 2) void fwd_p3_kernel(FwdArgs a, int num_qt, int total, int per_xcd) {
    using T = P3<NW>;
    constexpr int D = T::D;
    constexpr int WS = T::WSTRIDE;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    lds_char* const lds = (lds_char*)smem;

    const int w_hw = blockIdx.x;
    const int logical = (w_hw % NXCD) * per_xcd + w_hw / NXCD;
    if (logical >= total) return;
    const int bh = logical / num_qt;
    int qt = logical % num_qt;
    if (CAUSAL) qt = num_qt - 1 - qt;                // longest query tiles first

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5;
    const int col = lane & 31;
    const int q0 = qt * T::BR;
    const int qw0 = q0 + 32 * wave;

    const uint16_t* qh = static_cast<const uint16_t*>(a.q) + (size_t)bh * a.q_head_stride;
    const uint16_t* kh = static_cast<const uint16_t*>(a.k) + (size_t)bh * a.kv_head_stride;
    const uint16_t* vh = static_cast<const uint16_t*>(a.v) + (size_t)bh * a.kv_head_stride;

    const int q_last = min(q0 + T::BR, a.n_q) - 1;
    int kv_end = a.n_kv;
    if (CAUSAL) kv_end = max(0, min(a.n_kv, q_last + a.offset + 1));
    const int ntiles = (kv_end + T::BC - 1) / T::BC;
    const int qw_last = min(qw0 + 31, a.n_q - 1);
    const int wave_key_end = qw0 >= a.n_q ? 0 : CAUSAL ? min(kv_end, qw_last + a.offset + 1) : kv_end;
    const int wave_full_end = CAUSAL ? min(a.n_kv, qw0 + a.offset + 1) : a.n_kv;
    const int wave_tiles = min(ntiles, (wave_key_end + T::BC - 1) / T::BC);
    const int full_tiles = min(wave_tiles, wave_full_end / T::BC);

    // ---- global -> LDS loads (buffer loads straight into LDS; past the last key they return zeros)
    const long long kv_bytes = (long long)a.n_kv * T::ROW;
    int k_voff, v_voff;
    {
        const int r0 = T::RPS * wave + lane / T::LPR;
        const int p = lane % T::LPR;
        k_voff = r0 * T::ROW + 16 * (p ^ k_swz<D>(r0));
        v_voff = r0 * T::ROW + 16 * (p ^ v_swz<D>(r0));
    }
    auto load_k = [&](int j) __attribute__((always_inline)) {   // K_j into K buffer j % NK
        if (j >= ntiles) return;
        lds_char* buf = lds + (j % T::NK) * T::TILE;
        const long long base = (long long)j * T::TILE;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)kh + base), (short)0, (int)(kv_bytes - base), BUF_RSRC_WORD3);
#pragma unroll
        for (int k = 0; k < T::SEGS_PER_WAVE; ++k)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(buf + (wave + T::NW * k) * 1024), 16, k_voff, WS * k, 0, 0);
    };
    auto load_v = [&](int j) __attribute__((always_inline)) {   // V_j into V buffer j % NV
        if (j >= ntiles) return;
        lds_char* buf = lds + (T::NK + (j % T::NV)) * T::TILE;
        const long long base = (long long)j * T::TILE;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)vh + base), (short)0, (int)(kv_bytes - base), BUF_RSRC_WORD3);
#pragma unroll
        for (int k = 0; k < T::SEGS_PER_WAVE; ++k)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(buf + (wave + T::NW * k) * 1024), 16, v_voff, WS * k, 0, 0);
    };
    // Buffer bases pass through an empty statement as scalars, so that the compiler cannot split a constant
    // out of them into every read's address (it would be negative, which the offset field cannot hold).
    auto kbuf_of = [&](int j) __attribute__((always_inline)) {
        int o = (j % T::NK) * T::TILE;
        __asm__ volatile("" : "+s"(o));
        return (const lds_char*)(lds + o);
    };
    auto vbuf_of = [&](int j) __attribute__((always_inline)) {
        int o = (T::NK + (j % T::NV)) * T::TILE;
        __asm__ volatile("" : "+s"(o));
        return (const lds_char*)(lds + o);
    };

    // ---- Q^T fragments (B operand), held for the whole key loop
    const float scale_abs = fabsf(a.scale);
    const unsigned neg = a.scale < 0.f ? 0x80008000u : 0u;
    const unsigned keep = a.scale == 0.f ? 0u : 0xffffffffu;
    bf16x8 qf[T::NKS];
    {
        const int qi = qw0 + col;
#pragma unroll
        for (int ks = 0; ks < T::NKS; ++ks) {
            u32x4 x = qi < a.n_q ? *reinterpret_cast<const u32x4*>(qh + (size_t)qi * D + 16 * ks + 8 * h)
                                 : u32x4{0, 0, 0, 0};
            x = (x ^ neg) & keep;
            qf[ks] = as_bf16x8(x);
        }
    }
    const float c = a.scale == 0.f ? LOG2E : scale_abs * LOG2E;

    const int kslot = swap23(col);
    int k_roff[T::NKS];
#pragma unroll
    for (int ks = 0; ks < T::NKS; ++ks) k_roff[ks] = kslot * T::ROW + 16 * ((2 * ks + h) ^ k_swz<D>(kslot));
    int v_roff[T::NDB];
    {
        const int b = lane >> 4, j = lane & 15, e = j >> 2, s4 = j & 3, dp = b & 1;
#pragma unroll
        for (int db = 0; db < T::NDB; ++db) {
            const int chunk = 4 * db + 2 * dp + (s4 >> 1);
            v_roff[db] = (8 * h + e) * T::ROW + 16 * (chunk ^ v_swz<D>(e)) + 8 * (s4 & 1);
        }
    }

    f32x16 acc[T::NDB];
#pragma unroll
    for (int db = 0; db < T::NDB; ++db) acc[db] = f32x16{};
    float m = -INFINITY, l = 0.f, alpha_prev = 1.f;
    bool moved = false;
    f32x16 s[T::NKB];           // scores of the tile whose softmax is next
    u32x4 p[T::NKB][2];         // bf16 weights of the tile whose P.V is next
    float mcr = 0.f;            // m*c, or 0 while the row has no reference
    float bnd = -1.f;           // bound on a tile's weight sum: 2^64, or -1 (forcing the redo) while there is no reference

    auto s_all = [&](f32x16 (&sc)[T::NKB], const lds_char* kbuf) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < T::NKB; ++kb) sc[kb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < T::NKS; ++ks)
#pragma unroll
            for (int kb = 0; kb < T::NKB; ++kb) {
                const u32x4 kv = *(const lds_u32x4*)(kbuf + k_roff[ks] + 32 * kb * T::ROW);
                sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kv), qf[ks], sc[kb], 0, 0, 0);
            }
    };
    auto mask_tile = [&](int t, f32x16 (&sc)[T::NKB]) __attribute__((always_inline)) {
        const int kt = t * T::BC;
        const int qi = qw0 + col;
        const int lim = CAUSAL ? min(a.n_kv - 1, qi + a.offset) : a.n_kv - 1;
#pragma unroll
        for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int key = kt + 32 * kb + 16 * (j >> 3) + 8 * h + (j & 7);
                if (key > lim) sc[kb][j] = -INFINITY;
            }
    };
    // weights and their row sum against reference mc (the plain form, used by the rare redo)
    auto weights = [&](const f32x16 (&sc)[T::NKB], float mc) __attribute__((always_inline)) {
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < T::NKB; ++kb) {
            float e[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) e[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][j], c, -mc));
            float r8[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) r8[j] = e[2 * j] + e[2 * j + 1];
#pragma unroll
            for (int j = 0; j < 4; ++j) r8[j] = r8[2 * j] + r8[2 * j + 1];
            rs += (r8[0] + r8[1]) + (r8[2] + r8[3]);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int w = 0; w < 4; ++w) p[kb][ks][w] = pack_bf16(e[8 * ks + 2 * w], e[8 * ks + 2 * w + 1]);
        }
        return rs;
    };

    // One step t (see the header of this kernel).  kn = K_{t+1}, kc = K_t, vp = V_{t-1}, as restrict-qualified
    // pointers distinct from the buffers the loads issued at the step's end write (K_{t+NK}, V_{t+NV-1}), so
    // the compiler does not wait for those loads before reading; the explicit vmcnt wait before every
    // barrier is what makes that true.
    auto step = [&](auto do_soft, auto do_pv, auto do_s, int t, const lds_char* __restrict__ kn,
                    const lds_char* __restrict__ kc, const lds_char* __restrict__ vp) __attribute__((always_inline)) {
        constexpr bool SOFT = decltype(do_soft)::value, PV = decltype(do_pv)::value, S = decltype(do_s)::value;
        // The per-lane LDS offsets pass through an empty statement, so that "buffer + offset" is formed once
        // per offset and step and the (kb, ks) constants land in the reads' offset fields.
#pragma unroll
        for (int ks = 0; ks < T::NKS; ++ks) __asm__ volatile("" : "+v"(k_roff[ks]));
#pragma unroll
        for (int db = 0; db < T::NDB; ++db) __asm__ volatile("" : "+v"(v_roff[db]));
        // a reference moved by the previous softmax: rescale the output before P.V(t-1) adds to it
        if (moved) {
#pragma unroll
            for (int db = 0; db < T::NDB; ++db) acc[db] *= alpha_prev;
            moved = false;
        }
        if constexpr (SOFT) {
            if (t >= full_tiles) mask_tile(t, s);   // diagonal and ragged tiles
        }
        const float mc = mcr;
        float e[2 * 16];
        u32x4 kv[16];
        auto kread = [&](int i) __attribute__((always_inline)) {
            kv[i] = *(const lds_u32x4*)(kn + k_roff[i >> 1] + 32 * (i & 1) * T::ROW);
        };
        // ---- part 1: P.V(t-1) (two transpose reads per MFMA, two MFMAs ahead) with the exps of tile t
        {
            i16x4 vl[16], vhh[16];
            auto vread = [&](int i) __attribute__((always_inline)) {
                const int kb = i >> 3, ks = (i >> 2) & 1, db = i & 3;
                const lds_char* q = vp + v_roff[db] + (32 * kb + 16 * ks) * T::ROW;
                vl[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)q);
                vhh[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(q + 4 * T::ROW));
            };
            if constexpr (PV) {
                vread(0);
                vread(1);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if constexpr (PV) {
                    if (i + 2 < 16) vread(i + 2);
                    const int kb = i >> 3, ks = (i >> 2) & 1, db = i & 3;
                    const u32x4 vv = {__builtin_bit_cast(u32x2, vl[i])[0], __builtin_bit_cast(u32x2, vl[i])[1],
                                      __builtin_bit_cast(u32x2, vhh[i])[0], __builtin_bit_cast(u32x2, vhh[i])[1]};
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vv), as_bf16x8(p[kb][ks]), acc[db], 0, 0, 0);
                }
                if constexpr (SOFT) {
                    e[2 * i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i >> 3][(2 * i) & 15], c, -mc));
                    e[2 * i + 1] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i >> 3][(2 * i + 1) & 15], c, -mc));
                }
                if constexpr (S && PV) {
                    if (i >= 14) kread(i - 14);   // the first K operands of part 2, under the last P.V MFMAs
                }
                if constexpr (PV) __builtin_amdgcn_sched_barrier(0);
            }
        }
        // ---- part 2: S(t+1) (one K read per MFMA, two MFMAs ahead) with the sums and packs of tile t
        float rs = 0.f;   // the tile's weight sum, accumulated pair by pair under the S MFMAs
        {
            if constexpr (S && !PV) {
                kread(0);
                kread(1);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if constexpr (S) {
                    if (i + 2 < 16) kread(i + 2);
                    const int ks = i >> 1, kb = i & 1;
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kv[i]), qf[ks], ks == 0 ? f32x16{} : s[kb], 0, 0, 0);
                }
                if constexpr (SOFT) {
                    const float pair = e[2 * i] + e[2 * i + 1];
                    rs = i == 0 ? pair : rs + pair;
                    p[i >> 3][(i >> 2) & 1][i & 3] = pack_bf16(e[2 * i], e[2 * i + 1]);
                    __asm__ volatile("" ::"v"(p[i >> 3][(i >> 2) & 1][i & 3]));   // keep the pack in this slot
                }
                if constexpr (S) __builtin_amdgcn_sched_barrier(0);
            }
        }
        if constexpr (SOFT) {
            float alpha = 1.f;
            if (__any(!(rs <= bnd))) {
                // rare: no reference yet, or a weight sum above 2^64.  Tile t's scores were replaced by
                // S(t+1) (when there was one): recompute them from K_t, mask, and redo the tile against its max.
                f32x16 sc[T::NKB];
                if constexpr (S) {
                    s_all(sc, kc);
                    if (t >= full_tiles) mask_tile(t, sc);
                } else {
#pragma unroll
                    for (int kb = 0; kb < T::NKB; ++kb) sc[kb] = s[kb];
                }
                float mt = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
                    for (int j = 0; j < 16; ++j) mt = fmaxf(mt, sc[kb][j]);
                mt = fmaxf(mt, wave_xor32(mt));
                const float m_new = fmaxf(m, mt);
                alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m - m_new) * c);
                if (__any(m != -INFINITY && m_new != m)) {
                    alpha_prev = alpha;
                    moved = true;
                }
                m = m_new;
                mcr = m_new == -INFINITY ? 0.f : m_new * c;
                bnd = m_new == -INFINITY ? -1.f : REF_BOUND;
                rs = weights(sc, mcr);
            }
            l = __builtin_fmaf(l, alpha, rs);
        }
    };
    // End of step t: every wave's loads of K_{t+2} and V_t have landed and every wave is done with K_t and
    // V_{t-1}; K_{t+NK} and V_{t+NV-1} then go into their buffers.  All waves run exactly ntiles such barriers.
    auto retire = [&](int t) __attribute__((always_inline)) {
        // K_{t+2} and V_t were issued L steps ago; the loads of the L-1 later retires may still fly (when
        // all of them exist; near the end, wait for everything)
        if (t + T::L + 1 < ntiles) __builtin_amdgcn_s_waitcnt(0x0F70 | ((T::L - 1) * 2 * T::SEGS_PER_WAVE));
        else __builtin_amdgcn_s_waitcnt(0x0F70);
        lds_barrier();
        load_k(t + T::NK);
        load_v(t + T::NV - 1);
    };
    using yes = std::integral_constant<bool, true>;
    using no = std::integral_constant<bool, false>;

    // ---- prologue: K_0, K_1, K_2 and V_0 in flight; all must land (in every wave) before S(0)
    for (int j = 0; j < T::NK; ++j) load_k(j);
    for (int j = 0; j < T::NV - 1; ++j) load_v(j);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    lds_barrier();

    // Steps 0 .. nt-1 (step t: softmax of tile t, P.V of t-1, S of t+1), then the P.V of the last tile.
    const int nt = wave_tiles;
    int t = 0;
    // The wave's 32 rows of the running partial (when there is one) and of the output are addressed through
    // buffer resources bounded at the last query row: loads past it return zeros and stores are dropped.
    const int rows_left = __builtin_amdgcn_readfirstlane(max(0, min(32, a.n_q - qw0)));   // uniform, kept scalar
    // The running partial, in the order the epilogue writes: with fp32 output lane l holds floats
    // 4*(l%32)..+3 of row 2k + l/32 in prev[k]; with bf16 output floats 8*(l%16) + 4*(k%2)..+3 of row
    // 4*(k/2) + l/16.
    f32x4 prev[16];
    float lse_pv = -INFINITY;   // lse of the partial for row qw0 + col
    auto fetch_prev = [&]() __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(a.o_prev + (size_t)bh * a.q_head_stride + (size_t)qw0 * D), (short)0, rows_left * D * 4, BUF_RSRC_WORD3);
        const int voff = OUT_F32 ? (lane >> 5) * D * 4 + 16 * (lane & 31) : (lane >> 4) * D * 4 + 32 * (lane & 15);
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int koff = OUT_F32 ? 2 * k * D * 4 : 4 * (k >> 1) * D * 4 + 16 * (k & 1);
            prev[k] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, koff, 0));
        }
        if (col < rows_left) lse_pv = a.lse_prev[(size_t)bh * a.n_q + qw0 + col];
    };
    if (nt > 0) {
        s_all(s, kbuf_of(0));
        if (nt > 1) {
            step(yes{}, no{}, yes{}, 0, kbuf_of(1), kbuf_of(0), vbuf_of(0));
            retire(0);
            for (t = 1; t < nt - 1; ++t) {
                step(yes{}, yes{}, yes{}, t, kbuf_of(t + 1), kbuf_of(t), vbuf_of(t - 1));
                retire(t);
            }
            step(yes{}, yes{}, no{}, t, kbuf_of(t), kbuf_of(t), vbuf_of(t - 1));   // no next S
        } else {
            step(yes{}, no{}, no{}, 0, kbuf_of(0), kbuf_of(0), vbuf_of(0));
        }
        // P.V of the last tile, after the barrier that ends its step: that barrier is what makes the last V
        // tile visible (every wave waited for its loads of it), and it does not reload that V buffer
        retire(t);
        ++t;
        // the running partial is loaded now, to arrive during the last P.V
        if (a.o_prev) fetch_prev();
        step(no{}, yes{}, no{}, t, kbuf_of(t), kbuf_of(t), vbuf_of(nt - 1));
    } else if (a.o_prev) {
        fetch_prev();
    }
    for (; t < ntiles; ++t) retire(t);   // the rest of the workgroup's barriers and loads

    // ---- epilogue: one division by the final denominator, lse = scaled reference + ln(l), and the fold
    // into the running partial (two-term merge: M = max of the two lse, weights exp(lse - M) normalised to
    // sum 1, lse = M + ln of their sum).  Lane (col, h) holds head-dim elements 32*db + 8*g + 4*h + (0..3)
    // of its row; the scaled rows go through LDS so that loads and stores cover whole rows.
    {
        const int qi = qw0 + col;
        const float l_tot = l + wave_xor32(l);
        const float lb = l_tot > 0.f ? m * scale_abs + logf(l_tot) : -INFINITY;
        float cb = l_tot > 0.f ? 1.f / l_tot : 0.f;   // factor on this launch's accumulator
        float ca = 0.f;                               // factor on the running partial
        float lse = lb;
        if (a.o_prev) {
            const float big = fmaxf(lse_pv, lb);
            if (big != -INFINITY) {
                const float wa = expf(lse_pv - big), wb = expf(lb - big);
                const float inv = 1.f / (wa + wb);
                ca = wa * inv;
                cb *= wb * inv;
                lse = big + logf(wa + wb);
            } else {
                cb = 0.f;
                lse = -INFINITY;
            }
        }
        if (h == 0 && col < rows_left) a.lse[(size_t)bh * a.n_q + qi] = lse;
        // A free 16 KiB LDS buffer per wave: after the last barrier only the V buffer of the last tile may
        // still be read (by waves finishing their last P.V); nothing else is read or loaded any more.
        const int busy = ntiles > 0 ? T::NK + (ntiles - 1) % T::NV : T::NK + T::NV;
        const int slot = wave < busy ? wave : wave + 1;
        lds_char* const st = lds + slot * T::TILE;
        // row r, 16-byte piece q at piece q ^ r of the row (conflict-free writes and reads)
#pragma unroll
        for (int db = 0; db < T::NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int q = 8 * db + 2 * g + h;
                const f32x4 o4 = {acc[db][4 * g] * cb, acc[db][4 * g + 1] * cb, acc[db][4 * g + 2] * cb,
                                  acc[db][4 * g + 3] * cb};
                *(lds_f32x4*)(st + col * 512 + 16 * (q ^ col)) = o4;
            }
        __asm__ volatile("" ::: "memory");   // the reads below see this wave's writes (LDS keeps a wave's order)
        const int ca_bits = __builtin_bit_cast(int, ca);
        const size_t obase = (size_t)bh * a.q_head_stride + (size_t)qw0 * D;
        if constexpr (OUT_F32) {
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(static_cast<float*>(a.o) + obase), (short)0, rows_left * D * 4, BUF_RSRC_WORD3);
            const int q = lane & 31;
            f32x4 o4[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int r = 2 * k + (lane >> 5);
                o4[k] = *(const lds_f32x4*)(st + r * 512 + 16 * (q ^ r));
            }
            if (a.o_prev) {
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    const int r = 2 * k + (lane >> 5);
                    o4[k] += __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * r, ca_bits)) * prev[k];
                }
            }
            const int voff = (lane >> 5) * D * 4 + 16 * q;
#pragma unroll
            for (int k = 0; k < 16; ++k)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o4[k]), rs, voff, 2 * k * D * 4, 0);
        } else {
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(static_cast<uint16_t*>(a.o) + obase), (short)0, rows_left * D * 2, BUF_RSRC_WORD3);
            const int q = lane & 15;
            f32x4 lo[8], hi[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int r = 4 * k + (lane >> 4);
                lo[k] = *(const lds_f32x4*)(st + r * 512 + 16 * ((2 * q) ^ r));
                hi[k] = *(const lds_f32x4*)(st + r * 512 + 16 * ((2 * q + 1) ^ r));
            }
            if (a.o_prev) {
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int r = 4 * k + (lane >> 4);
                    const float car = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * r, ca_bits));
                    lo[k] += car * prev[2 * k];
                    hi[k] += car * prev[2 * k + 1];
                }
            }
            const int voff = (lane >> 4) * D * 2 + 16 * q;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const u32x4 o4 = {pack_bf16(lo[k][0], lo[k][1]), pack_bf16(lo[k][2], lo[k][3]),
                                  pack_bf16(hi[k][0], hi[k][1]), pack_bf16(hi[k][2], hi[k][3])};
                __builtin_amdgcn_raw_buffer_store_b128(o4, rs, voff, 4 * k * D * 2, 0);
            }
        }
    }
}

template <int NW, bool CAUSAL, bool OUT_F32>
hipError_t launch_p3(const FwdArgs& a, hipStream_t st) {
    using T = P3<NW>;
    const int num_qt = (a.n_q + T::BR - 1) / T::BR;
    const long long total_ll = (long long)num_qt * a.bh;
    if (total_ll > 0x7fffffffLL - NXCD) return hipErrorInvalidValue;
    if ((long long)a.n_kv * T::ROW > 0x7fffffffLL) return hipErrorInvalidValue;   // buffer bound is 31-bit
    const int total = (int)total_ll;
    const int per_xcd = (total + NXCD - 1) / NXCD;
    const int grid = per_xcd * NXCD;
    auto kern = fwd_p3_kernel<NW, CAUSAL, OUT_F32>;
    if (hipError_t e = allow_lds<fwd_p3_kernel<NW, CAUSAL, OUT_F32>>(T::LDS); e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(T::THREADS), T::LDS, st, a, num_qt, total, per_xcd);
    return hipGetLastError();
}

}  // namespace

// Workgroup size of the d = 128 kernel: eight waves (256 query rows, one workgroup per CU) when the launch
// has at least eight such workgroups per CU, four waves (128 rows, two workgroups per CU) otherwise, where
// smaller workgroups balance better.  ATTN_BF16_D128_WAVES=4 or 8 forces one of them (used by the tests to
// run every shape through both).
static int d128_waves(const FwdArgs& a) {
    if (const char* e = getenv("ATTN_BF16_D128_WAVES")) {
        const int v = atoi(e);
        if (v == 4 || v == 8) return v;
    }
    const long long wide = (long long)((a.n_q + 255) / 256) * a.bh;
    return wide >= 8LL * device_cus() ? 8 : 4;
}

hipError_t launch_fwd_bf16(const FwdArgs& a, bool out_f32, hipStream_t s) {
    const bool c = a.causal != 0;
    if (a.d == 128) {
        if (d128_waves(a) == 8) {
            if (c) return out_f32 ? launch_p3<8, true, true>(a, s) : launch_p3<8, true, false>(a, s);
            return out_f32 ? launch_p3<8, false, true>(a, s) : launch_p3<8, false, false>(a, s);
        }
        if (c) return out_f32 ? launch_p3<4, true, true>(a, s) : launch_p3<4, true, false>(a, s);
        return out_f32 ? launch_p3<4, false, true>(a, s) : launch_p3<4, false, false>(a, s);
    }
    if (a.d == 64) {
        if (c) return out_f32 ? launch_t<64, true, true>(a, s) : launch_t<64, true, false>(a, s);
        return out_f32 ? launch_t<64, false, true>(a, s) : launch_t<64, false, false>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace attn
