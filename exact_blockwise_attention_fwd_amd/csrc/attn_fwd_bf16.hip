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
//    (16 KiB of K and of V per tile at d = 128, 8 KiB at d = 64).  One kernel, fwd_p3_kernel, serves both
//    head dimensions with a three-stage software pipeline described where it is defined.
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
//  * The P.V products accumulate the weights rounded to bf16 (up to 2^-8 relative each).  At d = 64 the
//    kernel keeps two denominators per row: the fp32 sum of the weights, for the LSE, and the fp32 sum of
//    their bf16 roundings (one v_dot2c_f32_bf16 per pair), by which it divides O, so a row's output is a
//    convex combination of V rows with weights proportional to exactly the accumulated values and a
//    dominant weight's rounding cancels.  At d = 128 it divides O by the fp32 sum (no extra instruction per
//    pair): O then carries the dominant weights' rounding, at most 2^-8 of the largest |V| entry in a row
//    dominated by one key, and averaging out over rows spread across many keys.
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

// acc + a.lo + a.hi for two packed bf16 weights, summed in fp32 (one v_dot2c_f32_bf16 against (1, 1))
__device__ __forceinline__ float add_bf16_pair(unsigned a, float acc) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), ones, acc, false);
}

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

// As lds_barrier, but the wave's last four LDS reads may still be in flight (LDS reads return in order): the
// next step's first V^T operands, read from a buffer that no load issued after this barrier overwrites.  Every
// other read of the step has completed, since its value was consumed before the wave reached the barrier.
__device__ __forceinline__ void lds_barrier_keep4() {
    __builtin_amdgcn_s_waitcnt(0xC47F);   // lgkmcnt(4)
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
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

// ---- Three-stage software pipeline with a fixed interleave (d = 64 and d = 128).
//
// Step t of a wave computes the softmax of tile t, whose scores S(t) were produced by the previous step,
// next to two batches of MFMAs that do not depend on it:
//   part 1:  P.V of tile t-1 (d/8 MFMAs, V^T by transpose reads)     with the scaling and exp of tile t's scores
//   part 2:  S(t+1) = K_{t+1} Q^T (d/8 MFMAs)                        with the row sums and bf16 packs of tile t
// so every VALU instruction of a step has an MFMA of the same step to hide under, and the order (MFMAs,
// a share of the VALU work, the LDS reads for two MFMAs ahead) is pinned with scheduling fences.  Scores
// and weights need no double buffers: part 1 reads the scores before part 2 overwrites them, and part 2
// writes the new weights after part 1's MFMAs have read the old ones.  The rare redo of a tile (see the
// exponent reference rule in the file header) recomputes its scores from K_t, which stays in LDS until
// the step ends.  Two waves share every SIMD.  A workgroup is either four waves (128 query rows) or eight
// (256 rows: both waves of each SIMD then belong to it and share its K/V tiles, and with one workgroup per
// CU the LDS holds four K and four V buffers).  K_{t+NK} and V_{t+NV-1} are loaded when step t ends.  With
// eight waves V_{t+1} is waited for at the end of step t, one step before its P.V, so that each step can
// read the next step's first two V^T operands before its barrier and the next P.V starts without waiting
// for LDS.
template <int NW_, int D_>
struct P3 {
    static constexpr int D = D_, NW = NW_, THREADS = 64 * NW, BR = 32 * NW, BC = 64;
    static constexpr int NKB = BC / 32, NDB = D / 32, NKS = D / 16, ROW = 2 * D, TILE = BC * ROW;
    // MFMAs of a step's two parts: P.V(t-1) (NKB 32-key blocks x 2 k-steps x NDB head-dim blocks) and
    // S(t+1) (NKS k-steps x NKB key blocks); the tile's 32 scores per lane spread evenly over them
    static constexpr int NPV = NKB * 2 * NDB, NS = NKS * NKB;
    static constexpr int EXP_PER_PV = 16 * NKB / NPV, PAIRS_PER_S = 8 * NKB / NS;
    // d = 64 divides O by the fp32 sum of the weights' bf16 roundings (a second denominator, one dot2 per
    // weight pair); d = 128 by the fp32 sum of the weights
    static constexpr bool LT = D == 64;
    // Waves that load the tiles: in eight-wave workgroups only waves 0 .. 3 (one per SIMD), each issuing twice
    // the loads, so that the other wave of each SIMD goes from the barrier straight into its next step; the two
    // waves of a SIMD then start their steps a little apart (+0.8 % ring share, +1.8 % causal prefill 4k, +0.1 %
    // peaky 16k against all eight loading, same box).  The staggered alternative, the second wave of every
    // SIMD taking its barrier half a step later, measured -3 to -5 %.
    static constexpr int LOADERS = NW == 8 ? NW / 2 : NW;
    static constexpr int SEGS = TILE / 1024, SEGS_PER_WAVE = SEGS / LOADERS;   // load segments per loading wave
    static constexpr int RPS = 1024 / ROW, LPR = ROW / 16;
    // K and V buffers: K_j is loaded NK-2 steps and V_j NV-1 steps before its first use
    static constexpr int NK = NW == 8 ? 4 : 3, NV = NW == 8 ? 4 : 2;
    static constexpr int EXTRA = NK + NV >= NW + 1 ? 0 : NW + 1 - NK - NV;   // staging-only buffers
    static constexpr int LDS = (NK + NV + EXTRA) * TILE;
    static constexpr int WSTRIDE = LOADERS * RPS * ROW;   // bytes between the load segments of one wave
    // retire(t) needs K_{t+2} (issued by retire(t+2-NK)) and V_{t+VAHEAD} (by retire(t+VAHEAD+1-NV)) to have
    // landed; loads are issued K then V per retire, and AFTER load instructions issued after the later of the
    // two may still be in flight.  VAHEAD = 1: eight-wave steps read the first V operands of the next step
    // before the barrier that ends them, so V_{t+1} must have landed (every loading wave's share) by retire(t)
    static constexpr int VAHEAD = NW == 8 ? 1 : 0;
    static constexpr int DK = NK - 2, DV = NV - 1 - VAHEAD;
    static_assert(DV >= 1, "V is loaded at least one step before it is needed");
    // (AFTER goes into the low four vmcnt bits of the s_waitcnt immediate, so it must stay below 16)
    static constexpr int AFTER = (DK < DV ? 1 + 2 * (DK - 1) : 2 * (DV - 1)) * SEGS_PER_WAVE;
    static constexpr int LEAD = NK > NV - 1 ? NK : NV - 1;   // all loads up to retire(t-1) exist iff t-1+LEAD < ntiles
    static_assert(AFTER < 16, "loads allowed in flight fit the s_waitcnt vmcnt field");
    static_assert(NW == 4 || NW == 8, "four or eight waves per workgroup");
    static_assert(D == 64 || D == 128, "head dimension 64 or 128");
    static_assert(EXP_PER_PV * NPV == 16 * NKB && PAIRS_PER_S * NS == 8 * NKB, "scores spread evenly");
    static_assert(NK + NV + EXTRA >= NW + 1, "the epilogue stages every wave's rows in its own free buffer");
    static_assert((NK - 1) * TILE + 32 * ROW < 65536 && (NV - 1) * TILE + 52 * ROW < 65536,
                  "constant buffer bases fit the LDS reads' 16-bit offset field");
};

template <int NW, int D_, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__((P3<NW, D_>::THREADS), 2) void fwd_p3_kernel(FwdArgs a, int num_qt, int total,
                                                                        int per_xcd, int length_major) {
    using T = P3<NW, D_>;
    constexpr int D = T::D;
    constexpr int WS = T::WSTRIDE;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    lds_char* const lds = (lds_char*)smem;

    // Workgroup order.  Hardware workgroup w runs on XCD w mod 8.  Tiles of equal length: each XCD takes a
    // contiguous range of (head, query tile), so its heads' K/V streams share its L2.  Tiles of unequal length
    // (a causal diagonal inside the key range): length-major, w takes query tile rank w / BH (longest first) of
    // head w mod BH, so every XCD starts all of its longest tiles before any shorter one (a head-major order
    // left long tiles of later heads to start last and run into the launch's tail); XCD x then works on the
    // heads congruent to x mod 8.
    const int w_hw = blockIdx.x;
    int bh, qt;
    if (CAUSAL && length_major) {
        if (w_hw >= total) return;
        const int nbh = total / num_qt;
        bh = w_hw % nbh;
        qt = num_qt - 1 - w_hw / nbh;
    } else {
        const int logical = (w_hw % NXCD) * per_xcd + w_hw / NXCD;
        if (logical >= total) return;
        bh = logical / num_qt;
        qt = logical % num_qt;
    }

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
        if (j >= ntiles || wave >= T::LOADERS) return;
        lds_char* buf = lds + (j % T::NK) * T::TILE;
        const long long base = (long long)j * T::TILE;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)kh + base), (short)0, (int)(kv_bytes - base), BUF_RSRC_WORD3);
#pragma unroll
        for (int k = 0; k < T::SEGS_PER_WAVE; ++k)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(buf + (wave + T::LOADERS * k) * 1024), 16, k_voff, WS * k, 0, 0);
    };
    auto load_v = [&](int j) __attribute__((always_inline)) {   // V_j into V buffer j % NV
        if (j >= ntiles || wave >= T::LOADERS) return;
        lds_char* buf = lds + (T::NK + (j % T::NV)) * T::TILE;
        const long long base = (long long)j * T::TILE;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)vh + base), (short)0, (int)(kv_bytes - base), BUF_RSRC_WORD3);
#pragma unroll
        for (int k = 0; k < T::SEGS_PER_WAVE; ++k)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(buf + (wave + T::LOADERS * k) * 1024), 16, v_voff, WS * k, 0, 0);
    };
    // Buffer bases pass through an empty statement as scalars, so that the compiler cannot split a constant
    // out of them into every read's address (it would be negative, which the offset field cannot hold).
    // An LDS address as a plain number: this kernel declares no static LDS, so its dynamic LDS starts at
    // address 0.  A constant built this way folds into the reads' offset fields; one built from the
    // dynamic-LDS symbol keeps an add of its (zero) base per per-lane offset.
    auto lds_at = [](int byte) __attribute__((always_inline)) { return (const lds_char*)(uintptr_t)byte; };
    auto kbuf_of = [&](int j) __attribute__((always_inline)) {
        int o = (j % T::NK) * T::TILE;
        __asm__ volatile("" : "+s"(o));
        return (const lds_char*)(lds + o);
    };
    // V buffer j: relative to the V region in the eight-wave kernel (its V offsets carry the region's base, so
    // that constant buffer bases fit the reads' offset fields), absolute in the four-wave one
    constexpr int VBASE = T::NW == 8 ? T::NK * T::TILE : 0;
    auto vbuf_of = [&](int j) __attribute__((always_inline)) {
        int o = (T::NK - VBASE / T::TILE + (j % T::NV)) * T::TILE;
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
            v_roff[db] = VBASE + (8 * h + e) * T::ROW + 16 * (chunk ^ v_swz<D>(e)) + 8 * (s4 & 1);
        }
    }

    f32x16 acc[T::NDB];
#pragma unroll
    for (int db = 0; db < T::NDB; ++db) acc[db] = f32x16{};
    float m = -INFINITY, l = 0.f, alpha_prev = 1.f;
    [[maybe_unused]] float lt = 0.f;   // sum of the weights' bf16 roundings (the values P.V accumulates)
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
        // slot j of key block kb holds key kt + 8h + (32 kb + 16 (j >> 3) + (j & 7)): one per-lane threshold
        // against compile-time slot offsets, so no per-slot key index is kept in a register
        const int thr = lim - kt - 8 * h;
#pragma unroll
        for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                // all ones where the key is past the limit; the element goes through a local first, since
                // this compiler's __builtin_bit_cast of a vector-element operand reads element 0
                const unsigned msk = (unsigned)((thr - (32 * kb + 16 * (j >> 3) + (j & 7))) >> 31);
                const float x = sc[kb][j];
                const unsigned b = __builtin_bit_cast(unsigned, x);
                sc[kb][j] = __builtin_bit_cast(float, (b & ~msk) | (0xff800000u & msk));
            }
    };
    // weights and their row sums against reference mc (the plain form, used by the rare redo)
    auto weights = [&](const f32x16 (&sc)[T::NKB], float mc, float& rt) __attribute__((always_inline)) {
        float rs = 0.f;
        rt = 0.f;
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
                for (int w = 0; w < 4; ++w) {
                    p[kb][ks][w] = pack_bf16(e[8 * ks + 2 * w], e[8 * ks + 2 * w + 1]);
                    if constexpr (T::LT) rt = add_bf16_pair(p[kb][ks][w], rt);
                }
        }
        return rs;
    };

    // One step t (see the header of this kernel).  kn = K_{t+1}, kc = K_t, vp = V_{t-1}, as restrict-qualified
    // pointers distinct from the buffers the loads issued at the step's end write (K_{t+NK}, V_{t+NV-1}), so
    // the compiler does not wait for those loads before reading; the explicit vmcnt wait before every
    // barrier is what makes that true.
    i16x4 vpl[2], vph[2];   // the first two V^T operands of the next step's P.V, read before the barrier
    auto step = [&](auto do_soft, auto do_pv, auto do_s, int t, const lds_char* __restrict__ kn,
                    const lds_char* __restrict__ kc, const lds_char* __restrict__ vp,
                    const lds_char* __restrict__ vnx) __attribute__((always_inline)) {
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
        u32x4 kv[T::NS];
        auto kread = [&](int i) __attribute__((always_inline)) {
            kv[i] = *(const lds_u32x4*)(kn + k_roff[i / T::NKB] + 32 * (i % T::NKB) * T::ROW);
        };
        // ---- part 1: P.V(t-1) (two transpose reads per MFMA, two MFMAs ahead) with the exps of tile t.
        // The wave runs part 1, which carries most of the step's VALU work, at raised priority and part 2 at the
        // base one: where the two waves of a SIMD are in different parts, the exponentials issue first and the
        // other wave's S MFMAs keep the matrix pipe busy meanwhile.  Against no priorities: +2.0 % at d = 64
        // (peaky 16k); at d = 128 +0.8 to +1.0 % while all eight waves loaded tiles, +-0 since only waves 0 .. 3
        // do.  Raising part 2 instead measured -1.5 % at d = 64 and -0.6 % at d = 128.
        __builtin_amdgcn_s_setprio(1);
        {
            i16x4 vl[T::NPV], vhh[T::NPV];
            auto vread = [&](int i) __attribute__((always_inline)) {
                const int kb = i / (2 * T::NDB), ks = (i / T::NDB) & 1, db = i % T::NDB;
                const lds_char* q = vp + v_roff[db] + (32 * kb + 16 * ks) * T::ROW;
                vl[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)q);
                vhh[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(q + 4 * T::ROW));
            };
            if constexpr (PV) {
                if constexpr (T::VAHEAD) {
                    vl[0] = vpl[0];
                    vhh[0] = vph[0];
                    vl[1] = vpl[1];
                    vhh[1] = vph[1];
                } else {
                    vread(0);
                    vread(1);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < T::NPV; ++i) {
                if constexpr (PV) {
                    if (i + 2 < T::NPV) vread(i + 2);
                    const int kb = i / (2 * T::NDB), ks = (i / T::NDB) & 1, db = i % T::NDB;
                    const u32x4 vv = {__builtin_bit_cast(u32x2, vl[i])[0], __builtin_bit_cast(u32x2, vl[i])[1],
                                      __builtin_bit_cast(u32x2, vhh[i])[0], __builtin_bit_cast(u32x2, vhh[i])[1]};
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vv), as_bf16x8(p[kb][ks]), acc[db], 0, 0, 0);
                }
                if constexpr (SOFT) {
#pragma unroll
                    for (int x = T::EXP_PER_PV * i; x < T::EXP_PER_PV * (i + 1); ++x)
                        e[x] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[x >> 4][x & 15], c, -mc));
                }
                if constexpr (S && PV) {
                    if (i >= T::NPV - 2) kread(i - (T::NPV - 2));   // the first K operands of part 2, under the last P.V MFMAs
                }
                if constexpr (PV) __builtin_amdgcn_sched_barrier(0);
            }
        }
        // ---- part 2: S(t+1) (one K read per MFMA, two MFMAs ahead) with the sums and packs of tile t
        __builtin_amdgcn_s_setprio(0);
        float rs = 0.f;   // the tile's weight sum, accumulated pair by pair under the S MFMAs
        [[maybe_unused]] float rt = 0.f;   // and the sum of their bf16 roundings
        {
            if constexpr (S && !PV) {
                kread(0);
                kread(1);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < T::NS; ++i) {
                if constexpr (S) {
                    if (i + 2 < T::NS) kread(i + 2);
                    const int ks = i / T::NKB, kb = i % T::NKB;
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kv[i]), qf[ks], ks == 0 ? f32x16{} : s[kb], 0, 0, 0);
                }
                if constexpr (SOFT) {
#pragma unroll
                    for (int y = T::PAIRS_PER_S * i; y < T::PAIRS_PER_S * (i + 1); ++y) {
                        const float pair = e[2 * y] + e[2 * y + 1];
                        rs = y == 0 ? pair : rs + pair;
                        p[y >> 3][(y >> 2) & 1][y & 3] = pack_bf16(e[2 * y], e[2 * y + 1]);
                        __asm__ volatile("" ::"v"(p[y >> 3][(y >> 2) & 1][y & 3]));   // keep the pack in this slot
                        if constexpr (T::LT) rt = add_bf16_pair(p[y >> 3][(y >> 2) & 1][y & 3], rt);
                    }
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
                rs = weights(sc, mcr, rt);
            }
            l = __builtin_fmaf(l, alpha, rs);
            if constexpr (T::LT) lt = __builtin_fmaf(lt, alpha, rt);
        }
        if constexpr (SOFT && T::VAHEAD) {
            // the next step's first two V^T operands (V_t, landed by the previous retire), under this barrier
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const lds_char* q = vnx + v_roff[i];
                vpl[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)q);
                vph[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(q + 4 * T::ROW));
            }
        }
    };
    // End of step t: the loads of K_{t+2} and V_{t+VAHEAD} have landed (each loading wave waits for its own
    // before the barrier) and every wave is done with K_t and V_{t-1}; K_{t+NK} and V_{t+NV-1} then go into
    // their buffers.  All waves run exactly ntiles such barriers.
    auto retire = [&](int t) __attribute__((always_inline)) {
        // K_{t+2} and V_{t+VAHEAD} were issued steps ago; the loads of the later retires may still fly (when
        // all of them exist; near the end, and after step 0, whose lead loads the prologue issued in another
        // order, wait for everything)
        if (t > 0 && t - 1 + T::LEAD < ntiles) __builtin_amdgcn_s_waitcnt(0x0F70 | T::AFTER);
        else __builtin_amdgcn_s_waitcnt(0x0F70);
        if constexpr (T::VAHEAD) lds_barrier_keep4();
        else lds_barrier();
        load_k(t + T::NK);
        load_v(t + T::NV - 1);
    };
    using yes = std::integral_constant<bool, true>;
    using no = std::integral_constant<bool, false>;

    // ---- prologue: K_0 and K_1 must land (in every wave) before S(0) and S(1); the other lead loads (K_2 ..
    // K_{NK-1}, V_0 .. V_{NV-2}) are issued after that barrier and land under S(0) and step 0
    load_k(0);
    load_k(1);
    if constexpr (T::VAHEAD) load_v(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    lds_barrier();
    for (int j = 2; j < T::NK; ++j) load_k(j);
    for (int j = T::VAHEAD; j < T::NV - 1; ++j) load_v(j);

    // Steps 0 .. nt-1 (step t: softmax of tile t, P.V of t-1, S of t+1), then the P.V of the last tile.
    const int nt = wave_tiles;
    int t = 0;
    // The wave's 32 rows of the running partial (when there is one) and of the output are addressed through
    // buffer resources bounded at the last query row: loads past it return zeros and stores are dropped.
    const int rows_left = __builtin_amdgcn_readfirstlane(max(0, min(32, a.n_q - qw0)));   // uniform, kept scalar
    // Output rows move in 16-byte pieces: PPR pieces of four floats per fp32 row (RPI rows per wave
    // instruction), BPPR pieces of eight bf16 per bf16 row (BRPI rows per instruction).
    constexpr int PPR = D / 4, RPI = 64 / PPR, BPPR = D / 8, BRPI = 64 / BPPR;
    // The running partial, in the order the epilogue writes: with fp32 output lane l holds floats
    // 4*(l%PPR)..+3 of row RPI*k + l/PPR in prev[k]; with bf16 output floats 8*(l%BPPR) + 4*(k%2)..+3 of
    // row BRPI*(k/2) + l/BPPR.  Either way D/8 pieces per lane.
    f32x4 prev[D / 8];
    float lse_pv = -INFINITY;   // lse of the partial for row qw0 + col
    auto fetch_prev = [&]() __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(a.o_prev + (size_t)bh * a.q_head_stride + (size_t)qw0 * D), (short)0, rows_left * D * 4, BUF_RSRC_WORD3);
        const int voff = OUT_F32 ? (lane / PPR) * D * 4 + 16 * (lane % PPR) : (lane / BPPR) * D * 4 + 32 * (lane % BPPR);
#pragma unroll
        for (int k = 0; k < D / 8; ++k) {
            const int koff = OUT_F32 ? RPI * k * D * 4 : BRPI * (k >> 1) * D * 4 + 16 * (k & 1);
            prev[k] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, koff, 0));
        }
        if (col < rows_left) lse_pv = a.lse_prev[(size_t)bh * a.n_q + qw0 + col];
    };
    if (nt > 0) {
        s_all(s, kbuf_of(0));
        // The reference starts at tile 0's row max, taken here while its scores are still in registers, so that
        // step 0 does not redo the tile (recomputing its scores from K_0) as a row without a reference would.
        // A row whose tile-0 keys are all masked keeps no reference (m = -inf) and is redone as before.
        {
            if (0 >= full_tiles) mask_tile(0, s);
            float mt = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j) mt = fmaxf(mt, s[kb][j]);
            m = fmaxf(mt, wave_xor32(mt));
            mcr = m == -INFINITY ? 0.f : m * c;
            bnd = m == -INFINITY ? -1.f : REF_BOUND;
        }
        // Step 0: the softmax of tile 0 and S(1).  A wave with a single tile runs the same step (one call site
        // for both cases, so no second copy of the read offsets is kept across the loop) with its S part
        // recomputing the scores of tile 0, which nothing reads: its weights are already packed for P.V.
        step(yes{}, no{}, yes{}, 0, kbuf_of(nt > 1 ? 1 : 0), kbuf_of(0), vbuf_of(0), vbuf_of(0));
        if (nt > 1) {
            retire(0);
            // middle steps, four at a time with every buffer base a constant (t = 1 mod 4 at the start of
            // each group: K_{t+1}, K_t and V_{t-1} sit in buffers 2, 1 and 0, then 3, 2, 1, ...)
            static_assert((T::NK == 4 && T::NV == 4) || T::NW != 8, "the unrolled steps assume four K and four V buffers");
            t = 1;
            if constexpr (T::NW == 8) {
                for (; t + 4 < nt; t += 4) {
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int ph = (1 + u) & 3;   // t + u mod 4
                        step(yes{}, yes{}, yes{}, t + u, lds_at(((ph + 1) & 3) * T::TILE), lds_at(ph * T::TILE),
                             lds_at(((ph + 3) & 3) * T::TILE), lds_at(ph * T::TILE));
                        retire(t + u);
                    }
                }
            }
            for (; t < nt - 1; ++t) {
                step(yes{}, yes{}, yes{}, t, kbuf_of(t + 1), kbuf_of(t), vbuf_of(t - 1), vbuf_of(t));
                retire(t);
            }
            step(yes{}, yes{}, no{}, t, kbuf_of(t), kbuf_of(t), vbuf_of(t - 1), vbuf_of(t));   // no next S
        }
        // P.V of the last tile, after the barrier that ends its step: that barrier is what makes the last V
        // tile visible (every wave waited for its loads of it), and it does not reload that V buffer
        retire(t);
        ++t;
        // the running partial is loaded now, to arrive during the last P.V
        if (a.o_prev) fetch_prev();
        step(no{}, yes{}, no{}, t, kbuf_of(t), kbuf_of(t), vbuf_of(nt - 1), vbuf_of(nt - 1));
    } else if (a.o_prev) {
        fetch_prev();
    }
    for (; t < ntiles; ++t) retire(t);   // the rest of the workgroup's barriers and loads

    // ---- epilogue: one division by the final denominator, lse = scaled reference + ln(l), and the fold
    // into the running partial (two-term merge: M = max of the two lse, weights exp(lse - M) normalised to
    // sum 1, lse = M + ln of their sum).  Lane (col, h) holds head-dim elements 32*db + 8*g + 4*h + (0..3)
    // of its row; the scaled rows go through LDS so that loads and stores cover whole rows.
    {
        // The lane id passes through an empty statement here, so that the epilogue's per-lane addresses are
        // formed after the key loop instead of being hoisted above it and kept (in private memory) across it.
        int lane = tid & 63;
        __asm__ volatile("" : "+v"(lane));
        const int col = lane & 31;
        const int qi = qw0 + col;
        const float l_tot = l + wave_xor32(l);
        const float lb = l_tot > 0.f ? m * scale_abs + logf(l_tot) : -INFINITY;
        float cb = l_tot > 0.f ? 1.f / l_tot : 0.f;   // factor on this launch's accumulator
        if constexpr (T::LT) {
            const float lt_tot = lt + wave_xor32(lt);
            cb = l_tot > 0.f && lt_tot > 0.f ? 1.f / lt_tot : 0.f;
        }
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
        // A free tile buffer per wave (32 fp32 rows fill one): after the last barrier only the V buffer of the
        // last tile may still be read (by waves finishing their last P.V); nothing else is read or loaded.
        static_assert(32 * D * 4 == T::TILE, "a wave's fp32 rows fill one tile buffer");
        const int busy = ntiles > 0 ? T::NK + (ntiles - 1) % T::NV : T::NK + T::NV;
        const int slot = wave < busy ? wave : wave + 1;
        lds_char* const st = lds + slot * T::TILE;
        // row r, 16-byte piece q at piece q ^ (r mod PPR) of the row (conflict-free writes and reads); every
        // r here is below 32, so with 32 pieces per row the reduction is left out
        auto pswz = [](int r) __attribute__((always_inline)) { return PPR == 32 ? r : r % PPR; };
#pragma unroll
        for (int db = 0; db < T::NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int q = 8 * db + 2 * g + h;
                const f32x4 o4 = {acc[db][4 * g] * cb, acc[db][4 * g + 1] * cb, acc[db][4 * g + 2] * cb,
                                  acc[db][4 * g + 3] * cb};
                *(lds_f32x4*)(st + col * (D * 4) + 16 * (q ^ pswz(col))) = o4;
            }
        __asm__ volatile("" ::: "memory");   // the reads below see this wave's writes (LDS keeps a wave's order)
        const int ca_bits = __builtin_bit_cast(int, ca);
        const size_t obase = (size_t)bh * a.q_head_stride + (size_t)qw0 * D;
        if constexpr (OUT_F32) {
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(static_cast<float*>(a.o) + obase), (short)0, rows_left * D * 4, BUF_RSRC_WORD3);
            const int q = lane % PPR;
            f32x4 o4[32 / RPI];
#pragma unroll
            for (int k = 0; k < 32 / RPI; ++k) {
                const int r = RPI * k + lane / PPR;
                o4[k] = *(const lds_f32x4*)(st + r * (D * 4) + 16 * (q ^ pswz(r)));
            }
            if (a.o_prev) {
#pragma unroll
                for (int k = 0; k < 32 / RPI; ++k) {
                    const int r = RPI * k + lane / PPR;
                    o4[k] += __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * r, ca_bits)) * prev[k];
                }
            }
            const int voff = (lane / PPR) * D * 4 + 16 * q;
#pragma unroll
            for (int k = 0; k < 32 / RPI; ++k)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o4[k]), rs, voff, RPI * k * D * 4, 0);
        } else {
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(static_cast<uint16_t*>(a.o) + obase), (short)0, rows_left * D * 2, BUF_RSRC_WORD3);
            const int q = lane % BPPR;
            f32x4 lo[32 / BRPI], hi[32 / BRPI];
#pragma unroll
            for (int k = 0; k < 32 / BRPI; ++k) {
                const int r = BRPI * k + lane / BPPR;
                lo[k] = *(const lds_f32x4*)(st + r * (D * 4) + 16 * ((2 * q) ^ pswz(r)));
                hi[k] = *(const lds_f32x4*)(st + r * (D * 4) + 16 * ((2 * q + 1) ^ pswz(r)));
            }
            if (a.o_prev) {
#pragma unroll
                for (int k = 0; k < 32 / BRPI; ++k) {
                    const int r = BRPI * k + lane / BPPR;
                    const float car = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * r, ca_bits));
                    lo[k] += car * prev[2 * k];
                    hi[k] += car * prev[2 * k + 1];
                }
            }
            const int voff = (lane / BPPR) * D * 2 + 16 * q;
#pragma unroll
            for (int k = 0; k < 32 / BRPI; ++k) {
                const u32x4 o4 = {pack_bf16(lo[k][0], lo[k][1]), pack_bf16(lo[k][2], lo[k][3]),
                                  pack_bf16(hi[k][0], hi[k][1]), pack_bf16(hi[k][2], hi[k][3])};
                __builtin_amdgcn_raw_buffer_store_b128(o4, rs, voff, BRPI * k * D * 2, 0);
            }
        }
    }
}

template <int NW, int D, bool CAUSAL, bool OUT_F32>
hipError_t launch_p3(const FwdArgs& a, hipStream_t st) {
    using T = P3<NW, D>;
    const int num_qt = (a.n_q + T::BR - 1) / T::BR;
    const long long total_ll = (long long)num_qt * a.bh;
    if (total_ll > 0x7fffffffLL - NXCD) return hipErrorInvalidValue;
    if ((long long)a.n_kv * T::ROW > 0x7fffffffLL) return hipErrorInvalidValue;   // buffer bound is 31-bit
    const int total = (int)total_ll;
    const int per_xcd = (total + NXCD - 1) / NXCD;
    const int grid = per_xcd * NXCD;
    // query tiles differ in length when some row does not see every key (row 0 sees keys up to 0 + offset)
    const int length_major = CAUSAL && (long long)a.offset < (long long)a.n_kv - 1;
    auto kern = fwd_p3_kernel<NW, D, CAUSAL, OUT_F32>;
    if (hipError_t e = allow_lds<fwd_p3_kernel<NW, D, CAUSAL, OUT_F32>>(T::LDS); e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(T::THREADS), T::LDS, st, a, num_qt, total, per_xcd, length_major);
    return hipGetLastError();
}

}  // namespace

// Workgroup size of the bf16 kernel.  Eight waves (256 query rows, one workgroup per CU: both waves of a
// SIMD share each K/V tile) unless the launch has fewer such tiles than CUs, or its rows are short and causal
// (fewer than 3072 keys), where 128-row workgroups fill the chip and balance the diagonal better.  Measured
// at d = 128 against four waves with the length-major order of causal launches: +4 to +14 % on causal rows
// of 3072 to 8192 keys, +2 to +6 % without a mask from 1 to 8 tiles per CU, -4 to -6 % on causal rows of 1024
// and 2048 keys at 4 tiles per CU.  At d = 64: eight waves +1 to +4 % on causal rows of 4096 and 8192 keys and
// without a mask, four waves +4 to +7.5 % on causal rows of 512 to 2048 keys.  ATTN_BF16_D128_WAVES and
// ATTN_BF16_D64_WAVES (4 or 8) force one of them (used by the tests to run every shape through both).
static int bf16_waves(const FwdArgs& a) {
    if (const char* e = getenv(a.d == 128 ? "ATTN_BF16_D128_WAVES" : "ATTN_BF16_D64_WAVES")) {
        const int v = atoi(e);
        if (v == 4 || v == 8) return v;
    }
    const long long wide = (long long)((a.n_q + 255) / 256) * a.bh;
    if (wide < device_cus()) return 4;
    if (a.causal && a.n_kv < 3072) return 4;
    return 8;
}

hipError_t launch_fwd_bf16(const FwdArgs& a, bool out_f32, hipStream_t s) {
    const bool c = a.causal != 0;
    if (a.d == 128) {
        if (bf16_waves(a) == 8) {
            if (c) return out_f32 ? launch_p3<8, 128, true, true>(a, s) : launch_p3<8, 128, true, false>(a, s);
            return out_f32 ? launch_p3<8, 128, false, true>(a, s) : launch_p3<8, 128, false, false>(a, s);
        }
        if (c) return out_f32 ? launch_p3<4, 128, true, true>(a, s) : launch_p3<4, 128, true, false>(a, s);
        return out_f32 ? launch_p3<4, 128, false, true>(a, s) : launch_p3<4, 128, false, false>(a, s);
    }
    if (a.d == 64) {
        if (bf16_waves(a) == 8) {
            if (c) return out_f32 ? launch_p3<8, 64, true, true>(a, s) : launch_p3<8, 64, true, false>(a, s);
            return out_f32 ? launch_p3<8, 64, false, true>(a, s) : launch_p3<8, 64, false, false>(a, s);
        }
        if (c) return out_f32 ? launch_p3<4, 64, true, true>(a, s) : launch_p3<4, 64, true, false>(a, s);
        return out_f32 ? launch_p3<4, 64, false, true>(a, s) : launch_p3<4, 64, false, false>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace attn
