// Blockwise feed-forward on gfx950: FFN(x) = act(x W1^T + b1) W2^T + b2 for every row of a sequence, taken in
// contiguous row blocks ("Ring Attention with Blockwise Parallel Transformers" explainer, section 3:
// self-attention and the feedforward applied block by block), so the hidden activations exist for one block
// at a time.  Each block is two bf16 GEMMs with fp32 accumulation on the matrix cores; bias and activation
// are applied in the first GEMM's epilogue and the hidden block is stored in bf16, the second GEMM adds its
// bias in its epilogue.
//
// The GEMM is C[m][n] = epi(sum_k A[m][k] B[n][k]) with both operands K-contiguous (activations row-major,
// weights in the [out, in] layout), which is the layout the MFMA operands want:
//  * a workgroup computes a 256 x 256 tile of C with 8 waves (two per SIMD); wave w owns rows
//    64*(w%4) .. +63 and columns 128*(w/4) .. +127, as 2 x 4 blocks of 32 x 32.  (FFN_GEMM_WAVES=4 builds
//    the 4-wave form, 128 x 128 per wave: fewer LDS reads per MFMA, but with one wave per SIMD it measured
//    about 10 % slower, and it needs the accumulators in AGPRs);
//  * the tile is computed transposed (C^T = B A^T, v_mfma_f32_32x32x16_bf16 with A = B rows and B = A rows)
//    so that every lane ends with one row m of C and 4-element runs of its columns; the epilogue stages
//    each wave's bf16 sub-tile in LDS and stores whole row segments;
//  * K advances in tiles of 64: A and B tiles (256 rows x 128 bytes each) move HBM -> LDS with
//    buffer_load_dwordx4 ... lds, one barrier per k-tile, into rings of two A and three B tiles (the whole
//    160 KiB of LDS): A tile k+1 and B tile k+2 load while tile k is computed.  B tiles (weights) get the
//    longer lead because fewer of the concurrently running workgroups share each of them, so more of their
//    loads miss L2 (measured on the whole feed-forward: +4.4 % against two stages of both, +1.9 % with the
//    roles swapped).  Rows past the end of A or B read as zeros (the buffer resource's bound).  The
//    MFMAs of a k-tile's last 16-deep quarter are issued after the next barrier, under that tile's first
//    LDS reads (measured against 32-deep k-tiles in a ring of four: +5 % and +15 % on the two GEMMs);
//  * LDS rows are XOR-swizzled in 16-byte units (chunk c of row r sits in slot c ^ ((r >> 1) & 7)) so that
//    the operand reads of each 16-lane group hit 16 distinct bank groups; the swizzle is applied through
//    the global chunk each lane fetches;
//  * workgroups are ordered in groups of 4 row tiles with the column tile varying slowest inside a group,
//    and each XCD takes a contiguous range of that order, so concurrently running tiles share A and B
//    tiles in the XCD's L2 (groups of 8 speed up the 4096-column product by 3 % when it runs back to back,
//    but not inside the feed-forward, where it follows the other product; 2 and 16 are slower).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "attn_internal.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;

constexpr int NXCD = 8;
constexpr unsigned BUF_RSRC_WORD3 = 0x00020000u;   // raw buffer, 32-bit data format, bounds-checked

constexpr int G_BM = 256, G_BN = 256, G_BK = 64;    // C tile and k-tile
#ifndef FFN_GEMM_WAVES
#define FFN_GEMM_WAVES 8
#endif
constexpr int G_NW = FFN_GEMM_WAVES, G_THREADS = 64 * G_NW;
constexpr int G_WGM = G_NW == 8 ? 4 : 2;             // waves along the tile's rows (the rest along its columns)
constexpr int G_MB = G_BM / G_WGM / 32, G_NB = G_BN / (G_NW / G_WGM) / 32;   // 32 x 32 blocks per wave
// LDS rings: two A (activation) tiles and three B (weight) tiles, so that B tile k+2 loads while k computes and A
// tile k+1 (A tiles are shared by more of the concurrently running workgroups, so they hit L2 more often)
constexpr int G_STAGES_A = 2, G_STAGES_B = 3;
constexpr int G_ROW = 2 * G_BK;                     // 128 bytes per LDS row
constexpr int G_TILE = G_BM * G_ROW;                // 32 KiB per operand tile
constexpr int G_B0 = G_STAGES_A * G_TILE;           // the B ring follows the A ring
constexpr int G_LDS = (G_STAGES_A + G_STAGES_B) * G_TILE;   // 160 KiB
constexpr int G_SEGS = G_TILE / 1024;               // 1 KiB load segments per operand tile
constexpr int G_SEG_PER_WAVE = G_SEGS / G_NW;       // per operand and k-tile
constexpr int G_GROUP_M = 4;
static_assert(G_SEGS % G_NW == 0, "tiling");
static_assert(G_SEG_PER_WAVE < 16, "loads allowed in flight fit the s_waitcnt vmcnt field");

enum { ACT_NONE = 0, ACT_RELU = 1, ACT_GELU = 2 };

__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 p = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(unsigned, p);
}

// erf(z) by Abramowitz and Stegun, Handbook of Mathematical Functions, formula 7.1.26: for z >= 0,
// erf(z) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-z^2) with t = 1 / (1 + p z), |error| <= 1.5e-7;
// odd in z.  About a dozen instructions against the library erff's few dozen, and far below the bf16
// rounding the hidden block receives next.
__device__ __forceinline__ float erf_as(float z) {
    const float a = fabsf(z);
    const float t = __frcp_rn(__builtin_fmaf(0.3275911f, a, 1.f));
    float poly = __builtin_fmaf(1.061405429f, t, -1.453152027f);
    poly = __builtin_fmaf(poly, t, 1.421413741f);
    poly = __builtin_fmaf(poly, t, -0.284496736f);
    poly = __builtin_fmaf(poly, t, 0.254829592f);
    poly *= t;
    const float e = __builtin_amdgcn_exp2f(-a * a * 1.4426950408889634f);   // exp(-z^2)
    return copysignf(__builtin_fmaf(-poly, e, 1.f), z);
}

template <int ACT>
__device__ __forceinline__ float activate(float x) {
    if constexpr (ACT == ACT_RELU) return fmaxf(x, 0.f);
    else if constexpr (ACT == ACT_GELU) return 0.5f * x * (1.f + erf_as(x * 0.70710678118654752f));
    else return x;
}

template <int ACT>
__global__ __launch_bounds__(G_THREADS, 1) void gemm_nt_kernel(GemmArgs g, int tiles_m, int tiles_n, int total,
                                                               int per_xcd) {
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    lds_char* const lds = (lds_char*)smem;

    const int w_hw = blockIdx.x;
    const int logical = (w_hw % NXCD) * per_xcd + w_hw / NXCD;
    if (logical >= total) return;
    const int group = logical / (G_GROUP_M * tiles_n);
    const int first_m = group * G_GROUP_M;
    const int gm = min(G_GROUP_M, tiles_m - first_m);
    const int idx = logical % (G_GROUP_M * tiles_n);
    const int tm = first_m + idx % gm, tn = idx / gm;
    const int m0 = tm * G_BM, n0 = tn * G_BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, col = lane & 31;
    const int K = g.k;
    const int nk = K / G_BK;

    // ---- loads: this wave fills segments wave + 8j of the A and the B tile of every k-tile.  Lane L writes
    // LDS row 8*seg + L/8, slot L%8, which must hold chunk (L%8) ^ swz(row) of that row.
    const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const char*)g.a + (size_t)m0 * K * 2), (short)0, (g.rows - m0) * K * 2, BUF_RSRC_WORD3);
    const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const char*)g.b + (size_t)n0 * K * 2), (short)0, (g.n - n0) * K * 2, BUF_RSRC_WORD3);
    int voff[G_SEG_PER_WAVE];
#pragma unroll
    for (int j = 0; j < G_SEG_PER_WAVE; ++j) {
        const int row = 8 * (wave + G_NW * j) + lane / 8;
        voff[j] = row * K * 2 + 16 * ((lane % 8) ^ swz(row));
    }
    auto issue_a = [&](int kt) {
        if (kt >= nk) return;
        lds_char* st = lds + (kt % G_STAGES_A) * G_TILE;
#pragma unroll
        for (int j = 0; j < G_SEG_PER_WAVE; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, (lds_void*)(st + (wave + G_NW * j) * 1024), 16, voff[j],
                                                     kt * G_ROW, 0, 0);
    };
    auto issue_b = [&](int kt) {
        if (kt >= nk) return;
        lds_char* st = lds + G_B0 + (kt % G_STAGES_B) * G_TILE;
#pragma unroll
        for (int j = 0; j < G_SEG_PER_WAVE; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(brs, (lds_void*)(st + (wave + G_NW * j) * 1024), 16, voff[j],
                                                     kt * G_ROW, 0, 0);
    };

    // ---- operand reads: row col of a 32-row block, k-chunk 2*ks + h (8 bf16) of the k-tile; slot
    // (2*ks + h) ^ swz = (h ^ swz) ^ 2*ks, so quarter ks flips bits of the ks = 0 offset
    const int wm0 = 32 * G_MB * (wave % G_WGM), wn0 = 32 * G_NB * (wave / G_WGM);
    int aro[G_MB], bro[G_NB];   // byte offsets within a stage's A / B tile, for ks = 0
#pragma unroll
    for (int mb = 0; mb < G_MB; ++mb) {
        const int r = wm0 + 32 * mb + col;
        aro[mb] = r * G_ROW + 16 * (h ^ swz(r));
    }
#pragma unroll
    for (int nb = 0; nb < G_NB; ++nb) {
        const int r = wn0 + 32 * nb + col;
        bro[nb] = r * G_ROW + 16 * (h ^ swz(r));
    }

    f32x16 acc[G_NB][G_MB];
#pragma unroll
    for (int nb = 0; nb < G_NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < G_MB; ++mb) acc[nb][mb] = f32x16{};

    // Fragments of two 16-deep quarters of a k-tile, alternating.  The MFMAs of the last quarter of k-tile
    // kt run after the barrier of k-tile kt + 1, while that tile's first fragments are read, so every
    // barrier is followed by MFMA work that needs no new LDS data.
    u32x4 af0[G_MB], bf0[G_NB], af1[G_MB], bf1[G_NB];
    auto read = [&](const lds_char* sa, const lds_char* sb, int ks, u32x4 (&af)[G_MB], u32x4 (&bf)[G_NB]) {
#pragma unroll
        for (int mb = 0; mb < G_MB; ++mb) af[mb] = *(const lds_u32x4*)(sa + (aro[mb] ^ (32 * ks)));
#pragma unroll
        for (int nb = 0; nb < G_NB; ++nb) bf[nb] = *(const lds_u32x4*)(sb + (bro[nb] ^ (32 * ks)));
    };
    auto mma = [&](const u32x4 (&af)[G_MB], const u32x4 (&bf)[G_NB]) {
#pragma unroll
        for (int nb = 0; nb < G_NB; ++nb)
#pragma unroll
            for (int mb = 0; mb < G_MB; ++mb)
                acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, bf[nb]), __builtin_bit_cast(bf16x8, af[mb]), acc[nb][mb], 0, 0, 0);
    };
    // At k-tile kt this wave's loads of A_kt and B_kt have landed, and B_{kt+1} (issued after them) may still
    // fly; after the barrier every wave's have, and every wave is done reading A_{kt-1} and B_{kt-1}, whose
    // buffers A_{kt+1} and B_{kt+2} then take (issued A first, so the count of later loads is B's).
    auto land = [&](int kt) {
        if (kt + 1 < nk) __builtin_amdgcn_s_waitcnt(0x0F70 | G_SEG_PER_WAVE);
        else __builtin_amdgcn_s_waitcnt(0x0F70);
        lds_barrier();
        issue_a(kt + 1);
        issue_b(kt + 2);
    };

    issue_a(0);
    issue_b(0);
    issue_b(1);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // everything of the prologue (A_0 .. B_1) before the first barrier
    lds_barrier();
    issue_a(1);
    issue_b(2);
    const lds_char* sa = lds;
    const lds_char* sb = lds + G_B0;
    read(sa, sb, 0, af0, bf0);
    read(sa, sb, 1, af1, bf1);
    mma(af0, bf0);
    read(sa, sb, 2, af0, bf0);
    mma(af1, bf1);
    read(sa, sb, 3, af1, bf1);
    mma(af0, bf0);
    for (int kt = 1; kt < nk; ++kt) {
        land(kt);
        sa = lds + (kt % G_STAGES_A) * G_TILE;
        sb = lds + G_B0 + (kt % G_STAGES_B) * G_TILE;
        read(sa, sb, 0, af0, bf0);
        __builtin_amdgcn_sched_barrier(0);
        mma(af1, bf1);                     // last quarter of k-tile kt - 1
        __builtin_amdgcn_sched_barrier(0);
        read(sa, sb, 1, af1, bf1);
        __builtin_amdgcn_sched_barrier(0);
        mma(af0, bf0);
        __builtin_amdgcn_sched_barrier(0);
        read(sa, sb, 2, af0, bf0);
        __builtin_amdgcn_sched_barrier(0);
        mma(af1, bf1);
        __builtin_amdgcn_sched_barrier(0);
        read(sa, sb, 3, af1, bf1);
        __builtin_amdgcn_sched_barrier(0);
        mma(af0, bf0);
        __builtin_amdgcn_sched_barrier(0);
    }
    mma(af1, bf1);

    // ---- epilogue: lane holds C[m][n] for tile row wm0 + 32*mb + col and tile column wn0 + 32*nb + 8*q + 4*h + r
    // (accumulator element 4*q + r).  Bias and activation in fp32, bf16 into this wave's part of LDS (its
    // sub-tile, 128 columns = 256 bytes per row, 16-byte unit u of row r kept at unit u ^ (r & 15) so that both
    // the writes and the row reads are conflict-free), then whole 256-byte row segments to memory, four rows
    // per store instruction (8-byte stores straight from the accumulators left partial lines that reached
    // HBM twice over).
    lds_barrier();   // every wave is done reading the operand stages
    static_assert(G_NB == 4 && G_NW * 32 * G_MB * 256 <= G_LDS, "epilogue staging: 256-byte rows, 16 units");
    lds_char* const ct = lds + wave * (32 * G_MB * 256);
#pragma unroll
    for (int mb = 0; mb < G_MB; ++mb) {
        const int r = 32 * mb + col;
#pragma unroll
        for (int nb = 0; nb < G_NB; ++nb) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int unit = 4 * nb + q;
                const int n = n0 + wn0 + 8 * unit + 4 * h;
                const f32x4 b4 = (g.bias && n < g.n) ? *reinterpret_cast<const f32x4*>(g.bias + n)
                                                     : f32x4{0.f, 0.f, 0.f, 0.f};
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = activate<ACT>(acc[nb][mb][4 * q + e] + b4[e]);
                *(lds_u32x2*)(ct + r * 256 + 16 * (unit ^ (r & 15)) + 8 * h) =
                    u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
            }
        }
    }
    const int u = lane % 16;
#pragma unroll
    for (int i = 0; i < 8 * G_MB; ++i) {
        const int r = 4 * i + lane / 16;
        const int m = m0 + wm0 + r, n = n0 + wn0 + 8 * u;
        const u32x4 val = *(const lds_u32x4*)(ct + r * 256 + 16 * (u ^ (r & 15)));
        if (m < g.rows && n < g.n) *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(g.c) + (size_t)m * g.n + n) = val;
    }
}

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

template <int ACT>
hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
    const int tiles_m = (g.rows + G_BM - 1) / G_BM, tiles_n = (g.n + G_BN - 1) / G_BN;
    const int total = tiles_m * tiles_n;
    const int per_xcd = (total + NXCD - 1) / NXCD;
    if (hipError_t e = allow_lds<gemm_nt_kernel<ACT>>(G_LDS); e != hipSuccess) return e;
    hipLaunchKernelGGL(gemm_nt_kernel<ACT>, dim3(per_xcd * NXCD), dim3(G_THREADS), G_LDS, s, g, tiles_m, tiles_n,
                       total, per_xcd);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_nt(const GemmArgs& g, hipStream_t s) {
    switch (g.act) {
        case ACT_RELU: return launch_gemm<ACT_RELU>(g, s);
        case ACT_GELU: return launch_gemm<ACT_GELU>(g, s);
        default: return launch_gemm<ACT_NONE>(g, s);
    }
}

}  // namespace attn
