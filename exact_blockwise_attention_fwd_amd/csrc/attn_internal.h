// Internal interface between the C-ABI front end (attn_api.hip) and the kernels.  Not installed.
#pragma once

#include <hip/hip_runtime.h>

namespace attn {

// One forward launch over a key range.  All strides and offsets are in elements.
struct FwdArgs {
    const void* q;          // [bh][n_q][d], head stride q_head_stride
    const void* k;          // first key of the range, head stride kv_head_stride
    const void* v;
    void* o;                // [bh][n_q][d], same head stride as q
    float* lse;             // [bh][n_q]
    long long q_head_stride;
    long long kv_head_stride;
    int n_q, n_kv, d, bh;
    int causal;
    int offset;             // key j visible to query i iff j <= i + offset (clamped to [-n_q-1, n_kv])
    float scale;            // signed logit scale
    // Running partial to fold this launch's result into (both NULL: plain store).  fp32, laid out like O
    // (o_prev) and LSE (lse_prev); o_prev may equal o (fp32 output) and lse_prev may equal lse, since every
    // row is read and written by the lanes that own it.
    const float* o_prev;
    const float* lse_prev;
};

struct MergeArgs {
    const void* o_a;
    const float* lse_a;
    const void* o_b;
    const float* lse_b;
    void* o;
    float* lse;
    long long rows;
    int d;
    int in_bf16, out_bf16;
};

// One bf16 GEMM of the blockwise feed-forward: C[m][n] = act(sum_k A[m][k] B[n][k] + bias[n]) in bf16, fp32
// accumulation; A [rows][k] and B [n][k] K-contiguous, C [rows][n]; k and n multiples of 64; bias fp32 (16-byte
// aligned) or NULL.
struct GemmArgs {
    const void* a;
    const void* b;
    const float* bias;
    void* c;
    int rows, n, k;
    int act;                // 0 none, 1 ReLU, 2 GELU
};

// bf16 inputs, fp32 accumulation; d in {64, 128}; O in bf16 or fp32.
hipError_t launch_fwd_bf16(const FwdArgs& a, bool out_f32, hipStream_t s);
// fp32 inputs and output; 1 <= d <= 256.
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, hipStream_t s);
hipError_t launch_gemm_nt(const GemmArgs& g, hipStream_t s);

// Compute units of the current device, queried once per device (256 if the query fails).
int device_cus();

}  // namespace attn
