// C-ABI front end of libattn.so (declared in include/attn.h): argument validation before any HIP call,
// kernel dispatch by dtype and head dimension, the chunked driver, and opt-in launch timing.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "attn.h"
#include "attn_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

bool debug_sync() {
    static const bool on = [] {
        const char* e = getenv("ATTN_DEBUG");
        return e && e[0] == '1';
    }();
    return on;
}

// ---------------------------------------------------------------------------------------- launch timing
// Kinds of timed work (the length of attn_timing_read's arrays): forward kernel, merge kernel, chunk copy,
// feed-forward GEMM.
constexpr int kTimingKinds = 4;
struct Timed {
    int kind;
    hipEvent_t start, stop;
};
std::mutex g_timing_mu;
bool g_timing_on = false;
std::vector<Timed> g_timed;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t take_event() {
    if (!g_event_pool.empty()) {
        hipEvent_t e = g_event_pool.back();
        g_event_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Synchronisation events of attn_fwd_streamed, five per call (two "copied", two "done" and one "entry").  A
// set goes back to the pool with the event that completes last; it is handed out again only once that event
// has completed, so no pending wait or record of an earlier call can see it re-recorded.
constexpr int kQuadEvents = 5;
struct EventQuad {
    hipEvent_t e[kQuadEvents];
    hipEvent_t last;
};
std::mutex g_quad_mu;
std::vector<EventQuad*> g_quads;

EventQuad* take_quad() {
    {
        std::lock_guard<std::mutex> g(g_quad_mu);
        for (size_t i = 0; i < g_quads.size(); ++i) {
            EventQuad* q = g_quads[i];
            if (!q->last || hipEventQuery(q->last) == hipSuccess) {
                g_quads.erase(g_quads.begin() + i);
                return q;
            }
        }
    }
    EventQuad* q = new EventQuad{};
    for (int k = 0; k < kQuadEvents; ++k) {
        if (hipEventCreateWithFlags(&q->e[k], hipEventDisableTiming) != hipSuccess) {
            for (int j = 0; j < k; ++j) (void)hipEventDestroy(q->e[j]);
            delete q;
            return nullptr;
        }
    }
    return q;
}

void give_quad(EventQuad* q, hipEvent_t last) {
    q->last = last;
    std::lock_guard<std::mutex> g(g_quad_mu);
    g_quads.push_back(q);
}

// Runs one launch with optional timing and debug synchronisation; maps HIP failures to ATTN_ERR_HIP.
template <class F>
int run(int kind, hipStream_t s, const char* what, F&& launch) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    bool timed = false;
    {
        std::lock_guard<std::mutex> g(g_timing_mu);
        if (g_timing_on) {
            e0 = take_event();
            e1 = take_event();
            timed = e0 && e1;
        }
    }
    auto give_back = [&] {   // events of a launch that will not be timed go back to the pool
        std::lock_guard<std::mutex> g(g_timing_mu);
        if (e0) g_event_pool.push_back(e0);
        if (e1) g_event_pool.push_back(e1);
    };
    if (timed && hipEventRecord(e0, s) != hipSuccess) {
        give_back();
        return fail(ATTN_ERR_HIP, "%s: hipEventRecord failed", what);
    }
    hipError_t err = launch();
    if (err != hipSuccess) {
        give_back();
        return fail(ATTN_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(err));
    }
    if (timed) {
        if (hipEventRecord(e1, s) != hipSuccess) {
            give_back();
            return fail(ATTN_ERR_HIP, "%s: hipEventRecord failed", what);
        }
        std::lock_guard<std::mutex> g(g_timing_mu);
        g_timed.push_back({kind, e0, e1});
    } else if (e0 || e1) {
        give_back();
    }
    if (debug_sync()) {
        err = hipStreamSynchronize(s);
        if (err != hipSuccess) return fail(ATTN_ERR_HIP, "%s: kernel failed: %s", what, hipGetErrorString(err));
    }
    return ATTN_OK;
}

// ------------------------------------------------------------------------------------------- validation
size_t esize(attn_dtype t) { return t == ATTN_BF16 ? 2 : 4; }
bool valid_dtype(int t) { return t == ATTN_F32 || t == ATTN_BF16; }

bool overlap(const void* a, size_t an, const void* b, size_t bn) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return an && bn && x < y + bn && y < x + an;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// No array this library reads or writes may span 2^56 bytes (64 PiB, far past any device's memory); every byte
// count below is first formed in 128-bit arithmetic and checked against that bound, so none of them wraps.
constexpr __int128 kMaxBytes = (__int128)1 << 56;

struct FwdCheck {
    size_t q_bytes, kv_bytes, o_bytes, lse_bytes;
    long long kv_stride;
};

// Launch limits of the forward kernels: the grid counts blocks of at least 128 query rows (bf16) or 64
// (fp32) over every head and must stay below 2^31 workgroups; the bf16 kernels bound each K/V tile load by
// a 31-bit byte count, so one launch reads fewer than 2^31 bytes of K (and of V) per head.
int check_launch_limits(int B, int H, int N_q, long long keys_per_launch, int d, int dtype) {
    const long long rows = dtype == ATTN_BF16 ? 128 : 64;
    if ((N_q + rows - 1) / rows * (long long)B * H > 0x7fffffffLL - 8)
        return fail(ATTN_ERR_BAD_SHAPE, "ceil(N_q/%lld)*B*H query blocks exceed 2^31-9", rows);
    if (dtype == ATTN_BF16 && keys_per_launch * d * 2 > 0x7fffffffLL)
        return fail(ATTN_ERR_BAD_SHAPE,
                    "bf16 attention reads at most 2^31-1 bytes of K per head and launch: %lld keys at d = %d "
                    "exceed %lld (the chunked modes apply this per chunk)",
                    keys_per_launch, d, 0x7fffffffLL / (2LL * d));
    return ATTN_OK;
}

int check_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int N_q,
              int N_kv, int d, float scale, long long kv_head_stride, int in_dtype, int out_dtype,
              FwdCheck* out) {
    if (!Q || !K || !V || !O || !LSE) return fail(ATTN_ERR_NULL_PTR, "Q, K, V, O and LSE must be non-NULL");
    if (B < 1 || H < 1 || N_q < 1 || N_kv < 1)
        return fail(ATTN_ERR_BAD_SHAPE, "B, H, N_q, N_kv must be >= 1 (got %d, %d, %d, %d)", B, H, N_q, N_kv);
    if ((long long)B * H > 0x7fffffffLL) return fail(ATTN_ERR_BAD_SHAPE, "B*H exceeds 2^31-1");
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
        return fail(ATTN_ERR_BAD_DTYPE, "unknown dtype (%d, %d)", in_dtype, out_dtype);
    if (out_dtype != ATTN_F32 && out_dtype != in_dtype)
        return fail(ATTN_ERR_BAD_DTYPE, "output dtype must be fp32 or the input dtype");
    if (in_dtype == ATTN_BF16 && d != 64 && d != 128)
        return fail(ATTN_ERR_UNSUPPORTED_D, "bf16 attention supports d = 64 or 128 (got %d)", d);
    if (in_dtype == ATTN_F32 && (d < 1 || d > 256))
        return fail(ATTN_ERR_UNSUPPORTED_D, "fp32 attention supports 1 <= d <= 256 (got %d)", d);
    if (!isfinite(scale)) return fail(ATTN_ERR_BAD_SCALE, "scale must be finite");
    const long long head = (long long)N_kv * d;
    const long long stride = kv_head_stride == 0 ? head : kv_head_stride;
    if (stride < head)
        return fail(ATTN_ERR_BAD_SHAPE, "kv_head_stride %lld is smaller than N_kv*d = %lld", stride, head);
    const long long bh = (long long)B * H;
    if ((__int128)bh * N_q * d * 4 >= kMaxBytes || ((__int128)(bh - 1) * stride + head) * 4 >= kMaxBytes)
        return fail(ATTN_ERR_BAD_SHAPE, "Q, K, V or O would span 2^56 bytes or more");
    const size_t ei = esize((attn_dtype)in_dtype), eo = esize((attn_dtype)out_dtype);
    out->q_bytes = (size_t)(bh * N_q * d) * ei;
    out->kv_bytes = (size_t)((bh - 1) * stride + head) * ei;
    out->o_bytes = (size_t)(bh * N_q * d) * eo;
    out->lse_bytes = (size_t)(bh * N_q) * sizeof(float);
    out->kv_stride = stride;
    if (in_dtype == ATTN_BF16) {
        if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || (stride % 8) != 0)
            return fail(ATTN_ERR_MISALIGNED, "bf16 attention needs 16-byte aligned Q, K, V, O and head strides");
    } else if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O) & 3) {
        return fail(ATTN_ERR_MISALIGNED, "fp32 attention needs 4-byte aligned Q, K, V, O");
    }
    if (((uintptr_t)LSE & 3) != 0) return fail(ATTN_ERR_MISALIGNED, "LSE must be 4-byte aligned");
    const void* ins[3] = {Q, K, V};
    const size_t in_n[3] = {out->q_bytes, out->kv_bytes, out->kv_bytes};
    for (int i = 0; i < 3; ++i) {
        if (overlap(O, out->o_bytes, ins[i], in_n[i]))
            return fail(ATTN_ERR_BAD_ALIAS, "O overlaps an input (Q, K or V)");
        if (overlap(LSE, out->lse_bytes, ins[i], in_n[i]))
            return fail(ATTN_ERR_BAD_ALIAS, "LSE overlaps an input (Q, K or V)");
    }
    if (overlap(O, out->o_bytes, LSE, out->lse_bytes)) return fail(ATTN_ERR_BAD_ALIAS, "O overlaps LSE");
    return ATTN_OK;
}

int clamp_offset(long long off, int N_q, int N_kv) {
    if (off > N_kv) off = N_kv;
    if (off < -(long long)N_q - 1) off = -(long long)N_q - 1;
    return (int)off;
}

int launch_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int N_q,
               int N_kv, int d, int causal, float scale, long long offset, long long kv_stride, int in_dtype,
               int out_dtype, hipStream_t s, const float* o_prev = nullptr, const float* lse_prev = nullptr) {
    attn::FwdArgs a;
    a.q = Q;
    a.k = K;
    a.v = V;
    a.o = O;
    a.lse = LSE;
    a.q_head_stride = (long long)N_q * d;
    a.kv_head_stride = kv_stride;
    a.n_q = N_q;
    a.n_kv = N_kv;
    a.d = d;
    a.bh = B * H;
    a.causal = causal ? 1 : 0;
    a.offset = causal ? clamp_offset(offset, N_q, N_kv) : N_kv;
    a.scale = scale;
    a.o_prev = o_prev;
    a.lse_prev = lse_prev;
    if (in_dtype == ATTN_BF16)
        return run(0, s, "attn_fwd(bf16)", [&] { return attn::launch_fwd_bf16(a, out_dtype == ATTN_F32, s); });
    return run(0, s, "attn_fwd(fp32)", [&] { return attn::launch_fwd_f32(a, s); });
}

int launch_merge(const void* O_a, const float* lse_a, const void* O_b, const float* lse_b, void* O, float* lse,
                 long long rows, int d, int in_dtype, int out_dtype, hipStream_t s) {
    attn::MergeArgs m;
    m.o_a = O_a;
    m.lse_a = lse_a;
    m.o_b = O_b;
    m.lse_b = lse_b;
    m.o = O;
    m.lse = lse;
    m.rows = rows;
    m.d = d;
    m.in_bf16 = in_dtype == ATTN_BF16;
    m.out_bf16 = out_dtype == ATTN_BF16;
    return run(1, s, "attn_merge", [&] { return attn::launch_merge(m, s); });
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

namespace attn {
int device_cus() {
    static std::atomic<int> cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}
}  // namespace attn

extern "C" {

const char* attn_strerror(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL_PTR: return "null pointer";
        case ATTN_ERR_BAD_SHAPE: return "bad shape";
        case ATTN_ERR_UNSUPPORTED_D: return "unsupported head dimension";
        case ATTN_ERR_BAD_DTYPE: return "bad dtype";
        case ATTN_ERR_BAD_SCALE: return "bad scale";
        case ATTN_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case ATTN_ERR_BAD_ALIAS: return "forbidden aliasing";
        case ATTN_ERR_HIP: return "HIP error";
        case ATTN_ERR_MISALIGNED: return "misaligned pointer";
        default: return "unknown status";
    }
}

const char* attn_last_error(void) { return g_last_error.c_str(); }

int attn_fwd_ex(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int N_q, int N_kv,
                int d, int causal, float scale, long long causal_offset, long long kv_head_stride,
                attn_dtype in_dtype, attn_dtype out_dtype, void* hip_stream) {
    g_last_error.clear();
    FwdCheck c;
    int st = check_fwd(Q, K, V, O, LSE, B, H, N_q, N_kv, d, scale, kv_head_stride, in_dtype, out_dtype, &c);
    if (st) return st;
    if ((st = check_launch_limits(B, H, N_q, N_kv, d, in_dtype))) return st;
    return launch_fwd(Q, K, V, O, LSE, B, H, N_q, N_kv, d, causal, scale, causal_offset, c.kv_stride, in_dtype,
                      out_dtype, (hipStream_t)hip_stream);
}

int attn_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int N_q, int N_kv,
             int d, int causal, float scale, attn_dtype dtype, void* hip_stream) {
    return attn_fwd_ex(Q, K, V, O, LSE, B, H, N_q, N_kv, d, causal, scale, (long long)N_kv - N_q, 0, dtype, dtype,
                       hip_stream);
}

int attn_fwd_acc(const void* Q, const void* K, const void* V, const float* O_acc, const float* lse_acc, void* O,
                 float* LSE, int B, int H, int N_q, int N_kv, int d, int causal, float scale, long long causal_offset,
                 long long kv_head_stride, attn_dtype in_dtype, attn_dtype out_dtype, void* hip_stream) {
    g_last_error.clear();
    if (!O_acc || !lse_acc) return fail(ATTN_ERR_NULL_PTR, "O_acc and lse_acc must be non-NULL");
    FwdCheck c;
    int st = check_fwd(Q, K, V, O, LSE, B, H, N_q, N_kv, d, scale, kv_head_stride, in_dtype, out_dtype, &c);
    if (st) return st;
    if ((st = check_launch_limits(B, H, N_q, N_kv, d, in_dtype))) return st;
    const size_t acc_bytes = c.lse_bytes * (size_t)d;   // fp32 [B,H,N_q,d]
    if ((((uintptr_t)O_acc | (uintptr_t)lse_acc) & 3) != 0 || (in_dtype == ATTN_BF16 && !aligned16(O_acc)))
        return fail(ATTN_ERR_MISALIGNED, "O_acc must be 16-byte (bf16 inputs) or 4-byte aligned, lse_acc 4-byte");
    const void* ins[3] = {Q, K, V};
    const size_t in_n[3] = {c.q_bytes, c.kv_bytes, c.kv_bytes};
    for (int i = 0; i < 3; ++i)
        if (overlap(O_acc, acc_bytes, ins[i], in_n[i]) || overlap(lse_acc, c.lse_bytes, ins[i], in_n[i]))
            return fail(ATTN_ERR_BAD_ALIAS, "O_acc or lse_acc overlaps an input (Q, K or V)");
    // O may be exactly O_acc (fp32 output) and LSE exactly lse_acc; any other overlap is forbidden
    if ((const void*)O == (const void*)O_acc) {
        if (out_dtype != ATTN_F32) return fail(ATTN_ERR_BAD_ALIAS, "in-place accumulation needs an fp32 output");
    } else if (overlap(O, c.o_bytes, O_acc, acc_bytes)) {
        return fail(ATTN_ERR_BAD_ALIAS, "O partially overlaps O_acc");
    }
    if (LSE != lse_acc && overlap(LSE, c.lse_bytes, lse_acc, c.lse_bytes))
        return fail(ATTN_ERR_BAD_ALIAS, "LSE partially overlaps lse_acc");
    if (overlap(O, c.o_bytes, lse_acc, c.lse_bytes) || overlap(LSE, c.lse_bytes, O_acc, acc_bytes) ||
        overlap(O_acc, acc_bytes, lse_acc, c.lse_bytes))
        return fail(ATTN_ERR_BAD_ALIAS, "an output array overlaps the other partial array");
    return launch_fwd(Q, K, V, O, LSE, B, H, N_q, N_kv, d, causal, scale, causal_offset, c.kv_stride, in_dtype,
                      out_dtype, (hipStream_t)hip_stream, O_acc, lse_acc);
}

int attn_merge(const void* O_a, const float* lse_a, const void* O_b, const float* lse_b, void* O, float* lse,
               long long rows, int d, attn_dtype in_dtype, attn_dtype out_dtype, void* hip_stream) {
    g_last_error.clear();
    if (!O_a || !lse_a || !O_b || !lse_b || !O || !lse) return fail(ATTN_ERR_NULL_PTR, "merge pointers must be non-NULL");
    if (rows < 1 || d < 1) return fail(ATTN_ERR_BAD_SHAPE, "rows and d must be >= 1 (got %lld, %d)", rows, d);
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return fail(ATTN_ERR_BAD_DTYPE, "unknown dtype");
    if (rows > (1LL << 40) / d) return fail(ATTN_ERR_BAD_SHAPE, "rows*d too large");
    const size_t in_b = (size_t)rows * d * esize(in_dtype), out_b = (size_t)rows * d * esize(out_dtype);
    const size_t lse_b_n = (size_t)rows * sizeof(float);
    if ((((uintptr_t)O_a | (uintptr_t)O_b | (uintptr_t)O) & (esize(in_dtype) - 1)) ||
        ((uintptr_t)O & (esize(out_dtype) - 1)) || (((uintptr_t)lse_a | (uintptr_t)lse_b | (uintptr_t)lse) & 3))
        return fail(ATTN_ERR_MISALIGNED, "merge buffers must be aligned to their element size");
    // O may be exactly O_a or O_b (same dtype); any other overlap with an input is forbidden
    const bool same_t = in_dtype == out_dtype;
    for (const void* src : {O_a, O_b}) {
        if (O == src) {
            if (!same_t) return fail(ATTN_ERR_BAD_ALIAS, "in-place merge needs equal input and output dtypes");
        } else if (overlap(O, out_b, src, in_b)) {
            return fail(ATTN_ERR_BAD_ALIAS, "O partially overlaps O_a or O_b");
        }
    }
    for (const float* src : {lse_a, lse_b})
        if (lse != src && overlap(lse, lse_b_n, src, lse_b_n))
            return fail(ATTN_ERR_BAD_ALIAS, "lse partially overlaps lse_a or lse_b");
    for (const void* p : {(const void*)lse_a, (const void*)lse_b, (const void*)lse})
        if (overlap(O, out_b, p, lse_b_n)) return fail(ATTN_ERR_BAD_ALIAS, "O overlaps an lse array");
    for (const void* p : {O_a, O_b})
        if (overlap(lse, lse_b_n, p, in_b)) return fail(ATTN_ERR_BAD_ALIAS, "lse overlaps O_a or O_b");
    return launch_merge(O_a, lse_a, O_b, lse_b, O, lse, rows, d, in_dtype, out_dtype, (hipStream_t)hip_stream);
}

size_t attn_fwd_chunked_workspace_bytes(int B, int H, int N_q, int d, int P) {
    if (B < 1 || H < 1 || N_q < 1 || d < 1 || P < 1) return 0;
    if (P == 1) return 0;
    if ((__int128)B * H * N_q * d * 4 >= kMaxBytes) return 0;
    const size_t rows = (size_t)B * H * N_q;
    return align256(rows * d * sizeof(float)) + align256(rows * sizeof(float));
}

}  // extern "C"

namespace {

// Argument checks of the chunked mode that need no workspace; on success *c describes the arrays.
int check_chunked(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int N_q, int N_kv,
                  int d, float scale, int P, attn_dtype dtype, FwdCheck* c) {
    int st = check_fwd(Q, K, V, O, LSE, B, H, N_q, N_kv, d, scale, 0, dtype, dtype, c);
    if (st) return st;
    if (P < 1) return fail(ATTN_ERR_BAD_SHAPE, "P must be >= 1 (got %d)", P);
    return check_launch_limits(B, H, N_q, ((long long)N_kv + P - 1) / P, d, dtype);
}

// The chunked fold of attn_fwd_chunked after check_chunked, with a workspace of at least
// attn_fwd_chunked_workspace_bytes (unused when P == 1).
int run_chunked(const FwdCheck& c, const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                int N_q, int N_kv, int d, int causal, float scale, int P, attn_dtype dtype, void* workspace,
                size_t workspace_bytes, hipStream_t s) {
    int st = ATTN_OK;
    const long long offset = (long long)N_kv - N_q;
    if (P == 1)
        return launch_fwd(Q, K, V, O, LSE, B, H, N_q, N_kv, d, causal, scale, offset, c.kv_stride, dtype, dtype, s);

    const size_t need = attn_fwd_chunked_workspace_bytes(B, H, N_q, d, P);
    if (!workspace || workspace_bytes < need)
        return fail(ATTN_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
    if (((uintptr_t)workspace & 255) != 0) return fail(ATTN_ERR_MISALIGNED, "workspace must be 256-byte aligned");
    const void* others[5] = {Q, K, V, O, LSE};
    const size_t other_n[5] = {c.q_bytes, c.kv_bytes, c.kv_bytes, c.o_bytes, c.lse_bytes};
    for (int i = 0; i < 5; ++i)
        if (overlap(workspace, need, others[i], other_n[i]))
            return fail(ATTN_ERR_BAD_ALIAS, "workspace overlaps Q, K, V, O or LSE");

    // chunk p covers keys [floor(p*N_kv/P), floor((p+1)*N_kv/P)); empty or wholly-future chunks are skipped.
    // The live chunks are found by a scan, not stored, so that the call allocates no host memory either.
    auto is_live = [&](int p) {
        const long long lo = (long long)p * N_kv / P, hi = (long long)(p + 1) * N_kv / P;
        return hi != lo && !(causal && (long long)N_q - 1 + offset - lo < 0);
    };
    int first = -1, last = -1;
    for (int p = 0; p < P; ++p)
        if (is_live(p)) {
            if (first < 0) first = p;
            last = p;
        }
    if (first < 0) first = last = 0;   // unreachable with offset N_kv - N_q; kept for safety
    const size_t rows = (size_t)B * H * N_q;
    char* ws = static_cast<char*>(workspace);
    float* o_acc = reinterpret_cast<float*>(ws);
    float* lse_acc = reinterpret_cast<float*>(ws + align256(rows * d * sizeof(float)));
    const size_t es = esize(dtype);
    // chunk p into (o, lse); every chunk after the first live one folds into the running partial in its
    // own epilogue (in place in the workspace, or into O and LSE for the last one)
    auto chunk = [&](int p, void* o, float* lse, attn_dtype out_t, const float* prev_o, const float* prev_lse) {
        const long long lo = (long long)p * N_kv / P, hi = (long long)(p + 1) * N_kv / P;
        const char* kp = static_cast<const char*>(K) + lo * d * es;
        const char* vp = static_cast<const char*>(V) + lo * d * es;
        return launch_fwd(Q, kp, vp, o, lse, B, H, N_q, (int)(hi - lo), d, causal, scale, offset - lo, c.kv_stride,
                          dtype, out_t, s, prev_o, prev_lse);
    };
    if (first == last) return chunk(first, O, LSE, dtype, nullptr, nullptr);
    if ((st = chunk(first, o_acc, lse_acc, ATTN_F32, nullptr, nullptr))) return st;
    for (int p = first + 1; p <= last; ++p) {
        if (!is_live(p)) continue;
        st = p == last ? chunk(p, O, LSE, dtype, o_acc, lse_acc)
                       : chunk(p, o_acc, lse_acc, ATTN_F32, o_acc, lse_acc);
        if (st) return st;
    }
    return ATTN_OK;
}

// ------------------------------------------------------------- fixed scratch of attn_fwd_chunked_noalloc
// The running fp32 partial of attn_fwd_chunked_noalloc lives in `scratch`, one copy per device, which the HIP
// runtime allocates when this file's device code is loaded on that device and holds until the process ends.
// In host code the name `scratch` is a host-side placeholder, not a device address: the device address is
// looked up once per device with hipGetSymbolAddress (with that device current), kept in g_scratch_ptr, and
// only that address is handed to kernels.  Nothing in the fold needs the array cleared: the first live
// chunk writes every row of the partial before any later chunk reads it.
std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};   // per device; written once, under g_scratch_mu

}  // namespace

static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

// This device's copy of `scratch` (the calling thread's current device), or nullptr with *err set.
void* scratch_address(hipError_t* err) {
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= 64) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        if (ptr == nullptr) {
            *err = hipErrorInvalidSymbol;
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int attn_fwd_chunked_noalloc(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int N_q,
                             int N_kv, int d, int causal, float scale, int P, attn_dtype dtype, void* hip_stream) {
    g_last_error.clear();
    FwdCheck c;
    if (int st = check_chunked(Q, K, V, O, LSE, B, H, N_q, N_kv, d, scale, P, dtype, &c)) return st;
    const size_t need = attn_fwd_chunked_workspace_bytes(B, H, N_q, d, P);
    if (need > ATTN_NOALLOC_SCRATCH_BYTES)
        return fail(ATTN_ERR_WORKSPACE_TOO_SMALL,
                    "attn_fwd_chunked_noalloc: the running partial needs %zu bytes, more than its fixed scratch of %zu "
                    "bytes (B*H*N_q*(d+1)*4 must fit); use attn_fwd_chunked with a workspace",
                    need, (size_t)ATTN_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if (need > 0) {
        hipError_t e = hipSuccess;
        ws = scratch_address(&e);
        if (!ws) return fail(ATTN_ERR_HIP, "attn_fwd_chunked_noalloc: hipGetSymbolAddress failed: %s", hipGetErrorString(e));
    }
    return run_chunked(c, Q, K, V, O, LSE, B, H, N_q, N_kv, d, causal, scale, P, dtype, ws,
                       (size_t)ATTN_NOALLOC_SCRATCH_BYTES, (hipStream_t)hip_stream);
}

int attn_fwd_chunked(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int N_q,
                     int N_kv, int d, int causal, float scale, int P, attn_dtype dtype, void* workspace,
                     size_t workspace_bytes, void* hip_stream) {
    g_last_error.clear();
    FwdCheck c;
    if (int st = check_chunked(Q, K, V, O, LSE, B, H, N_q, N_kv, d, scale, P, dtype, &c)) return st;
    return run_chunked(c, Q, K, V, O, LSE, B, H, N_q, N_kv, d, causal, scale, P, dtype, workspace, workspace_bytes,
                       (hipStream_t)hip_stream);
}

size_t attn_fwd_streamed_workspace_bytes(int B, int H, int N_q, int N_kv, int d, int P, attn_dtype dtype) {
    if (B < 1 || H < 1 || N_q < 1 || N_kv < 1 || d < 1 || P < 1 || !valid_dtype(dtype)) return 0;
    if ((__int128)B * H * N_q * d * 4 >= kMaxBytes || (__int128)B * H * N_kv * d * 4 >= kMaxBytes) return 0;
    const size_t rows = (size_t)B * H * N_q;
    const size_t cmax = ((size_t)N_kv + P - 1) / P;   // the longest chunk
    const size_t slot = (size_t)B * H * cmax * d * esize(dtype);
    return align256(rows * d * sizeof(float)) + align256(rows * sizeof(float)) + 4 * align256(slot);
}

int attn_fwd_streamed(const void* Q, const void* K_host, const void* V_host, void* O, float* LSE, int B, int H,
                      int N_q, int N_kv, int d, int causal, float scale, int P, attn_dtype dtype, void* workspace,
                      size_t workspace_bytes, void* hip_stream, void* copy_stream) {
    g_last_error.clear();
    FwdCheck c;
    int st = check_fwd(Q, K_host, V_host, O, LSE, B, H, N_q, N_kv, d, scale, 0, dtype, dtype, &c);
    if (st) return st;
    if (P < 1) return fail(ATTN_ERR_BAD_SHAPE, "P must be >= 1 (got %d)", P);
    if ((st = check_launch_limits(B, H, N_q, ((long long)N_kv + P - 1) / P, d, dtype))) return st;
    if (hip_stream == copy_stream) return fail(ATTN_ERR_BAD_ALIAS, "the copy stream must differ from the compute stream");
    const size_t need = attn_fwd_streamed_workspace_bytes(B, H, N_q, N_kv, d, P, dtype);
    if (!workspace || workspace_bytes < need)
        return fail(ATTN_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
    if (((uintptr_t)workspace & 255) != 0) return fail(ATTN_ERR_MISALIGNED, "workspace must be 256-byte aligned");
    const void* others[5] = {Q, K_host, V_host, O, LSE};
    const size_t other_n[5] = {c.q_bytes, c.kv_bytes, c.kv_bytes, c.o_bytes, c.lse_bytes};
    for (int i = 0; i < 5; ++i)
        if (overlap(workspace, need, others[i], other_n[i]))
            return fail(ATTN_ERR_BAD_ALIAS, "workspace overlaps Q, K, V, O or LSE");

    hipStream_t s = (hipStream_t)hip_stream, cs = (hipStream_t)copy_stream;
    const long long offset = (long long)N_kv - N_q;
    // the chunks of attn_fwd_chunked with the same P, in the same order
    std::vector<int> live;
    for (int p = 0; p < P; ++p) {
        const long long lo = (long long)p * N_kv / P, hi = (long long)(p + 1) * N_kv / P;
        if (hi == lo) continue;
        if (causal && (long long)N_q - 1 + offset - lo < 0) continue;
        live.push_back(p);
    }
    if (live.empty()) live.push_back(0);
    const size_t rows = (size_t)B * H * N_q, es = esize(dtype);
    const size_t cmax = ((size_t)N_kv + P - 1) / P, slot = align256((size_t)B * H * cmax * d * es);
    char* ws = static_cast<char*>(workspace);
    float* o_acc = reinterpret_cast<float*>(ws);
    float* lse_acc = reinterpret_cast<float*>(ws + align256(rows * d * sizeof(float)));
    char* slots = ws + align256(rows * d * sizeof(float)) + align256(rows * sizeof(float));
    char* kslot[2] = {slots, slots + 2 * slot};
    char* vslot[2] = {slots + slot, slots + 3 * slot};

    // copied[b]: slot b holds its chunk; done[b]: the kernel reading slot b has finished; entry: everything
    // enqueued on the compute stream before this call (an earlier call's kernels may still read the staging
    // slots, and memory handed back to the caller's allocator may still be in use there)
    EventQuad* ev = take_quad();
    if (!ev) return fail(ATTN_ERR_HIP, "attn_fwd_streamed: hipEventCreate failed");
    hipEvent_t* copied = ev->e;
    hipEvent_t* done = ev->e + 2;
    hipEvent_t entry = ev->e[4];
    const size_t n = live.size();
    auto bounds = [&](size_t i, long long& lo, long long& hi) {
        lo = (long long)live[i] * N_kv / P;
        hi = (long long)(live[i] + 1) * N_kv / P;
    };
    // chunk i into slot i % 2: the first two once the compute stream's earlier work is done, later ones once
    // the kernel of chunk i-2 is done with the slot
    auto copy = [&](size_t i) -> int {
        const int b = (int)(i & 1);
        long long lo, hi;
        bounds(i, lo, hi);
        const size_t row = (size_t)(hi - lo) * d * es, pitch = (size_t)N_kv * d * es;
        if (hipStreamWaitEvent(cs, i >= 2 ? done[b] : entry, 0) != hipSuccess)
            return fail(ATTN_ERR_HIP, "attn_fwd_streamed: hipStreamWaitEvent failed");
        return run(2, cs, "attn_fwd_streamed copy", [&] {
            hipError_t e = hipMemcpy2DAsync(kslot[b], row, static_cast<const char*>(K_host) + lo * d * es, pitch, row,
                                            (size_t)B * H, hipMemcpyDefault, cs);
            if (e == hipSuccess)
                e = hipMemcpy2DAsync(vslot[b], row, static_cast<const char*>(V_host) + lo * d * es, pitch, row,
                                     (size_t)B * H, hipMemcpyDefault, cs);
            if (e == hipSuccess) e = hipEventRecord(copied[b], cs);
            return e;
        });
    };
    // chunk i from slot i % 2 (rows packed: head stride = chunk length * d), folded as in attn_fwd_chunked
    auto compute = [&](size_t i) -> int {
        const int b = (int)(i & 1);
        long long lo, hi;
        bounds(i, lo, hi);
        if (hipStreamWaitEvent(s, copied[b], 0) != hipSuccess)
            return fail(ATTN_ERR_HIP, "attn_fwd_streamed: hipStreamWaitEvent failed");
        const int len = (int)(hi - lo);
        const bool first = i == 0, last = i + 1 == n;
        void* o = last ? O : (void*)o_acc;
        float* l = last ? LSE : lse_acc;
        const attn_dtype ot = last ? dtype : ATTN_F32;
        int r = launch_fwd(Q, kslot[b], vslot[b], o, l, B, H, N_q, len, d, causal, scale, offset - lo,
                           (long long)len * d, dtype, ot, s, first ? nullptr : o_acc, first ? nullptr : lse_acc);
        if (r) return r;
        if (hipEventRecord(done[b], s) != hipSuccess) return fail(ATTN_ERR_HIP, "attn_fwd_streamed: hipEventRecord failed");
        return ATTN_OK;
    };
    if (hipEventRecord(entry, s) != hipSuccess) {
        give_quad(ev, nullptr);   // nothing waits on the set yet
        return fail(ATTN_ERR_HIP, "attn_fwd_streamed: hipEventRecord failed");
    }
    st = copy(0);
    if (!st && n > 1) st = copy(1);
    for (size_t i = 0; i < n && !st; ++i) {
        st = compute(i);
        if (!st && i + 2 < n) st = copy(i + 2);
    }
    // Compute n-1 waits for the last copy and follows every earlier compute on its stream, so its "done"
    // event completes after every use of the set.  After a failure some copy may have no compute waiting
    // for it; that set is never handed out again.
    if (!st) give_quad(ev, done[(n - 1) & 1]);
    return st;
}

size_t attn_ffn_workspace_bytes(long long M, int d_ff, long long block) {
    if (M < 1 || d_ff < 1 || block < 1) return 0;
    if ((__int128)(block < M ? block : M) * d_ff * 2 >= kMaxBytes) return 0;
    return align256((size_t)(block < M ? block : M) * d_ff * 2);
}

int attn_ffn_blockwise(const void* X, const void* W1, const float* b1, const void* W2, const float* b2, void* Y,
                       long long M, int d_model, int d_ff, long long block, attn_act act, void* workspace,
                       size_t workspace_bytes, void* hip_stream) {
    g_last_error.clear();
    if (!X || !W1 || !W2 || !Y) return fail(ATTN_ERR_NULL_PTR, "X, W1, W2 and Y must be non-NULL");
    if (M < 1 || block < 1) return fail(ATTN_ERR_BAD_SHAPE, "M and block must be >= 1 (got %lld, %lld)", M, block);
    if (d_model < 64 || d_ff < 64 || d_model % 64 || d_ff % 64)
        return fail(ATTN_ERR_UNSUPPORTED_D, "d_model and d_ff must be positive multiples of 64 (got %d, %d)",
                    d_model, d_ff);
    if (act != ATTN_ACT_NONE && act != ATTN_ACT_RELU && act != ATTN_ACT_GELU)
        return fail(ATTN_ERR_BAD_DTYPE, "unknown activation %d", (int)act);
    if (M > (1LL << 40) / d_model) return fail(ATTN_ERR_BAD_SHAPE, "M*d_model too large");
    const long long rows = block < M ? block : M;   // at most 2^34 after the bound on M
    const long long lim = 0x7fffffffLL;
    if (rows * d_ff * 2 > lim || rows * d_model * 2 > lim || (long long)d_ff * d_model * 2 > lim)
        return fail(ATTN_ERR_BAD_SHAPE,
                    "a row block (%lld x %d), its hidden block (%lld x %d) and each weight (%d x %d) must stay "
                    "below 2^31 bytes",
                    rows, d_model, rows, d_ff, d_ff, d_model);
    if (!aligned16(X) || !aligned16(W1) || !aligned16(W2) || !aligned16(Y) || !aligned16(b1) || !aligned16(b2))
        return fail(ATTN_ERR_MISALIGNED, "X, W1, W2, Y, b1 and b2 need 16-byte alignment");
    const size_t need = attn_ffn_workspace_bytes(M, d_ff, block);
    if (!workspace || workspace_bytes < need)
        return fail(ATTN_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
    if (!aligned16(workspace)) return fail(ATTN_ERR_MISALIGNED, "workspace must be 16-byte aligned");
    const size_t xy = (size_t)M * d_model * 2, w = (size_t)d_ff * d_model * 2;
    const void* ins[5] = {X, W1, W2, b1, b2};
    const size_t in_n[5] = {xy, w, w, b1 ? (size_t)d_ff * 4 : 0, b2 ? (size_t)d_model * 4 : 0};
    for (int i = 0; i < 5; ++i) {
        if (overlap(Y, xy, ins[i], in_n[i])) return fail(ATTN_ERR_BAD_ALIAS, "Y overlaps an input");
        if (overlap(workspace, need, ins[i], in_n[i])) return fail(ATTN_ERR_BAD_ALIAS, "workspace overlaps an input");
    }
    if (overlap(workspace, need, Y, xy)) return fail(ATTN_ERR_BAD_ALIAS, "workspace overlaps Y");

    hipStream_t s = (hipStream_t)hip_stream;
    for (long long r0 = 0; r0 < M; r0 += rows) {
        const int n_rows = (int)(M - r0 < rows ? M - r0 : rows);
        attn::GemmArgs g1{static_cast<const char*>(X) + (size_t)r0 * d_model * 2, W1, b1, workspace, n_rows, d_ff,
                          d_model, (int)act};
        attn::GemmArgs g2{workspace, W2, b2, static_cast<char*>(Y) + (size_t)r0 * d_model * 2, n_rows, d_model,
                          d_ff, ATTN_ACT_NONE};
        if (int st = run(3, s, "attn_ffn_blockwise (W1)", [&] { return attn::launch_gemm_nt(g1, s); })) return st;
        if (int st = run(3, s, "attn_ffn_blockwise (W2)", [&] { return attn::launch_gemm_nt(g2, s); })) return st;
    }
    return ATTN_OK;
}

int attn_timing_enable(int on) {
    std::lock_guard<std::mutex> g(g_timing_mu);
    g_timing_on = on != 0;
    return ATTN_OK;
}

int attn_timing_read(long long counts[4], double total_ms[4]) {
    std::vector<Timed> recs;
    {
        std::lock_guard<std::mutex> g(g_timing_mu);
        recs.swap(g_timed);
    }
    for (int k = 0; k < kTimingKinds; ++k) {
        counts[k] = 0;
        total_ms[k] = 0.0;
    }
    int st = ATTN_OK;
    for (const Timed& r : recs) {
        float ms = 0.f;
        if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) {
            st = fail(ATTN_ERR_HIP, "attn_timing_read: event query failed");
        } else if (r.kind >= 0 && r.kind < kTimingKinds) {
            counts[r.kind] += 1;
            total_ms[r.kind] += ms;
        }
    }
    std::lock_guard<std::mutex> g(g_timing_mu);
    for (const Timed& r : recs) {
        g_event_pool.push_back(r.start);
        g_event_pool.push_back(r.stop);
    }
    return st;
}

}  // extern "C"
