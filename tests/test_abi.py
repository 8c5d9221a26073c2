"""The C-ABI library on a host without a GPU: it loads, exports what include/attn.h declares, and rejects
invalid arguments with the documented status before any HIP call (no call here reaches a kernel)."""
import ctypes
import math
import os
import re

import pytest

import exact_blockwise_attention_fwd_amd as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

# distinct, 256-byte aligned fake device addresses: never dereferenced, because validation fails first
P = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(8)]


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = A.lib()
    names = declared_functions()
    assert {"attn_fwd", "attn_fwd_ex", "attn_fwd_acc", "attn_merge", "attn_fwd_chunked",
            "attn_fwd_chunked_workspace_bytes", "attn_fwd_streamed", "attn_fwd_streamed_workspace_bytes",
            "attn_strerror", "attn_last_error",
            "attn_ffn_blockwise", "attn_ffn_workspace_bytes", "attn_timing_enable", "attn_timing_read"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in attn.h but not exported"


def test_status_codes_match_header():
    text = open(HEADER).read()
    codes = dict((name, int(v)) for name, v in re.findall(r"(ATTN_(?:OK|ERR_[A-Z_]+))\s*=\s*(\d+)", text))
    assert codes == {v: k for k, v in A.STATUS.items()}
    for name, code in codes.items():
        s = A.lib().attn_strerror(code).decode()
        assert s and s != "unknown status", name
    assert A.lib().attn_strerror(99).decode() == "unknown status"


def fwd(*, q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=1, H=2, N_q=8, N_kv=8, d=64, causal=0, scale=0.125,
        dtype=A.ATTN_BF16):
    return A.lib().attn_fwd(q, k, v, o, lse, B, H, N_q, N_kv, d, causal, scale, dtype, None)


def fwd_ex(*, q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=1, H=2, N_q=8, N_kv=8, d=64, causal=0, scale=0.125,
           offset=0, stride=0, din=A.ATTN_BF16, dout=A.ATTN_BF16):
    return A.lib().attn_fwd_ex(q, k, v, o, lse, B, H, N_q, N_kv, d, causal, scale, offset, stride, din, dout, None)


def merge(*, oa=P[0], la=P[1], ob=P[2], lb=P[3], o=P[4], lse=P[5], rows=16, d=64, din=A.ATTN_F32, dout=A.ATTN_F32):
    return A.lib().attn_merge(oa, la, ob, lb, o, lse, rows, d, din, dout, None)


def fwd_acc(*, q=P[0], k=P[1], v=P[2], oa=P[5], la=P[6], o=P[3], lse=P[4], B=1, H=2, N_q=8, N_kv=8, d=64,
            din=A.ATTN_BF16, dout=A.ATTN_BF16):
    return A.lib().attn_fwd_acc(q, k, v, oa, la, o, lse, B, H, N_q, N_kv, d, 0, 0.125, 0, 0, din, dout, None)


def chunked(*, o=P[3], lse=P[4], P_=4, ws=P[6], ws_n=1 << 40, d=64, dtype=A.ATTN_BF16, N_q=8, N_kv=8):
    return A.lib().attn_fwd_chunked(P[0], P[1], P[2], o, lse, 1, 2, N_q, N_kv, d, 0, 0.125, P_, dtype, ws, ws_n, None)


def streamed(*, o=P[3], lse=P[4], P_=4, ws=P[6], ws_n=1 << 40, s1=P[0], s2=P[1], d=64, N_kv=8):
    # the stream handles are never used: every case here fails validation first
    return A.lib().attn_fwd_streamed(P[0], P[1], P[2], o, lse, 1, 2, 8, N_kv, d, 0, 0.125, P_, A.ATTN_BF16, ws, ws_n,
                                     s1, s2)


def last_error():
    return A.lib().attn_last_error().decode()


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse"])
def test_null_pointers(which):
    assert fwd(**{which: None}) == 1 and "non-NULL" in last_error()
    assert fwd_ex(**{which: None}) == 1


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N_q=0), dict(N_kv=0), dict(N_q=-3), dict(B=-1)])
def test_bad_shapes(kw):
    assert fwd(**kw) == 2


def test_bad_kv_stride():
    assert fwd_ex(stride=8 * 64 - 1) == 2      # smaller than N_kv*d


@pytest.mark.parametrize("d,dtype", [(32, A.ATTN_BF16), (96, A.ATTN_BF16), (256, A.ATTN_BF16), (0, A.ATTN_F32),
                                     (257, A.ATTN_F32)])
def test_unsupported_head_dim(d, dtype):
    assert fwd(d=d, dtype=dtype) == 3


def test_bad_dtypes():
    assert fwd(dtype=7) == 4
    assert fwd_ex(din=A.ATTN_F32, dout=A.ATTN_BF16) == 4     # fp32 input cannot produce bf16 output
    assert merge(din=3) == 4


@pytest.mark.parametrize("scale", [math.nan, math.inf, -math.inf])
def test_bad_scale(scale):
    assert fwd(scale=scale) == 5


def test_aliasing():
    assert fwd(o=P[0]) == 7                     # O on top of Q
    assert fwd(lse=P[2]) == 7                   # LSE on top of V
    assert fwd(lse=P[3]) == 7                   # LSE on top of O
    assert fwd(o=ctypes.c_void_p(P[1].value + 256)) == 7   # O inside K


def test_misaligned():
    assert fwd(q=ctypes.c_void_p(P[0].value + 8)) == 9      # bf16 needs 16-byte alignment
    assert fwd(q=ctypes.c_void_p(P[0].value + 2), dtype=A.ATTN_F32) == 9
    assert fwd_ex(stride=8 * 64 + 4) == 9       # bf16 head stride must keep 16-byte alignment


def test_launch_limits():
    """Sizes past the kernels' launch limits are refused as shapes before any HIP call: bf16 K of one head
    and launch below 2^31 bytes (per chunk in the chunked modes), and fewer than 2^31-8 query blocks."""
    far = [ctypes.c_void_p((1 << 47) * (i + 1)) for i in range(8)]   # 128 TiB apart: no overlaps
    kw = dict(q=far[0], k=far[1], v=far[2], o=far[3], lse=far[4])
    assert fwd(**kw, B=1, H=1, N_q=64, N_kv=8388608, d=128) == 2
    assert "8388607" in last_error()
    assert fwd(**kw, B=1, H=1, N_q=64, N_kv=16777216, d=64) == 2
    assert "16777215" in last_error()
    assert fwd_ex(**kw, B=1, H=1, N_q=64, N_kv=8388608, d=128) == 2
    lib = A.lib()
    # chunked: 2 chunks of 8,388,608 keys are too long, the same keys in 3 chunks would not be
    assert lib.attn_fwd_chunked(far[0], far[1], far[2], far[3], far[4], 1, 1, 64, 2 * 8388608, 128, 1, 0.1, 2,
                                A.ATTN_BF16, far[5], 1 << 40, None) == 2
    assert "per chunk" in last_error()
    assert lib.attn_fwd_streamed(far[0], far[1], far[2], far[3], far[4], 1, 1, 64, 2 * 8388608, 128, 1, 0.1, 2,
                                 A.ATTN_BF16, far[5], 1 << 40, far[6], far[7]) == 2
    # query blocks: ceil(8192/128) * 32768 * 1024 = 2^31 workgroups
    assert fwd(**kw, B=32768, H=1024, N_q=8192, N_kv=1, d=64) == 2
    assert "query blocks" in last_error()
    assert fwd(**kw, B=32768, H=1024, N_q=4096, N_kv=1, d=64, dtype=A.ATTN_F32) == 2


def test_sizes_that_would_wrap():
    """Shapes whose byte counts exceed 2^56 are refused (or give a zero workspace size) instead of wrapping
    around 2^64 into a small size that a too-small workspace or an overlapping buffer would then pass."""
    far = [ctypes.c_void_p((1 << 47) * (i + 1)) for i in range(8)]
    kw = dict(q=far[0], k=far[1], v=far[2], o=far[3], lse=far[4])
    assert fwd(**kw, B=1, H=1 << 30, N_q=1 << 30, N_kv=1, d=64) == 2
    assert "2^56" in last_error()
    assert fwd_ex(**kw, B=1, H=4, N_q=8, N_kv=8, d=64, stride=1 << 62) == 2   # K/V extent via the head stride
    assert "2^56" in last_error()
    lib = A.lib()
    # B*H*N_q*d*4 = 2^70: the formula would wrap to 2^62; the size query reports it as invalid
    assert lib.attn_fwd_chunked_workspace_bytes(1, 1 << 30, 1 << 30, 256, 2) == 0
    assert lib.attn_fwd_chunked(far[0], far[1], far[2], far[3], far[4], 1, 1 << 30, 1 << 30, 8, 256, 0, 0.1, 2,
                                A.ATTN_F32, far[5], 1 << 40, None) == 2
    assert lib.attn_fwd_streamed_workspace_bytes(1, 1 << 30, 8, 1 << 30, 64, 2, A.ATTN_BF16) == 0
    assert lib.attn_ffn_workspace_bytes(1 << 62, 16384, 1 << 62) == 0
    assert ffn(x=far[0], w1=far[1], w2=far[2], y=far[3], ws=far[4], M=1 << 62, block=1 << 62) == 2
    assert "too large" in last_error()


def test_merge_validation():
    assert merge(oa=None) == 1
    assert merge(rows=0) == 2 and merge(d=0) == 2
    assert merge(o=ctypes.c_void_p(P[0].value + 64)) == 7            # partial overlap with O_a
    assert merge(o=P[0], din=A.ATTN_F32, dout=A.ATTN_BF16) == 7      # in place across dtypes
    assert merge(lse=ctypes.c_void_p(P[1].value + 4)) == 7           # lse partially overlaps lse_a
    assert merge(o=P[1]) == 7                                         # O over lse_a


def test_chunked_validation():
    need = A.lib().attn_fwd_chunked_workspace_bytes(1, 2, 8, 64, 4)
    assert chunked(P_=0) == 2
    assert chunked(ws=None) == 6
    assert chunked(ws_n=need - 1) == 6
    assert chunked(ws=ctypes.c_void_p(P[6].value + 16)) == 9
    assert chunked(ws=P[1]) == 7                                      # workspace over K
    assert chunked(d=100) == 3


def test_workspace_formula():
    f = A.lib().attn_fwd_chunked_workspace_bytes
    assert f(1, 2, 8, 64, 1) == 0
    rows = 1 * 32 * 16384
    a256 = lambda x: (x + 255) // 256 * 256
    assert f(1, 32, 16384, 128, 8) == a256(rows * 128 * 4) + a256(rows * 4)
    assert f(1, 1, 3, 5, 2) == 256 + 256
    assert f(0, 1, 1, 64, 2) == 0 and f(1, 1, 1, 64, 0) == 0


def test_streamed_workspace_formula():
    f = A.lib().attn_fwd_streamed_workspace_bytes
    a256 = lambda x: (x + 255) // 256 * 256
    rows = 1 * 32 * 16384
    slot = 1 * 32 * 16384 * 128 * 2                     # 131072 keys in 8 chunks of 16384, bf16
    assert f(1, 32, 16384, 131072, 128, 8, A.ATTN_BF16) == a256(rows * 512) + a256(rows * 4) + 4 * a256(slot)
    # ragged chunks: the slots hold the longest one, ceil(10 / 3) = 4 keys
    assert f(1, 1, 3, 10, 5, 3, A.ATTN_F32) == 256 + 256 + 4 * a256(1 * 4 * 5 * 4)
    assert f(1, 1, 3, 10, 5, 0, A.ATTN_F32) == 0 and f(1, 1, 3, 10, 5, 2, 7) == 0


def test_streamed_validation():
    need = A.lib().attn_fwd_streamed_workspace_bytes(1, 2, 8, 8, 64, 4, A.ATTN_BF16)
    assert streamed(P_=0) == 2
    assert streamed(s1=None, s2=None) == 7                          # the default stream twice
    assert streamed(s2=P[0]) == 7                                    # the same stream twice
    assert streamed(ws=None) == 6
    assert streamed(ws_n=need - 1) == 6
    assert streamed(ws=ctypes.c_void_p(P[6].value + 16)) == 9
    assert streamed(ws=P[3]) == 7                                     # workspace over O
    assert streamed(d=100) == 3
    assert "workspace" in last_error() or "d = 64" in last_error()


def test_chunked_noalloc_validation():
    """The allocation-free chunked entry point validates like attn_fwd_chunked and refuses, before any HIP call,
    a running partial larger than its fixed scratch (ATTN_NOALLOC_SCRATCH_BYTES = 64 MiB)."""
    lib = A.lib()

    far = [ctypes.c_void_p((1 << 44) * (i + 1)) for i in range(5)]   # 16 TiB apart: no overlaps

    def call(B=1, H=2, N_q=8, N_kv=8, d=64, P_=4, q=far[0], o=far[3], lse=far[4]):
        return lib.attn_fwd_chunked_noalloc(q, far[1], far[2], o, lse, B, H, N_q, N_kv, d, 0, 0.125, P_, A.ATTN_BF16,
                                            None)

    assert A.NOALLOC_SCRATCH_BYTES == 64 << 20
    header = open(HEADER).read()
    assert "#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in header
    assert call(q=None) == 1
    assert call(P_=0) == 2
    assert call(d=100) == 3
    # at d = 128, 130,055 rows fit in 64 MiB (rows * 129 * 4 bytes, 256-byte aligned pieces) and 130,056 do not
    ws = lambda rows: lib.attn_fwd_chunked_workspace_bytes(1, 1, rows, 128, 2)
    assert ws(130055) <= A.NOALLOC_SCRATCH_BYTES < ws(130056)
    assert call(B=1, H=1, N_q=130056, N_kv=64, d=128, P_=2) == 6
    assert "fixed scratch" in last_error()
    # at d = 64 the limit is 258,111 rows
    ws64 = lambda rows: lib.attn_fwd_chunked_workspace_bytes(1, 1, rows, 64, 3)
    assert ws64(258111) <= A.NOALLOC_SCRATCH_BYTES < ws64(258112)
    assert call(B=1, H=1, N_q=258112, N_kv=64, d=64, P_=3) == 6


def test_timing_read_writes_exactly_four_entries():
    """attn_timing_read fills arrays of 4 (one entry per kind of timed work) and nothing past them: sentinels
    placed right after each array survive (works without a GPU: no launch has been recorded)."""
    counts = (ctypes.c_longlong * 8)(*([7] * 8))
    ms = (ctypes.c_double * 8)(*([7.5] * 8))
    lib = A.lib()
    assert lib.attn_timing_read(counts, ms) == 0
    assert list(counts[:4]) == [0] * 4 and list(ms[:4]) == [0.0] * 4
    assert list(counts[4:]) == [7] * 4 and list(ms[4:]) == [7.5] * 4


def test_no_fallback_without_the_library(tmp_path):
    """Without libattn.so every call that needs it raises ImportError, and host tensors are refused: there
    is no CPU path to fall back to."""
    import torch
    saved = (A.LIB_PATH, A._lib)
    try:
        A.LIB_PATH, A._lib = str(tmp_path / "libattn.so"), None
        with pytest.raises(ImportError):
            A.lib()
        with pytest.raises(ImportError):
            A.workspace_bytes(1, 2, 8, 64, 4)
        with pytest.raises(ImportError):
            A.ffn_workspace_bytes(100, 256, 64)
    finally:
        A.LIB_PATH, A._lib = saved
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        A.fwd(q, q, q)
    with pytest.raises(ValueError, match="device tensor"):
        A.ffn_blockwise(torch.zeros(4, 64, dtype=torch.bfloat16), torch.zeros(64, 64, dtype=torch.bfloat16), None,
                        torch.zeros(64, 64, dtype=torch.bfloat16), None)


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one device's share: --gpus N > 1 exits with status 2 and says so, before it
    touches a GPU."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=root)
    assert r.returncode == 2 and "one GPU" in r.stderr and not r.stdout


def test_last_error_is_per_thread():
    """Two threads fail validation at the same time with different errors; each reads its own message
    (ctypes drops the interpreter lock inside each call, so the calls interleave)."""
    import threading
    start = threading.Barrier(2)
    bad = []

    def worker(call, status, text):
        start.wait()
        for _ in range(2000):
            if call() != status or text not in last_error():
                bad.append((status, last_error()))
                return

    ts = [threading.Thread(target=worker, args=(lambda: fwd(scale=math.nan), 5, "finite")),
          threading.Thread(target=worker, args=(lambda: fwd(d=48), 3, "d = 64 or 128"))]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not bad, bad


def test_last_error_is_per_call():
    assert fwd(scale=math.nan) == 5
    assert "finite" in last_error()
    assert fwd(d=48) == 3
    assert "d = 64 or 128" in last_error()


def ffn(*, x=P[0], w1=P[1], b1=None, w2=P[2], b2=None, y=P[3], M=100, d=64, d_ff=256, block=64, act=2, ws=P[4],
        ws_n=1 << 40):
    return A.lib().attn_ffn_blockwise(x, w1, b1, w2, b2, y, M, d, d_ff, block, act, ws, ws_n, None)


def test_ffn_workspace_formula():
    ws = A.lib().attn_ffn_workspace_bytes
    assert ws(100, 256, 64) == 64 * 256 * 2                 # one block of 64 rows, bf16
    assert ws(10, 256, 64) == 10 * 256 * 2                  # M < block: one block of M rows
    assert ws(4096, 16384, 4096) == 4096 * 16384 * 2
    assert ws(0, 256, 64) == 0 and ws(10, 0, 4) == 0 and ws(10, 256, 0) == 0


def test_ffn_validation():
    """Every rejection of attn_ffn_blockwise happens before any HIP call."""
    assert ffn(x=None) == 1 and ffn(w1=None) == 1 and ffn(w2=None) == 1 and ffn(y=None) == 1
    assert ffn(M=0) == 2 and ffn(block=0) == 2
    assert ffn(d=48) == 3 and ffn(d_ff=100) == 3 and ffn(d=0) == 3     # multiples of 64
    assert ffn(d=96) == 3 and ffn(d_ff=288) == 3 and ffn(d=32) == 3
    assert ffn(act=7) == 4
    assert ffn(ws=None) == 6 and ffn(ws_n=64 * 256 * 2 - 1) == 6
    assert ffn(x=ctypes.c_void_p(P[0].value + 8)) == 9 and ffn(y=ctypes.c_void_p(P[3].value + 2)) == 9
    assert ffn(b1=ctypes.c_void_p(P[5].value + 4)) == 9 and ffn(ws=ctypes.c_void_p(P[4].value + 8)) == 9
    assert ffn(y=ctypes.c_void_p(P[0].value + 64)) == 7      # Y overlaps X
    assert ffn(ws=ctypes.c_void_p(P[1].value + 4096)) == 7   # workspace overlaps W1
    assert ffn(y=P[4]) == 7                                   # Y overlaps the workspace
    assert ffn(b2=ctypes.c_void_p(P[3].value + 16)) == 7     # Y overlaps b2
    far = [ctypes.c_void_p((1 << 47) * (i + 1)) for i in range(6)]
    # a hidden block of 2^31 bytes (65536 rows x 16384) and weights of 2^31 bytes (32768 x 32768) are refused
    assert ffn(x=far[0], w1=far[1], w2=far[2], y=far[3], ws=far[4], M=65536, d=64, d_ff=16384, block=65536) == 2
    assert ffn(x=far[0], w1=far[1], w2=far[2], y=far[3], ws=far[4], M=64, d=32768, d_ff=32768, block=64) == 2
    assert "2^31" in last_error()


def test_timing_read_without_launches():
    assert A.lib().attn_timing_enable(1) == 0
    assert A.timing_read() == {"fwd": (0, 0.0), "merge": (0, 0.0), "copy": (0, 0.0), "ffn": (0, 0.0)}
    assert A.lib().attn_timing_enable(0) == 0


def test_python_errors_name_the_status():
    err = A.AttnError(3, "attn_fwd", "x")
    assert "ATTN_ERR_UNSUPPORTED_D" in str(err) and err.status == 3


def test_fwd_acc_validation():
    assert fwd_acc(oa=None) == 1 and "O_acc" in last_error()
    assert fwd_acc(la=None) == 1
    assert fwd_acc(d=100) == 3
    assert fwd_acc(oa=ctypes.c_void_p(P[5].value + 8)) == 9            # bf16 inputs: O_acc 16-byte aligned
    assert fwd_acc(la=ctypes.c_void_p(P[6].value + 2)) == 9
    assert fwd_acc(oa=P[0]) == 7 and "overlaps an input" in last_error()   # O_acc over Q
    assert fwd_acc(la=P[2]) == 7                                        # lse_acc over V
    assert fwd_acc(o=P[5]) == 7 and "fp32 output" in last_error()       # in place needs an fp32 O
    assert fwd_acc(o=ctypes.c_void_p(P[5].value + 64), dout=A.ATTN_F32) == 7   # partial overlap of O and O_acc
    assert fwd_acc(lse=ctypes.c_void_p(P[6].value + 4)) == 7            # partial overlap of LSE and lse_acc
    assert fwd_acc(la=ctypes.c_void_p(P[5].value + 256)) == 7           # lse_acc inside O_acc
    assert fwd_acc(din=A.ATTN_F32, dout=A.ATTN_BF16) == 4
