"""Compile libattn.so (the C-ABI library) in-tree for gfx950 with hipcc.

Usage: ``python -m exact_blockwise_attention_fwd_amd.build`` (or ``__graft_entry__.build()``).  Every call
recompiles: sources are compiled in parallel to objects under ``_build/`` and linked into
``exact_blockwise_attention_fwd_amd/libattn.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libattn.so")
ARCH = "gfx950"

SOURCES = ["attn_api.hip", "attn_fwd_bf16.hip", "attn_fwd_f32.hip", "attn_merge.hip", "ffn_bf16.hip"]

# Packed fp32 VALU instructions are switched off for all device code (the compiler would otherwise form
# them from ordinary float code); the host pass warns that it does not know the feature, which is harmless.
# MFMA results are allocated to ordinary VGPRs where possible (the softmax reads the score accumulators
# with VALU instructions; accumulators parked in AGPRs would need a copy per element and tile).
CODEGEN_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Werror",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]
HIPCC_FLAGS = CODEGEN_FLAGS + ["-I", INCLUDE, "-I", CSRC]


# Per-source additions.  The bf16 attention kernel is scheduled with the machine scheduler's memory-clause
# strategy: the order between MFMA batches is pinned in the source, and inside each batch this strategy
# measured bit-identical results at +0.6-0.8 % at d = 128 (the max-ILP strategies were slower on short causal
# rows); at d = 64 the strategies measure the same within 0.5 %.
SOURCE_FLAGS = {
    "attn_fwd_bf16.hip": ["-mllvm", "-amdgpu-sched-strategy=max-memory-clause"],
}


def code_text(text: str) -> str:
    """C/C++ source with its comments removed and every run of whitespace made one space: what the compiler
    sees of it, up to layout (string and character literals are kept as written)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def fingerprint(src: str) -> str:
    """sha256 of a source file's code (comments and layout left out) and the code-generation flags it is
    compiled with (include paths left out, as they differ between machines): recorded counter figures are
    valid only for the build they name, and a change to a comment does not make another build."""
    import hashlib

    h = hashlib.sha256(code_text(open(os.path.join(CSRC, src)).read()).encode())
    h.update(("\n" + " ".join(CODEGEN_FLAGS + SOURCE_FLAGS.get(src, []))).encode())
    return h.hexdigest()


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    flags = HIPCC_FLAGS + list(extra_flags or [])
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmd = [cc, *flags, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if p.returncode != 0:
            failed.append(src)
            print(out, file=sys.stderr)
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        print(r.stdout, file=sys.stderr)
        raise RuntimeError("linking libattn.so failed")
    os.replace(tmp, LIB)
    return LIB


def resource_usage(out_path: str | None = None) -> str:
    """Registers, scratch (spill) bytes and occupancy of every kernel, from the compiler's kernel-resource-usage
    remarks for the device code as built (same flags).  Returns the summary text; writes it to out_path."""
    import re

    cc = hipcc()
    rows = []
    for src in SOURCES:
        cmd = [cc, *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), "--cuda-device-only", "-c", os.path.join(CSRC, src),
               "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}")
        cur = None
        for line in r.stdout.splitlines():
            m = re.search(r"remark: (?:\s*)(Function Name|TotalSGPRs|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|"
                          r"Occupancy \[waves/SIMD\]|SGPRs Spill|VGPRs Spill|LDS Size \[bytes/block\]): (\S+)", line)
            if not m:
                continue
            key, val = m.group(1), m.group(2)
            if key == "Function Name":
                cur = {"src": src, "name": val}
                rows.append(cur)
            elif cur is not None:
                cur[key] = val
    hdr = ("kernel", "source", "VGPRs", "AGPRs", "SGPRs", "scratch B/lane", "VGPR spill", "SGPR spill", "waves/SIMD")
    lines = ["# Kernel resource usage (compiler remarks, -Rpass-analysis=kernel-resource-usage)", "",
             "Command: python -m exact_blockwise_attention_fwd_amd.build --resource-usage (hipcc --cuda-device-only",
             "with the library's own flags: " + " ".join(CODEGEN_FLAGS) + "; per-source: " +
             "; ".join(f"{k}: {' '.join(v)}" for k, v in SOURCE_FLAGS.items()) + ")", "",
             "| " + " | ".join(hdr) + " |", "|" + "---|" * len(hdr)]
    for r_ in rows:
        lines.append(f"| `{r_['name']}` | {r_['src']} | {r_.get('VGPRs')} | {r_.get('AGPRs')} | {r_.get('TotalSGPRs')} | "
                     f"{r_.get('ScratchSize [bytes/lane]')} | {r_.get('VGPRs Spill')} | {r_.get('SGPRs Spill')} | "
                     f"{r_.get('Occupancy [waves/SIMD]')} |")
    lines += ["", "fingerprints (sha256 of source and code-generation flags):", ""]
    lines += [f"{src}: {fingerprint(src)}" for src in SOURCES]
    text = "\n".join(lines) + "\n"
    if out_path:
        with open(out_path, "w") as f:
            f.write(text)
    return text


if __name__ == "__main__":
    if "--resource-usage" in sys.argv:
        print(resource_usage(os.path.join(ROOT, "profiles", "kernel_resource_usage.txt")))
    else:
        print(build(verbose="-v" in sys.argv))
