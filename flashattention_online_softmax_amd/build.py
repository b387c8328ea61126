"""Builds libfa.so (the gfx950 attention forward library) in-tree.

Two kinds of device code go into it:
  * fa_abi / fa_dense / fa_topk: ordinary HIP sources compiled by hipcc.
  * fa_fwd16 and fa_topk16: the 16-bit forward kernels, compiled on their own
    into one gfx950 code object that libfa.so embeds and loads at run time.
    They keep MFMA-only state in AGPRs (fa_fwd16 its Q operands, fa_topk16
    its O accumulators) and need most of the VGPRs next to it; with both
    register files in use the compiler would split a wave's registers evenly
    between the two files. The build therefore stops after
    the device IR, links the two modules, sets each kernel's
    "amdgpu-agpr-alloc" (the number of AGPRs to reserve), generates code with
    llc and links the code object with lld.
"""
import concurrent.futures
import os
import re
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfa.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["fa_abi.hip", "fa_dense.hip", "fa_topk.hip", "fa_module.hip", "fa_bwd.hip", "fa_split.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
LLVM_BIN = os.environ.get("FA_LLVM_BIN", "/opt/rocm/lib/llvm/bin")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         # Packed fp32 VALU ops are kept out of every kernel.
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(HERE, "..", "include")]


CODE_OBJECT_SOURCES = ["fa_fwd16.hip", "fa_topk16.hip"]


def _agprs(kernel: str) -> int:
    """AGPRs reserved for a code-object kernel.

    fa_fwd16: for each 32-row block of the wave its Q^T operands (D / 4 per
    lane; the O^T accumulators are VGPRs); name fields d<D>, q<blocks>.
    fa_topk16: the O^T accumulators of 32 heads x 512 (256 per lane)."""
    if kernel.startswith("fa_topk16_"):
        return 256
    d = int(re.search(r"_d(\d+)_", kernel).group(1))
    q = int(re.search(r"_q(\d+)_", kernel).group(1))
    return (d // 4) * q


def _sched_strategy(kernel: str):
    """Machine scheduler strategy of a code-object kernel. Interleaved A/B
    on one MI355X host, against the default: "max-ilp" measured 0.7-0.9%
    faster on the dense causal BNSD kernels and 2% on block-sparse, but
    0.6-0.9% slower with a boolean mask or split-KV ranges; "iterative-ilp"
    measured 0.2-1.1% faster on the masked, split-KV and packed kernels, 1.3-
    1.5% faster than "max-ilp" on top-k and 1% slower than it on dense causal
    S = 8192. "max-ilp" therefore goes to the BNSD kernels without a mask
    (fields m0, x0), "iterative-ilp" to all others."""
    if re.search(r"m0s\dx0$", kernel):
        return "max-ilp"
    return "iterative-ilp"


def _run(cmd, what):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("%s failed:\n%s\n%s" % (what, " ".join(cmd), r.stderr))
    return r


# Per-source extra flags. The backward kernels let the compiler place MFMA
# accumulators; asking for the VGPR form keeps the scores, which the VALU
# reads right away, out of AGPRs (fewer accumulator moves per tile).
EXTRA_FLAGS = {"fa_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
    _run([HIPCC, *FLAGS, *EXTRA_FLAGS.get(src, []), "-I", BUILD_DIR, "-c", os.path.join(CSRC, src), "-o", obj],
         "hipcc " + src)
    return obj


def _set_agpr_alloc(ir: str) -> str:
    """Gives every code-object kernel its own attribute group with
    amdgpu-agpr-alloc (and, where chosen, amdgpu-sched-strategy) set."""
    groups = dict(re.findall(r"^attributes #(\d+) = \{(.*)\}$", ir, re.M))
    next_id = max(int(g) for g in groups) + 1
    new_groups = []

    def patch_define(m):
        nonlocal next_id
        name, gid = m.group(2), m.group(4)
        body = re.sub(r'\s*"amdgpu-agpr-alloc"="[^"]*"', "", groups[gid]).rstrip()
        sched = _sched_strategy(name)
        extra = ' "amdgpu-sched-strategy"="%s"' % sched if sched else ""
        new_groups.append('attributes #%d = {%s "amdgpu-agpr-alloc"="%d"%s }' % (next_id, body, _agprs(name), extra))
        out = m.group(1) + name + m.group(3) + str(next_id)
        next_id += 1
        return out

    ir, n = re.subn(r"^(define [^@]*amdgpu_kernel void @)(fa_(?:fwd|topk)16_\w+)(\(.*\) [^#]*#)(\d+)",
                    patch_define, ir, flags=re.M)
    if n == 0:
        raise RuntimeError("no code-object kernels found in the device IR")
    return ir + "\n" + "\n".join(new_groups) + "\n"


def _device_ir(src: str) -> str:
    bc = os.path.join(BUILD_DIR, src.replace(".hip", ".bc"))
    _run([HIPCC, *FLAGS, "--cuda-device-only", "-emit-llvm", "-c",
          os.path.join(CSRC, src), "-o", bc], "hipcc %s (device IR)" % src)
    return bc


def _build_code_object() -> str:
    """fa_fwd16.hip + fa_topk16.hip -> gfx950 code object -> C array include
    for fa_module.hip."""
    bc = os.path.join(BUILD_DIR, "fa_kernels.bc")
    ll = os.path.join(BUILD_DIR, "fa_kernels.ll")
    obj = os.path.join(BUILD_DIR, "fa_kernels.gfx950.o")
    hsaco = os.path.join(BUILD_DIR, "fa_kernels.hsaco")
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(CODE_OBJECT_SOURCES)) as ex:
        bcs = list(ex.map(_device_ir, CODE_OBJECT_SOURCES))
    _run([os.path.join(LLVM_BIN, "llvm-link"), *bcs, "-o", bc], "llvm-link")
    _run([os.path.join(LLVM_BIN, "llvm-dis"), bc, "-o", ll], "llvm-dis")
    with open(ll) as f:
        ir = _set_agpr_alloc(f.read())
    with open(ll, "w") as f:
        f.write(ir)
    _run([os.path.join(LLVM_BIN, "llc"), "-O3", "-mtriple=amdgcn-amd-amdhsa", "-mcpu=gfx950",
          "-filetype=obj", ll, "-o", obj], "llc code object")
    _run([os.path.join(LLVM_BIN, "ld.lld"), "-shared", obj, "-o", hsaco], "ld.lld code object")
    with open(hsaco, "rb") as f:
        blob = f.read()
    inc = os.path.join(BUILD_DIR, "fa_kernels_hsaco.inc")
    lines = []
    for i in range(0, len(blob), 24):
        lines.append(",".join(str(b) for b in blob[i:i + 24]) + ",")
    with open(inc + ".tmp", "w") as f:
        f.write("// generated by build.py from csrc/%s; do not edit\n" % " + csrc/".join(CODE_OBJECT_SOURCES))
        f.write("static const unsigned char kCodeObject[%d] __attribute__((aligned(4096))) = {\n" % len(blob))
        f.write("\n".join(lines))
        f.write("\n};\n")
    os.replace(inc + ".tmp", inc)
    return inc


def build(verbose: bool = False) -> str:
    """Compiles every HIP source for gfx950 and links libfa.so next to this file."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        kernels = ex.submit(_build_code_object)
        others = [ex.submit(_compile, s) for s in SOURCES if s != "fa_module.hip"]
        kernels.result()
        objs = [f.result() for f in others] + [_compile("fa_module.hip")]
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], "link")
    # A kernel template whose host-side instantiation is silently rejected
    # leaves its launch stub undefined; catch that here rather than at load.
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [l.split()[-1] for l in nm.stdout.splitlines() if "__device_stub__" in l]
    if missing:
        os.remove(tmp)
        raise RuntimeError("undefined kernel launch stubs in libfa.so:\n  " + "\n  ".join(missing))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
