"""Build the HIP library ``libdg.so`` (gfx950 only) in-tree.

Every HIP source is compiled by hipcc for ``--offload-arch=gfx950`` with packed
fp32 instructions disabled; the host-only planner is compiled the same way so
the library links as one unit.  Objects go to ``_build/``, the library to
``tile_planned_generator_amd/libdg.so``.
"""
import concurrent.futures as cf
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdg.so")

KERNEL_SOURCES = ["gemm_tiled_f16.hip", "gemm_tiled_bf16.hip", "gemm_tiled_i8.hip",
                  "gemm_tiled_e2m1.hip", "gemm_tiled_mx.hip", "quant_mx.hip", "skinny.hip", "probe.hip",
                  "scratch.hip"]
HOST_SOURCES = ["gemm_tiled.hip", "api.cpp", "planner.cpp"]
# kernel sources that issue transposing LDS reads (row-major B operands)
TILED_TR_SOURCES = ["gemm_tiled_f16.hip", "gemm_tiled_bf16.hip", "gemm_tiled_i8.hip"]
RESOURCES = os.path.join(CSRC, "resources.inc")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I" + CSRC, "-I" + os.path.join(ROOT, "include")]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [HIPCC, *DEVICE, *COMMON, "-x", "hip", "-c", path, "-o", obj]
        if src in KERNEL_SOURCES:
            cmd.append("-Rpass-analysis=kernel-resource-usage")
    else:
        cmd = [HIPCC, *COMMON, "-D__HIP_PLATFORM_AMD__", "-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{out}")
    return obj, out


# kernel family ids (planner.h: F_TILED, F_SKINNY_VALU, F_SKINNY_MFMA, F_SKINNY_E2M1)
_FAMILIES = {"gemm_tiled_kernel": 0, "skinny_valu_kernel": 1, "skinny_mfma_kernel": 2,
             "skinny_e2m1_kernel": 3}


def _parse_resources(remarks):
    """Per compiled kernel: (family, template args) -> VGPRs, AGPRs, LDS bytes,
    waves per SIMD, from the compiler's kernel-resource-usage remarks."""
    rows, cur = {}, None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            fam = next((f for k, f in _FAMILIES.items() if k in name), None)
            if fam is None:
                cur = None
                continue
            args = [int(x) for x in re.findall(r"Li(-?\d+)E", name)]
            cur = (fam, tuple(args + [0] * (8 - len(args))))
            rows[cur] = {}
            continue
        if cur is None:
            continue
        for key, field in (("VGPRs:", "vgpr"), ("AGPRs:", "agpr"), ("LDS Size [bytes/block]:", "lds"),
                           ("Occupancy [waves/SIMD]:", "occ"), ("VGPRs Spill:", "spill"),
                           ("ScratchSize [bytes/lane]:", "scratch")):
            m = re.search(re.escape(key) + r" (\d+)", line)
            if m:
                rows[cur][field] = int(m.group(1))
    return rows


def _regs(operands):
    out = set()
    for m in re.finditer(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b", operands):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _check_transposing_reads(src):
    """The tiled kernel issues its transposing LDS reads from inline assembly,
    which the compiler's wait insertion does not see: until a wait covers such a
    read, its destination registers are still being written.  LDS operations
    complete in order, so while a read is in flight so is every later LDS
    operation, and the counter (which also counts scalar memory reads) is above
    their number: an lgkmcnt(N) wait covers every read followed by at least N
    later LDS operations.  Scan the device assembly of `src` in program order and return every
    instruction that touches a register of a read not yet covered (one that
    would read a value not yet landed, or write a register the read will
    overwrite)."""
    path = os.path.join(CSRC, src)
    cmd = [HIPCC, *DEVICE, *COMMON, "-x", "hip", "--cuda-device-only", "-S", path, "-o", "-"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"assembling {src} failed:\n{r.stderr}")
    return scan_transposing_reads(r.stdout)


def scan_transposing_reads(asm):
    """The scan of _check_transposing_reads over device assembly text."""
    bad, kernel = [], None
    pend = []           # [registers, LDS operations issued after the read]
    for line in asm.splitlines():
        if re.match(r"^_ZN\w+:", line):
            kernel, pend = line.split(":")[0], []
            continue
        t = line.strip()
        if not t or t.startswith((";", ".")) or kernel is None:
            continue
        op = t.split()[0]
        if op == "s_waitcnt":
            m = re.search(r"lgkmcnt\((\d+)\)", t)
            if m:
                n = int(m.group(1))
                pend = [e for e in pend if e[1] < n]
            continue
        operands = t.split(";")[0][len(op):]
        regs = set().union(*(e[0] for e in pend)) if pend else set()
        if op.startswith("ds_read_b64_tr"):
            dst = _regs(operands.split(",")[0])
            if regs & _regs(operands):
                bad.append(f"{kernel}: {t}")
            for e in pend:
                e[1] += 1
            pend.append([dst, 0])
            continue
        if regs & _regs(operands):
            bad.append(f"{kernel}: {t}")
        if op.startswith("ds_"):
            for e in pend:
                e[1] += 1
    return bad


def _write_resources(rows):
    lines = ["// resources.inc - registers, LDS and occupancy of every compiled kernel variant,",
             "// extracted from the compiler's kernel-resource-usage remarks by build.py.",
             "// {family, template args (8, zero-padded), VGPRs, AGPRs, LDS bytes, waves/SIMD, spills}"]
    for (fam, args), r in sorted(rows.items()):
        lines.append("{%d, %s, %d, %d, %d, %d, %d}," % (
            fam, ", ".join(str(a) for a in args), r.get("vgpr", 0), r.get("agpr", 0),
            r.get("lds", 0), r.get("occ", 0), r.get("spill", 0)))
    text = "\n".join(lines) + "\n"
    old = open(RESOURCES).read() if os.path.exists(RESOURCES) else None
    if old != text:
        with open(RESOURCES, "w") as fh:
            fh.write(text)


def build(verbose: bool = False, jobs: int = 0) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(jobs) as ex:
        done = list(ex.map(lambda s: _compile(s, verbose), KERNEL_SOURCES))
    rows = _parse_resources("\n".join(out for _, out in done))
    spills = [k for k, r in rows.items() if r.get("spill", 0) or r.get("scratch", 0)]
    if spills:
        raise RuntimeError(f"kernel variants spill registers or use private memory: {spills}")
    _write_resources(rows)
    with cf.ThreadPoolExecutor(jobs) as ex:
        hazards = [h for hs in ex.map(_check_transposing_reads, TILED_TR_SOURCES) for h in hs]
    if hazards:
        raise RuntimeError("instructions touch registers of in-flight transposing LDS reads:\n" +
                           "\n".join(hazards[:20]))
    with cf.ThreadPoolExecutor(jobs) as ex:
        done += list(ex.map(lambda s: _compile(s, verbose), HOST_SOURCES))
    objs = [o for o, _ in done]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
