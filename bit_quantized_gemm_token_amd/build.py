"""Build libw8gemm.so (HIP, gfx950 only) in-tree.

Compiles every translation unit under csrc/ with hipcc in parallel and links
them into bit_quantized_gemm_token_amd/libw8gemm.so.  The GEMM instance file is
compiled once per (format, swap_ab, part).  Beside it, the phase probe
(csrc/w8_phase_probe.hip: the GEMM kernel with timing stamps, a timing-study
executable, not part of the library) is built as w8_phase_probe.  Flags:
  -fhip-fp32-correctly-rounded-divide-sqrt  the quantizer's x / s is the IEEE
                                            correctly rounded division
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                            no packed fp32 VALU instructions
  no fast-math.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libw8gemm.so")
PROBE = os.path.join(HERE, "w8_phase_probe")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Wno-unused-command-line-argument",
         "-fhip-fp32-correctly-rounded-divide-sqrt",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         f"-I{INCLUDE}"]


def _units():
    units = [("w8_quant.hip", [], "w8_quant.o"),
             ("w8_pack.hip", [], "w8_pack.o"),
             ("w8_floor.hip", [], "w8_floor.o"),
             ("w8_tune.hip", [], "w8_tune.o"),
             ("w8_capi.cpp", ["-x", "hip"], "w8_capi.o"),
             ("w8_table.cpp", ["-x", "hip"], "w8_table.o"),
             ("w8_model.cpp", ["-x", "hip"], "w8_model.o"),
             ("w8_moe.cpp", ["-x", "hip"], "w8_moe.o"),
             ("w8_registry.cpp", ["-x", "hip"], "w8_registry.o")]
    # the instance file in 40 parts (the GEMM parts, the largest, first so
    # the pool stays busy; parts 4 and 5 exist for Block_FP8 only), then the
    # small units
    inst = [("w8_gemm_inst.hip", [f"-DW8_FMT={fmt}", f"-DW8_SWAP={swap}", f"-DW8_PART={part}"],
             f"w8_gemm_f{fmt}_s{swap}_p{part}.o")
            for part in (0, 1, 2, 3, 6, 7, 4, 5) for fmt in (0, 1, 2) for swap in (0, 1)
            if part not in (4, 5) or fmt == 2]
    return inst + units


def _compile(unit, verbose):
    src, extra, obj = unit
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", os.path.join(OBJ, obj)]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src} {' '.join(extra)}:\n{out}")
    return out


def _build_probe(verbose):
    tmp = PROBE + ".tmp"
    cmd = [HIPCC, *[f for f in FLAGS if f != "-fPIC"], os.path.join(CSRC, "w8_phase_probe.hip"),
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on w8_phase_probe.hip:\n{r.stdout}{r.stderr}")
    os.replace(tmp, PROBE)


def build(verbose: bool = False, jobs: int = 0) -> str:
    os.makedirs(OBJ, exist_ok=True)
    units = _units()
    jobs = jobs or min(len(units), max(1, min(os.cpu_count() or 4, 8)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        probe = ex.submit(_build_probe, verbose)
        for msg in ex.map(lambda u: _compile(u, verbose), units):
            if msg and verbose:
                print(msg, flush=True)
        probe.result()
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
           f"-Wl,--version-script={os.path.join(CSRC, 'w8gemm.map')}",
           *[os.path.join(OBJ, u[2]) for u in units]]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
