"""The CPU test suite under AddressSanitizer and UndefinedBehaviorSanitizer
(host code only; no GPU).

    python tests/run_sanitized.py [extra pytest arguments]

Builds, beside the normal builds (which must exist: __graft_entry__.build()):
  - bit_quantized_gemm_token_amd/_build_san/libw8gemm.so: every translation
    unit with host code (the C-ABI's argument validation and dispatch, the
    config table's parser, the cost model, the tuner's host side, the
    registry) compiled again with both sanitizers on its host side only
    (each flag behind -Xarch_host: device code is never instrumented), linked
    with the normal build's kernel-instance objects;
  - oracle/_build_san/libw8oracle.so: the oracle, with ROCm's clang so that
    both share one sanitizer runtime (without OpenMP: its loops run on one
    thread, with the same arithmetic);
then runs `pytest tests -m "not gpu"` in a child process that loads these
two builds (W8_LIBRARY, W8_ORACLE_LIBRARY) with clang's AddressSanitizer
runtime preloaded.  Any sanitizer report ends that process with an error
(UBSan does not recover; leak checking is off, the interpreter's own
allocations never being freed).  Exit status: pytest's.
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "bit_quantized_gemm_token_amd")
CLANG_DIR = "/opt/rocm/llvm"

# host-only flags, each behind -Xarch_host
HOST_SAN = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
            "-Xarch_host -fno-sanitize-recover=undefined "
            "-Xarch_host -fno-omit-frame-pointer -Xarch_host -g").split()
ORACLE_SAN = "-fsanitize=address,undefined -fno-sanitize-recover=undefined".split()


def _load_build():
    import importlib.util
    spec = importlib.util.spec_from_file_location("w8_build", os.path.join(PKG, "build.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def build_library():
    b = _load_build()
    out_dir = os.path.join(PKG, "_build_san")
    os.makedirs(out_dir, exist_ok=True)
    host = [u for u in b._units() if u[0] != "w8_gemm_inst.hip"]
    inst = [os.path.join(b.OBJ, u[2]) for u in b._units() if u[0] == "w8_gemm_inst.hip"]
    missing = [o for o in inst if not os.path.exists(o)]
    if missing:
        raise SystemExit(f"build the library first ({len(missing)} kernel objects missing)")

    def one(u):
        src, extra, obj = u
        cmd = [b.HIPCC, *b.FLAGS, *HOST_SAN, *extra, "-c", os.path.join(b.CSRC, src), "-o",
               os.path.join(out_dir, obj)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")

    with cf.ThreadPoolExecutor(min(len(host), 8)) as ex:
        list(ex.map(one, host))
    lib = os.path.join(out_dir, "libw8gemm.so")
    # the sanitizer runtime is not linked in: it is preloaded into the test process
    subprocess.run([b.HIPCC, f"--offload-arch={b.ARCH}", "-shared", "-fPIC", "-o", lib,
                    f"-Wl,--version-script={os.path.join(b.CSRC, 'w8gemm.map')}",
                    *[os.path.join(out_dir, u[2]) for u in host], *inst], check=True)
    return lib


def build_oracle():
    src = os.path.join(ROOT, "oracle", "w8_oracle.c")
    out_dir = os.path.join(ROOT, "oracle", "_build_san")
    os.makedirs(out_dir, exist_ok=True)
    lib = os.path.join(out_dir, "libw8oracle.so")
    subprocess.run([os.path.join(CLANG_DIR, "bin", "clang"), "-O1", "-g", "-fPIC", "-shared",
                    "-fno-omit-frame-pointer", *ORACLE_SAN, "-fno-fast-math", "-ffp-contract=off",
                    "-std=c11", "-Wall", "-Wextra", "-Wno-unknown-pragmas", "-Werror",
                    "-o", lib, src, "-lm"], check=True)
    return lib


def main(argv):
    lib, olib = build_library(), build_oracle()
    rt = glob.glob(os.path.join(CLANG_DIR, "lib", "clang", "*", "lib", "linux",
                                "libclang_rt.asan-x86_64.so"))
    if not rt:
        raise SystemExit("clang's AddressSanitizer runtime not found")
    env = dict(os.environ, W8_LIBRARY=lib, W8_ORACLE_LIBRARY=olib, LD_PRELOAD=rt[0],
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    print(f"[sanitized] {lib}\n[sanitized] {olib}\n[sanitized] runtime {rt[0]}", flush=True)
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-m", "not gpu", "-q",
           "-p", "no:cacheprovider", *argv]
    return subprocess.run(cmd, env=env, cwd=ROOT).returncode


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
