"""Runs the CPU test suite against host-sanitizer builds (AddressSanitizer and
UndefinedBehaviorSanitizer on the host code of libvsa -- plan, groups, timing,
argument checks -- and on the oracle's C), in a child process with clang's ASan
runtime preloaded. Usage: python tests/run_sanitized.py [extra pytest args].
Exits with pytest's status; any sanitizer report aborts the run."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _load(path, name):
    spec = importlib.util.spec_from_file_location(name, path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def main() -> int:
    builder = _load(os.path.join(ROOT, "tile_sparse_video_amd", "build.py"), "_vsa_build")
    lib = builder.build(sanitize=True)
    import oracle
    orc = oracle.build(sanitize=True)
    clang = "/opt/rocm/lib/llvm/bin/clang"
    runtime = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                             capture_output=True, text=True, check=True).stdout.strip()
    env = dict(os.environ, VSA_LIBRARY=lib, ORACLE_LIBRARY=orc, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-m", "not gpu",
           "-p", "no:cacheprovider", *sys.argv[1:]]
    print("sanitized run:", " ".join(cmd), flush=True)
    return subprocess.run(cmd, env=env, cwd=ROOT).returncode


if __name__ == "__main__":
    sys.exit(main())
