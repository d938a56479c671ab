"""Host-code sanitizer run, CPU only (no GPU is touched).

Builds the oracle with g++ -fsanitize=address,undefined and the library with
its host code under AddressSanitizer and UndefinedBehaviorSanitizer (hipcc,
each flag behind -Xarch_host; the GPU code is built as usual) into a scratch
directory, then runs, each in its own process with its sanitizer runtime
preloaded:
  - the oracle's pins (tests/test_oracle_pins.py) against the sanitized oracle;
  - the library's host-side checks (tests/test_abi_host.py,
    tests/test_binding_host.py) against the sanitized library.
Any report fails the run (UBSan does not recover; ASan aborts).

    python tests/sanitize_host.py [scratch_dir]
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def gcc_runtime(name: str) -> str:
    return subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True,
                          check=True).stdout.strip()


def clang_asan_runtime() -> str:
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("no clang ASan runtime under /opt/rocm/llvm")
    return hits[-1]


def run(tests, env_extra) -> int:
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["CUDA_VISIBLE_DEVICES"] = ""  # host checks only
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu", *tests]
    print("+", " ".join(f"{k}={v}" for k, v in env_extra.items()), " ".join(cmd), flush=True)
    return subprocess.run(cmd, cwd=ROOT, env=env).returncode


def main() -> int:
    scratch = sys.argv[1] if len(sys.argv) > 1 else tempfile.mkdtemp(prefix="hw_sanitize_")
    os.makedirs(scratch, exist_ok=True)
    import oracle
    from decode_attention_shared_hw_amd import build

    olib = oracle.build(out=os.path.join(scratch, "libhogwild_oracle_san.so"), sanitize=True)
    hlib = build.build(out=os.path.join(scratch, "libhogwild_attn_san.so"), sanitize=True)
    rc = run(["tests/test_oracle_pins.py"],
             {"LD_PRELOAD": gcc_runtime("libasan.so") + ":" + gcc_runtime("libubsan.so"),
              "HWO_LIB": olib})
    rc2 = run(["tests/test_abi_host.py", "tests/test_binding_host.py"],
              {"LD_PRELOAD": clang_asan_runtime(), "HW_TEST_LIB": hlib})
    print(f"oracle pins: rc {rc}; library host checks: rc {rc2}", flush=True)
    return rc or rc2


if __name__ == "__main__":
    sys.exit(main())
