"""The CPU sanitizer tier: the CPU test suite (pytest -m "not gpu") under
AddressSanitizer + UndefinedBehaviorSanitizer, in two runs, because one
process can hold only one ASan runtime:

  1. the oracle (oracle/oracle.c) built by gcc with -fsanitize=address,undefined,
     gcc's runtimes preloaded;
  2. libpma's host code (the C ABI's argument checks, workspace arithmetic and
     launch set-up in api.cpp, block_api.cpp, io_api.cpp) built by hipcc with
     the sanitizers on the host pass only (-Xarch_host), clang's shared ASan
     runtime preloaded.  Without a GPU the entry points stop at the device
     check, after every host check has run.

Leak detection is off (the Python interpreter's allocations are not ours);
every other report aborts the run.  Usage: python tests/run_sanitizers.py
Exit status 0 means both runs passed with no sanitizer report.
"""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

CLANG_RT = "/opt/rocm/llvm/lib/clang"


def _gcc_runtimes() -> str:
    libs = [subprocess.run(["gcc", f"-print-file-name={n}"], capture_output=True, text=True,
                           check=True).stdout.strip() for n in ("libasan.so", "libubsan.so")]
    return " ".join(libs)


def _clang_asan() -> str:
    for ver in sorted(os.listdir(CLANG_RT), reverse=True):
        p = os.path.join(CLANG_RT, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    raise FileNotFoundError("clang's shared ASan runtime")


def _pytest(env_extra: dict, label: str) -> int:
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-x", "-m", "not gpu",
           "-p", "no:cacheprovider"]
    print(f"[sanitizers] {label}: {' '.join(cmd)}", flush=True)
    r = subprocess.run(cmd, env=env, cwd=ROOT)
    print(f"[sanitizers] {label}: exit {r.returncode}", flush=True)
    return r.returncode


_PROBE = (
    "import sys; sys.path.insert(0, {root!r})\n"
    "import {mod} as m\n"
    "m.{fn}()\n"
    "maps = open('/proc/self/maps').read()\n"
    "assert {lib!r} in maps, 'sanitized library not loaded'\n"
    "assert 'asan' in maps, 'no ASan runtime in the process'\n"
    "print('loaded', {lib!r})\n")


def _probe(env_extra: dict, mod: str, fn: str, lib: str) -> int:
    """The sanitized build is the one a test process loads, under a live ASan
    runtime, and it is instrumented (it calls the ASan report hooks)."""
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    if "__asan_report" not in syms:
        print(f"[sanitizers] {lib} carries no ASan instrumentation", flush=True)
        return 1
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0"
    code = _PROBE.format(root=ROOT, mod=mod, fn=fn, lib=os.path.basename(lib))
    return subprocess.run([sys.executable, "-c", code], env=env).returncode


def main() -> int:
    import oracle
    from packed_masked_attention_amd import build as pb
    print("[sanitizers] building", oracle.build(force=True, sanitize=True), flush=True)
    print("[sanitizers] building", pb.build(sanitize=True), flush=True)
    env1 = {"LD_PRELOAD": _gcc_runtimes(), "ORACLE_SANITIZED": "1"}
    env2 = {"LD_PRELOAD": _clang_asan(), "PMA_SANITIZED": "1"}
    if _probe(env1, "oracle", "lib", oracle._SAN_PATH) or \
            _probe(env2, "packed_masked_attention_amd.binding", "lib", pb.SAN_LIB):
        return 1
    rc1 = _pytest(env1, "oracle under ASan+UBSan (gcc)")
    rc2 = _pytest(env2, "libpma host code under ASan+UBSan (clang)")
    return 0 if rc1 == 0 and rc2 == 0 else 1


if __name__ == "__main__":
    sys.exit(main())
