"""Runs the CPU test suite (-m "not gpu") against AddressSanitizer + UndefinedBehaviorSanitizer
builds of the library's host code (argument validation, planning, workspace layout, launch set-up
in api.hip and the launchers) and of the C oracle.

    python tests/run_sanitized.py [extra pytest args]

Both builds go to a temporary directory; the run preloads clang's ASan runtime, stops at the first
report (halt_on_error, -fno-sanitize-recover) and leaves leak checking off (the interpreter keeps
its allocations until exit).  The GPU code is built as usual: no GPU sanitizer is used."""
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from selective_state_space_55_amd import build as hipbuild  # noqa: E402


def main(argv):
    with tempfile.TemporaryDirectory(prefix="mscan_san_") as d:
        lib = hipbuild.build(out_path=os.path.join(d, "libmamba_scan_san.so"), host_sanitize=True)
        orc = oracle.build(out_path=os.path.join(d, "liboracle_scan_san.so"), sanitize=True)
        env = dict(os.environ)
        env.update(LD_PRELOAD=hipbuild.asan_runtime(), MAMBA_SCAN_LIBRARY=lib, ORACLE_SCAN_LIBRARY=orc,
                   ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
        for path in (lib, orc):   # both builds carry the instrumentation
            syms = subprocess.run(["nm", "-D", "--undefined-only", path], capture_output=True, text=True).stdout
            assert "__asan_report" in syms and "__ubsan_handle" in syms, path
        probe = ("import ctypes, oracle, selective_state_space_55_amd as m; m.load_library(); oracle.max_threads(); "
                 "maps = open('/proc/self/maps').read(); "
                 "assert 'libmamba_scan_san.so' in maps and 'liboracle_scan_san.so' in maps and 'asan' in maps; "
                 "print('sanitized builds loaded')")
        subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, check=True)
        cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-m", "not gpu", "-x", "-q",
               "-p", "no:cacheprovider"] + list(argv)
        print("sanitized run:", " ".join(cmd), flush=True)
        return subprocess.run(cmd, cwd=ROOT, env=env).returncode


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
