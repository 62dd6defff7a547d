"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host code only) runs every pin of tests/pins.py in a child process
without a sanitizer report: no out-of-bounds access, use after free,
signed overflow, misaligned access or other undefined behaviour on the
paths the pins exercise."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")


def _sanitized(tmp_path):
    import importlib.util
    spec = importlib.util.spec_from_file_location("_orc_build_san", os.path.join(ROOT, "oracle", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    lib = b.build(sanitize=True, out=str(tmp_path / "liborc_san.so"))
    env = dict(os.environ)
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = b.sanitizer_runtime() + (":" + pre if pre else "")
    # leaks: CPython and torch keep allocations until exit by design
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return lib, env


def _run(code, env, tmp_path):
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=1200,
                       cwd=str(tmp_path))
    return r, r.stdout + r.stderr


def test_sanitizer_is_live(tmp_path):
    """Negative control: the same harness reports a planted heap overflow
    (a 16-element block read from an 8-element buffer)."""
    lib, env = _sanitized(tmp_path)
    code = ("import sys; sys.path[:0] = [%r]\n"
            "import ctypes, numpy as np, oracle\n"
            "o = oracle.Oracle(%r)\n"
            "xb = np.ones(8, np.float32); q = np.zeros(8, np.uint8)\n"
            "o.L.orc_quantize_block(xb.ctypes.data_as(oracle._f32p), 1.0, q.ctypes.data_as(oracle._u8p))\n"
            "print('NOT_CAUGHT', flush=True)\n") % (ROOT, lib)
    r, log = _run(code, env, tmp_path)
    assert r.returncode != 0 and "NOT_CAUGHT" not in r.stdout, log[-3000:]
    assert "AddressSanitizer" in log and "heap-buffer-overflow" in log, log[-3000:]


def test_pins_under_asan_ubsan(tmp_path):
    lib, env = _sanitized(tmp_path)
    code = ("import sys; sys.path[:0] = [%r, %r]\n"
            "import oracle, pins\n"
            "o = oracle.Oracle(%r)\n"
            "for p in pins.ALL_PINS:\n"
            "    p(o); print('pin ok', p.__name__, flush=True)\n"
            "print('ALL_PINS_OK', flush=True)\n") % (ROOT, TESTS, lib)
    r, log = _run(code, env, tmp_path)
    (tmp_path / "sanitizer.log").write_text(log)
    assert r.returncode == 0, log[-6000:]
    assert "ALL_PINS_OK" in r.stdout, log[-6000:]
    for marker in ("AddressSanitizer", "runtime error:", "UndefinedBehaviorSanitizer"):
        assert marker not in log, log[-6000:]
