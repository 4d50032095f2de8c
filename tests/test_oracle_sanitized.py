"""The fp64 oracle's C library built with AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): the forward and backward recurrences, with and without an init state, a
ragged tail, several groups and one and several threads, must run clean and give exactly
the bits of the normal build.

The sanitized library runs in a child process with the ASan runtime preloaded (the test
process itself is not instrumented).  Any sanitizer report aborts the child
(-fno-sanitize-recover, halt_on_error), which fails the test."""
import os
import subprocess
import sys
import textwrap

import numpy as np
import pytest

import oracle
from oracle import build as oracle_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = textwrap.dedent("""
    import sys
    import numpy as np
    sys.path.insert(0, {root!r})
    import oracle
    lib = oracle.load_library({lib!r})
    out = {{}}
    rng = np.random.default_rng(7)
    for case, (b, t, h, p, n, g, init, nth) in enumerate([
            (2, 67, 4, 8, 6, 2, True, 0), (1, 130, 2, 4, 3, 1, False, 1),
            (3, 1, 3, 5, 2, 3, True, 3), (1, 0, 2, 4, 4, 1, True, 0)]):
        x = rng.standard_normal((b, t, h, p))
        dt = np.log1p(np.exp(rng.standard_normal((b, t, h)) - 2))
        A = -np.exp(rng.uniform(np.log(0.01), np.log(1.0), h))
        B = rng.standard_normal((b, t, g, n)) / np.sqrt(n)
        C = rng.standard_normal((b, t, g, n)) / np.sqrt(n)
        D = rng.standard_normal(h)
        s0 = rng.standard_normal((b, h, n, p)) * 0.3 if init else None
        dy = rng.standard_normal((b, t, h, p))
        df = rng.standard_normal((b, h, n, p))
        y, fin, bound = oracle.ssd_ref(x, dt, A, B, C, D, init_state=s0, chunk_len=16,
                                       nthreads=nth, lib=lib)
        gr = oracle.ssd_bwd_ref(x, dt, A, B, C, D, dy, init_state=s0, d_final=df,
                                chunk_len=16, nthreads=nth, lib=lib)
        out[f"y{{case}}"], out[f"f{{case}}"] = y, fin
        if bound is not None:
            out[f"b{{case}}"] = bound
        for k in ("dx", "ddt", "dA", "dB", "dC", "dD", "d_init"):
            out[f"{{k}}{{case}}"] = gr[k]
    np.savez({npz!r}, **out)
    print("child ok", flush=True)
""")


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    d = tmp_path_factory.mktemp("asan")
    path = str(d / "libssd_oracle_asan.so")
    oracle_build.compile_oracle(output=path, extra_flags=(
        "-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
        "-fno-sanitize-recover=all"))
    return path


def test_oracle_runs_clean_under_asan_and_ubsan(sanitized_lib, tmp_path):
    npz = str(tmp_path / "out.npz")
    env = dict(os.environ)
    env["LD_PRELOAD"] = subprocess.run(["gcc", "-print-file-name=libasan.so"], check=True,
                                       capture_output=True, text=True).stdout.strip()
    # the interpreter's own allocations are not under test: no leak report at exit
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    code = CHILD.format(root=ROOT, lib=sanitized_lib, npz=npz)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and "child ok" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    # the same calls on the normal build give the same bits
    env2 = {k: v for k, v in os.environ.items() if k != "LD_PRELOAD"}
    npz2 = str(tmp_path / "ref.npz")
    code2 = CHILD.format(root=ROOT, lib=oracle.library()._name, npz=npz2)
    r2 = subprocess.run([sys.executable, "-c", code2], env=env2, capture_output=True, text=True,
                        timeout=300)
    assert r2.returncode == 0, r2.stderr[-2000:]
    a, b = np.load(npz), np.load(npz2)
    assert sorted(a.files) == sorted(b.files)
    for k in a.files:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_the_sanitized_build_catches_a_planted_overrun(tmp_path):
    """A copy of the oracle whose per-thread state buffer is one element short must be
    reported: the check above would not notice a sanitizer that is not really on."""
    src = open(oracle_build.SOURCE).read()
    needle = "(double*)malloc((size_t)(d->dstate * d->headdim) * sizeof(double))"
    assert src.count(needle) == 1
    bad = tmp_path / "ssd_oracle_short.c"
    bad.write_text(src.replace(needle,
                               "(double*)malloc((size_t)(d->dstate * d->headdim - 1) * sizeof(double))"))
    lib = str(tmp_path / "libshort.so")
    oracle_build.compile_oracle(source=str(bad), output=lib, extra_flags=(
        "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"))
    env = dict(os.environ)
    env["LD_PRELOAD"] = subprocess.run(["gcc", "-print-file-name=libasan.so"], check=True,
                                       capture_output=True, text=True).stdout.strip()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    code = CHILD.format(root=ROOT, lib=lib, npz=str(tmp_path / "x.npz"))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr
