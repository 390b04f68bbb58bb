"""The oracle's pins under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): the C oracle is rebuilt with -fsanitize=address,undefined and
every pin runs against that build in a child process (the sanitizer runtime
is preloaded there, since the Python interpreter itself is not
instrumented). A copy with one planted out-of-bounds write must abort, which
shows the sanitizer is live in that build."""
import os
import subprocess
import sys

import pytest

from oracle.build import SOURCE, compile_source

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]
RUN_PINS = (
    "import sys\n"
    f"sys.path[:0] = [{HERE!r}, {ROOT!r}]\n"
    "import oracle, oracle_pins\n"
    "orc = oracle.Oracle(sys.argv[1])\n"
    "for pin in oracle_pins.ALL_PINS:\n"
    "    pin(orc)\n"
    "print('pins passed:', len(oracle_pins.ALL_PINS))\n"
)


def _runtime() -> str:
    cc = os.environ.get("CC", "gcc")
    path = subprocess.run([cc, "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not path or not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("no AddressSanitizer runtime for the host compiler")
    return path


def _run(lib: str) -> subprocess.CompletedProcess:
    env = dict(os.environ, LD_PRELOAD=_runtime(), ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return subprocess.run([sys.executable, "-c", RUN_PINS, lib], capture_output=True, text=True,
                          env=env, timeout=600)


def test_pins_pass_under_sanitizers(tmp_path):
    lib = compile_source(SOURCE, str(tmp_path / "liboracle_san.so"), SAN)
    res = _run(lib)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    assert "pins passed" in res.stdout


def test_sanitizer_catches_a_planted_overflow(tmp_path):
    src = open(SOURCE).read()
    old = "double* s = (double*)malloc(sizeof(double) * (size_t)Sk);"
    assert src.count(old) == 2
    bad = src.replace(old, old + "\n        s[Sk] = 0.0;", 1)
    path = tmp_path / "overflow.c"
    path.write_text(bad)
    lib = compile_source(str(path), str(tmp_path / "liboverflow.so"), SAN)
    res = _run(lib)
    assert res.returncode != 0
    assert "heap-buffer-overflow" in res.stderr
