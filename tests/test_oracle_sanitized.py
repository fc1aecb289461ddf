"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc, host code only) runs
every pin, and the tree helpers refuse inputs that would overrun their fixed work arrays.  The
pins run in a child process that preloads the sanitizer runtime (the Python interpreter itself is
not instrumented); any report aborts it."""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import oracle
from tests import pins
lib = oracle.load({lib!r})
for pin in pins.ALL_PINS:
    pin(lib)
    print("ok", pin.__name__, flush=True)
"""


def test_pins_under_address_and_undefined_sanitizers(tmp_path):
    lib = str(tmp_path / "libev_oracle_asan.so")
    subprocess.run(["gcc", "-O1", "-g", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-std=c11", "-Wall",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                    "-o", lib, os.path.join(ROOT, "oracle", "ev_oracle.c"), "-lm"], check=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=asan, OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", _CHILD.format(root=ROOT, lib=lib)], env=env, capture_output=True,
                       text=True, timeout=900)
    assert r.returncode == 0, f"sanitized pins failed ({r.returncode}):\n{r.stdout[-3000:]}\n{r.stderr[-6000:]}"
    from tests import pins
    assert r.stdout.count("ok ") == len(pins.ALL_PINS)


def test_tree_helpers_refuse_overruns(oracle_lib):
    # a parent chain that is not topological (a cycle) is refused instead of looping
    assert oracle.ancestor_path([-1, 2, 1], 2, lib=oracle_lib).size == 0
    # an index past the work arrays' capacity is refused
    big = np.concatenate([[-1], np.arange(0, 1500)]).astype(np.int32)
    assert oracle.ancestor_path(big, 1200, lib=oracle_lib).size == 0
    assert oracle.tree_errors(big[:1100], 2048, lib=oracle_lib) == 2
    assert oracle.tree_errors(big[:1024], 2048, lib=oracle_lib) == 0
