"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before any GPU work (CPU only: no compute calls)."""

import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fasa.h")
LIB = os.path.join(ROOT, "sparse_kv_cache_rope_amd", "libfasa.so")


@pytest.fixture(scope="module")
def fasa():
    if not os.path.exists(LIB):
        subprocess.run([sys.executable, os.path.join(ROOT, "sparse_kv_cache_rope_amd", "build.py")], cwd=ROOT,
                       check=True, capture_output=True)
    import sparse_kv_cache_rope_amd as m
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fasa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("fasa_append_kv", "fasa_tip_scores", "fasa_topk", "fasa_sparse_attn",
                 "fasa_decode_step", "fasa_dense_attn", "fasa_create", "fasa_destroy"):
        assert must in names


def test_every_declared_symbol_is_exported(fasa):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (fasa_\w+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing


def test_binding_covers_every_declared_symbol(fasa):
    assert sorted(fasa.EXPORTED) == declared_functions()


def test_status_strings(fasa):
    assert fasa.status_string(0) == "ok"
    assert "invalid" in fasa.status_string(-1)
    assert fasa.status_string(-99) == "unknown status"


@pytest.mark.parametrize("args,code,msg", [
    ((1, 3, 1, 64, 128, 1e4, 1, [[0]] * 3, 1, 8), -3, "not in {1,2,4,8}"),
    ((1, 2, 1, 96, 128, 1e4, 1, [[0]] * 2, 1, 8), -3, "head_dim"),
    ((1, 2, 1, 64, 100, 1e4, 1, [[0]] * 2, 1, 8), -1, "multiple of 64"),
    ((1, 2, 1, 64, 128, 1e4, 1, [[0], [40]], 1, 8), -1, "outside"),
    ((1, 2, 1, 64, 128, 1e4, 1, [[0, 0], [1, 2]], 2, 8), -1, "repeats"),
    ((1, 2, 1, 64, 128, 1e4, 1, [[0], [1]], 1, 200), -1, "max_budget"),
    ((1, 2, 1, 64, 128, 1e4, 1, [[0], [1]], 0, 8), -1, "n_dom"),
    ((1, 2, 1, 64, 128, 0.5, 1, [[0], [1]], 1, 8), -1, "rope_theta"),
    ((1, 2, 1, 64, 128, 1e4, 7, [[0], [1]], 1, 8), -3, "dtype"),
    ((0, 2, 1, 64, 128, 1e4, 1, [[0], [1]], 1, 8), -1, "batch"),
    ((1, 5, 2, 64, 128, 1e4, 1, [[0]] * 5, 1, 8), -1, "multiple"),
    ((1, 2, 1, 64, 128, 1e4, 1, None, 1, 8), -1, "dom_fc is null"),
    ((1, 129, 129, 64, 128, 1e4, 1, [[0]] * 129, 1, 8), -3, "n_kv_heads"),
    ((1, 2, 1, 64, (1 << 24) + 64, 1e4, 1, [[0], [1]], 1, 8), -2, "capacity"),
    ((4096, 8, 8, 64, 1 << 20, 1e4, 1, [[0]] * 8, 1, 1 << 20), -3, "one FAC launch"),
])
def test_create_rejects_bad_arguments(fasa, args, code, msg):
    st, detail = fasa.raw_create(*args)
    assert st == code and msg in detail, (st, detail)


@pytest.mark.parametrize("rotary_dim", [0, 3, 66, -2])
def test_partial_rope_rejects_bad_rotary_dim(fasa, rotary_dim):
    st, detail = fasa.raw_create(1, 2, 1, 64, 128, 1e4, 1, [[0], [1]], 1, 8,
                                 rotary_dim=rotary_dim)
    assert st == -1 and "rotary_dim" in detail, (st, detail)


@pytest.mark.parametrize("buf,nbytes,sink", [
    (None, 64, 256),     # null buffer
    (256, 64, None),     # null sink
    (256, 0, 256),       # nothing to read
    (256, 40, 256),      # not a multiple of 16
    (264, 64, 256),      # misaligned buffer
])
def test_read_probe_rejects_bad_arguments(fasa, buf, nbytes, sink):
    """fasa_read_probe checks its arguments on the host and launches nothing
    when they are wrong (the addresses here are never dereferenced)."""
    import ctypes
    st = fasa._lib.fasa_read_probe(ctypes.c_void_p(buf), nbytes, ctypes.c_void_p(sink), None)
    assert st == -1, st
    assert fasa._lib.fasa_last_error().decode()


def _run_host_calls(env_extra):
    """A child process makes two host-only calls (one valid, one refused)."""
    code = ("import numpy as np, sparse_kv_cache_rope_amd as f\n"
            "ca = np.linspace(0, 1, 64, dtype=np.float32).reshape(2, 4, 8)\n"
            "f.select_dominant(ca, 2)\n"
            "try:\n    f.select_dominant(ca, 9)\nexcept Exception:\n    pass\n")
    env = dict(os.environ, **env_extra)
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                          text=True, check=True)


def test_call_log_off_by_default(fasa):
    r = _run_host_calls({"FASA_LOG": "0"})
    assert "fasa:" not in r.stderr


def test_call_log_lines(fasa):
    r = _run_host_calls({"FASA_LOG": "1"})
    lines = [ln for ln in r.stderr.splitlines() if ln.startswith("fasa:")]
    assert lines[0] == "fasa: fasa_select_dominant(samples=2 hq=4 n_fc=8 n_dom=2)"
    assert lines[1] == "fasa: fasa_select_dominant(samples=2 hq=4 n_fc=8 n_dom=9)"
    assert lines[2].startswith("fasa: fasa_select_dominant: error -1: sizes out of range")
    assert len(lines) == 3


def test_roctx_ranges_load_quietly(fasa):
    # The marker library loads on first use; a call with ranges on behaves
    # like one without.
    r = _run_host_calls({"FASA_ROCTX": "1", "FASA_LOG": "0"})
    assert "did not load" not in r.stderr
