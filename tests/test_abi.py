"""The C ABI library without a GPU: it loads, exports every declared entry point,
and its host-only validation answers with the documented error codes."""
import ctypes
import os
import re

import pytest

import causal_draft_correction_amd as dca
from causal_draft_correction_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "domino_head.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(domino_\w+)\s*\(", src)))


def test_header_declares_the_expected_entry_points():
    assert declared_functions() == sorted(dca.SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = dca.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_library_has_no_oracle_dependency():
    # the product library must not link or embed the oracle
    data = open(dca.LIB_PATH, "rb").read()
    assert b"oracle_draft_row" not in data and b"liboracle" not in data


def cfg(**kw):
    base = dict(d=64, h=32, r=16, V=100, K=16, max_batch=4, wdtype=dca.DOMINO_F32, flags=0,
                W1=16, W2=32, W_ih=48, W_hh=64, b_ih=None, b_hh=None, E=80)
    base.update(kw)
    c = binding.Config()
    for k, v in base.items():
        setattr(c, k, v)
    return c


def ws_size(c):
    n = ctypes.c_size_t()
    rc = dca.load_library().domino_head_workspace_size(ctypes.byref(c), ctypes.byref(n))
    return rc, n.value


def last_error():
    return dca.load_library().domino_last_error().decode()


def test_workspace_size_accepts_valid_config_and_grows_with_batch():
    rc, n1 = ws_size(cfg(max_batch=1))
    assert rc == 0 and n1 > 0 and n1 % 256 == 0
    rc, n8 = ws_size(cfg(max_batch=8))
    assert rc == 0 and n8 > n1


@pytest.mark.parametrize("kw,code", [
    (dict(K=0), -1), (dict(K=17), -1), (dict(max_batch=0), -1), (dict(max_batch=1025), -1), (dict(V=0), -1),
    (dict(d=12), -2), (dict(h=20), -2), (dict(r=12), -2), (dict(r=24), -2), (dict(wdtype=7), -2),
    (dict(wdtype=dca.DOMINO_BF16, r=4), -2), (dict(W2=None), -1), (dict(E=8), -1), (dict(flags=3), -1),
    (dict(flags=256), -1), (dict(flags=dca.MARKOV | dca.FOLD_EMBED), -1),
    (dict(flags=dca.MARKOV | dca.EXEC_STREAM_W2), -1),
])
def test_config_validation_codes(kw, code):
    rc, _ = ws_size(cfg(**kw))
    assert rc == code
    assert last_error() != ""


def test_fold_flag_adds_the_gate_table_to_the_workspace():
    rc, plain = ws_size(cfg(V=1000, h=32))
    rc2, folded = ws_size(cfg(V=1000, h=32, flags=dca.FOLD_EMBED))
    assert rc == rc2 == 0
    # the table (V x 3h float32) in, the unfolded launch's tagged input-gate words
    # (at most 8 rows x 3h x 8 bytes) out
    assert folded - plain >= 1000 * 3 * 32 * 4 - 8 * 3 * 32 * 8
    assert ws_size(cfg(flags=dca.FOLD_EMBED | dca.EXEC_PERSISTENT))[0] == 0


def test_markov_flag_adds_the_token_table_to_the_workspace():
    """The Markov head's table M [V, r] float32 lives in the workspace, plus a
    create-time region for one chunk of tokens."""
    rc, plain = ws_size(cfg(V=1000, h=32, r=16))
    rc2, mk = ws_size(cfg(V=1000, h=32, r=16, flags=dca.MARKOV))
    assert rc == rc2 == 0
    assert mk - plain >= 1000 * 16 * 4 + 1000 * 4 * 32 * 4


def test_param_count_closed_form():
    lib = dca.load_library()
    n = ctypes.c_int64()
    c = cfg(d=4096, h=1024, r=256, V=151936)
    assert lib.domino_head_param_count(ctypes.byref(c), ctypes.byref(n)) == 0
    assert n.value == 55_934_976
    c = cfg(d=4096, h=1024, r=256, V=151936, b_ih=96, b_hh=112)
    assert lib.domino_head_param_count(ctypes.byref(c), ctypes.byref(n)) == 0
    assert n.value == 55_934_976 + 6 * 1024


def test_create_rejects_missing_or_small_workspace():
    lib = dca.load_library()
    h = ctypes.c_void_p()
    c = cfg()
    assert lib.domino_head_create(ctypes.byref(c), None, 0, ctypes.byref(h)) == -3
    rc, need = ws_size(c)
    assert lib.domino_head_create(ctypes.byref(c), ctypes.c_void_p(4096), need - 256, ctypes.byref(h)) == -3
    assert lib.domino_head_create(ctypes.byref(c), ctypes.c_void_p(4096 + 16), need, ctypes.byref(h)) == -3


def test_accept_len_host_validation():
    lib = dca.load_library()
    assert lib.domino_accept_len(0, 16, None, None, None, None) == 0  # B = 0 is a no-op
    assert lib.domino_accept_len(-1, 16, None, None, None, None) == -1
    assert lib.domino_accept_len(4, 0, None, None, None, None) == -1
    assert lib.domino_accept_len(4, 17, None, None, None, None) == -1
    assert lib.domino_accept_len(4, 16, None, None, None, None) == -1
    assert lib.domino_accept_len(4, 16, ctypes.c_void_p(16), ctypes.c_void_p(32), ctypes.c_void_p(40), None) == -1


def test_null_handle_calls_fail_cleanly():
    lib = dca.load_library()
    assert lib.domino_head_draft(None, 1, None, None, None, None, None, None, None, None, None, None) == -1
    assert lib.domino_head_check_error(None, None) == -1
    assert lib.domino_head_set_spin_limit(None, 0) == -1
    lib.domino_head_destroy(None)


def test_binding_refuses_to_run_without_the_library(tmp_path, monkeypatch):
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        binding.load_library(str(tmp_path / "missing.so"))


def test_verify_workspace_size_and_host_validation():
    lib = dca.load_library()
    n = ctypes.c_size_t()
    assert lib.domino_verify_workspace_size(32, 16, 151936, ctypes.byref(n)) == 0
    assert n.value > 0 and n.value % 8 == 0
    assert lib.domino_verify_workspace_size(0, 16, 151936, ctypes.byref(n)) == 0 and n.value == 0
    assert dca.verify_workspace_size(1, 16, 151936) >= 17 * 8  # one key per target row at least
    assert lib.domino_verify_workspace_size(-1, 16, 100, ctypes.byref(n)) == -1
    assert lib.domino_verify_workspace_size(1, 0, 100, ctypes.byref(n)) == -1
    assert lib.domino_verify_workspace_size(1, 17, 100, ctypes.byref(n)) == -1
    assert lib.domino_verify_workspace_size(1, 4, 0, ctypes.byref(n)) == -1
    assert lib.domino_verify_workspace_size(1, 4, 100, None) == -1
    # host-side checks come before any device work
    assert lib.domino_verify(0, 16, 100, None, None, None, 0, None, None, None, None) == 0  # B = 0: no-op
    assert lib.domino_verify(1, 16, 100, None, 16, 32, 1024, None, 48, 64, None) == -1     # NULL logits
    assert lib.domino_verify(1, 16, 100, 16, 32, 48, 1024, None, 64, None, None) == -1     # NULL next
    assert lib.domino_verify(1, 16, 100, 18, 32, 48, 1024, None, 64, 80, None) == -1       # misaligned
    need = dca.verify_workspace_size(2, 16, 100)
    assert lib.domino_verify(2, 16, 100, 16, 32, 48, need - 8, None, 64, 80, None) == -3   # small workspace
    assert b"workspace" in lib.domino_last_error()
