"""The C ABI library loads and exports every function include/sv.h declares;
host-side argument checks reject bad input without touching a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "sv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sv_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    from rejection_sampling_verify_sv_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from rejection_sampling_verify_sv_amd import build
        build.build()
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) >= {"sv_verify", "sv_workspace_bytes", "sv_strerror"}
    for n in names:
        assert hasattr(lib, n), f"libsv.so does not export {n}"


def test_workspace_bytes_is_pure_and_validates(lib):
    from rejection_sampling_verify_sv_amd import _lib
    f = _lib.workspace_bytes
    assert f(1024, 3, 151936, 0) > 0
    assert f(1024, 3, 151936, 0) == f(1024, 3, 151936, 0)
    assert f(4, 0, 100, 0) > 0  # K = 0: a plain draw per row
    for bad in [(0, 3, 100, 0), (4, -1, 100, 0), (4, 1025, 100, 0), (4, 3, 1, 0), (4, 3, 100, 7)]:
        assert f(*bad) == 0


def test_verify_rejects_bad_arguments_on_host(lib):
    from rejection_sampling_verify_sv_amd import _lib
    cfg = _lib.SvConfig()
    cfg.batch, cfg.max_draft, cfg.vocab, cfg.dtype = 2, 1, 100, 0
    dummy = ctypes.c_void_p(0x1000)
    args = [dummy] * 8
    assert lib.sv_verify(*args, None) == -1           # no config
    bad = list(args)
    bad[0] = None
    assert lib.sv_verify(*bad, ctypes.byref(cfg)) == -1  # null target
    cfg.target_row_stride = 50                           # stride < V
    assert lib.sv_verify(*args, ctypes.byref(cfg)) == -1
    cfg.target_row_stride = 0
    cfg.workspace = None                                 # no workspace
    assert lib.sv_verify(*args, ctypes.byref(cfg)) == -2
    cfg.workspace = 0x1000
    cfg.workspace_bytes = 16
    assert lib.sv_verify(*args, ctypes.byref(cfg)) == -2
    assert b"workspace" in lib.sv_strerror(-2)
    assert lib.sv_strerror(0) == b"ok"


def test_sample_and_k0_reject_bad_arguments_on_host(lib):
    from rejection_sampling_verify_sv_amd import _lib
    cfg = _lib.SvConfig()
    cfg.batch, cfg.max_draft, cfg.vocab, cfg.dtype = 2, 1, 100, 0
    dummy = ctypes.c_void_p(0x1000)
    args = [dummy] * 8
    bad = list(args)
    bad[1] = None                                        # no draft with K = 1
    assert lib.sv_verify(*bad, ctypes.byref(cfg)) == -1
    cfg.max_draft = 0                                    # K = 0: draft may be NULL
    bad[2] = None
    assert lib.sv_verify(*bad, ctypes.byref(cfg)) == -2  # passes to the workspace check
    s_args = [dummy] * 5
    assert lib.sv_sample(*s_args, None) == -1            # no config
    s_bad = list(s_args)
    s_bad[0] = None                                      # no logits
    assert lib.sv_sample(*s_bad, ctypes.byref(cfg)) == -1
    cfg.max_draft = 7                                    # ignored by sv_sample
    assert lib.sv_sample(*s_args, ctypes.byref(cfg)) == -2
    s_bad = list(s_args)
    s_bad[4] = None                                      # status kept in the workspace
    assert lib.sv_sample(*s_bad, ctypes.byref(cfg)) == -2
    cfg.batch = 0
    assert lib.sv_sample(*s_args, ctypes.byref(cfg)) == -1
    # a position-by-position step: one launch pair per position
    per_position = lib.sv_launch_count(1024, 2, 1) - lib.sv_launch_count(1024, 1, 1)
    assert per_position == 2
    assert lib.sv_launch_count(1024, 0, 1) == lib.sv_launch_count(1024, 1, 1) - per_position
    # the automatic mode merges the last positions of a large batch: one pair
    # per position before the merge start, one for the rest (B (2 (K - d0) + 1)
    # units at most 3072): 1024 rows, K = 3 merge from position 2, 256 rows,
    # K = 4 from position 1; 1024 rows, K = 1 and 2048 rows, K = 2 do not merge
    assert lib.sv_launch_count(1024, 3, 0) == lib.sv_launch_count(1024, 3, 1) - per_position
    assert lib.sv_launch_count(256, 4, 0) == lib.sv_launch_count(256, 4, 1) - 3 * per_position
    assert lib.sv_launch_count(1024, 1, 0) == lib.sv_launch_count(1024, 1, 1)
    assert lib.sv_launch_count(2048, 2, 0) == lib.sv_launch_count(2048, 2, 1)
    # small batches take the dense step: one pair for every position
    assert lib.sv_launch_count(64, 4, 0) == lib.sv_launch_count(64, 0, 0) == 5
    assert lib.sv_launch_count(64, 4, 1) == 13 and lib.sv_launch_count(64, 4, 2) == 5
    assert lib.sv_launch_count(513, 0, 0) == 5 and lib.sv_launch_count(513, 1, 0) == 7
    assert lib.sv_launch_count(513, 1, 2) == 0  # dense is not served for that batch
    assert lib.sv_launch_count(4, 1, 7) == 0    # no such mode
    assert [lib.sv_launch_name(1, 1, 0, i) for i in range(5)] == [
        b"plan", b"rowpass", b"cut_decide", b"sample_sums", b"sample_pick"]
    assert lib.sv_launch_count(1, -1, 0) == 0 and lib.sv_launch_count(1, 1025, 0) == 0
    assert lib.sv_launch_count(0, 1, 0) == 0


def test_accept_stats_rejects_bad_arguments_on_host(lib):
    from rejection_sampling_verify_sv_amd import _lib
    cfg = _lib.SvConfig()
    cfg.batch, cfg.max_draft, cfg.vocab, cfg.dtype = 3, 0, 100, 0
    dummy = ctypes.c_void_p(0x1000)
    args = [dummy] * 4
    assert lib.sv_accept_stats(*args, None) == -1             # no config
    for i in range(4):                                        # every pointer is required
        bad = list(args)
        bad[i] = None
        assert lib.sv_accept_stats(*bad, ctypes.byref(cfg)) == -1
    assert lib.sv_accept_stats(*args, ctypes.byref(cfg)) == -2  # no workspace
    cfg.workspace = 0x100000
    cfg.workspace_bytes = lib.sv_workspace_bytes(3, 1, 100, 0)
    cfg.target_row_stride = 50                                # shorter than a row
    assert lib.sv_accept_stats(*args, ctypes.byref(cfg)) == -1
    cfg.target_row_stride = 0
    cfg.workspace_bytes -= 1
    assert lib.sv_accept_stats(*args, ctypes.byref(cfg)) == -2
    cfg.dtype = 7
    assert lib.sv_accept_stats(*args, ctypes.byref(cfg)) == -1


def test_verify_tree_rejects_bad_arguments_on_host(lib):
    from rejection_sampling_verify_sv_amd import _lib
    cfg = _lib.SvConfig()
    cfg.batch, cfg.max_draft, cfg.vocab, cfg.dtype = 2, 4, 100, 0
    d = ctypes.c_void_p(0x1000)
    args = [d] * 10
    assert lib.sv_verify_tree(*args, 2, 2, None) == -1          # no config
    assert lib.sv_verify_tree(*args, 5, 2, ctypes.byref(cfg)) == -1   # max_depth > K
    assert lib.sv_verify_tree(*args, -1, 2, ctypes.byref(cfg)) == -1  # max_depth < 0
    assert lib.sv_verify_tree(*args, 2, 0, ctypes.byref(cfg)) == -1   # max_children < 1
    assert lib.sv_verify_tree(*args, 2, 65, ctypes.byref(cfg)) == -1  # max_children > 64
    bad = list(args)
    bad[3] = None                                               # no parents with K > 0
    assert lib.sv_verify_tree(*bad, 2, 2, ctypes.byref(cfg)) == -1
    assert lib.sv_verify_tree(*args, 2, 2, ctypes.byref(cfg)) == -2   # no workspace
    # sv_verify_noalloc refuses shapes beyond its static scratch before any launch
    cfg.batch, cfg.max_draft, cfg.vocab = 4096, 3, 151936
    assert lib.sv_workspace_bytes(4096, 3, 151936, 0) > lib.sv_noalloc_scratch_bytes()
    assert lib.sv_verify_noalloc(*([d] * 8), ctypes.byref(cfg)) == -4
