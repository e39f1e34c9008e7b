"""sv_verify_noalloc (the entry point for callers that cannot allocate) against
sv_verify, through the C ABI: identical outputs on two calls in a row, the
second with a smaller input (the static scratch keeps the first call's
contents, which the second must not see), and the size limit."""
import ctypes

import numpy as np
import pytest

from rejection_sampling_verify_sv_amd import _lib, workloads

pytestmark = pytest.mark.gpu


def _cfg(B, K, V, code, stream, ws=None, ws_bytes=0, diag=None):
    c = _lib.SvConfig()
    c.batch, c.max_draft, c.vocab, c.dtype = B, K, V, code
    c.target_row_stride = c.draft_row_stride = 0
    c.stream = stream
    c.workspace = ws
    c.workspace_bytes = ws_bytes
    c.diag = diag
    return c


def _run(lib, entry, wl, dev, with_workspace):
    import torch

    t, d, tok, dl, prm, uni = workloads.to_torch(wl, dev)
    B, K, V = wl.B, wl.K, wl.V
    code = _lib.SV_F32 if wl.dtype == "f32" else _lib.SV_BF16
    out_tok = torch.full((B, K + 1), -7, dtype=torch.int32, device=dev)
    out_acc = torch.full((B,), -7, dtype=torch.int32, device=dev)
    dg = torch.empty((B, K + 1, 4), dtype=torch.float64, device=dev)
    ws, nbytes = None, 0
    if with_workspace:
        nbytes = lib.sv_workspace_bytes(B, K, V, code)
        wbuf = torch.empty(nbytes + 256, dtype=torch.uint8, device=dev)
        ws = wbuf.data_ptr() + (-wbuf.data_ptr()) % 256
    st = torch.cuda.current_stream(dev).cuda_stream
    cfg = _cfg(B, K, V, code, st, ws, nbytes, dg.data_ptr())
    torch.cuda.synchronize()
    rc = entry(t.data_ptr(), d.data_ptr(), tok.data_ptr(), dl.data_ptr(), prm.data_ptr(),
               uni.data_ptr(), out_tok.data_ptr(), out_acc.data_ptr(), ctypes.byref(cfg))
    assert rc == 0, lib.sv_strerror(rc)
    torch.cuda.synchronize()
    return out_tok.cpu().numpy(), out_acc.cpu().numpy(), dg.cpu().numpy()


@pytest.fixture(scope="module")
def lib():
    import torch

    assert torch.cuda.is_available(), "GPU tests need cuda:0"
    lib = _lib.load()
    lib.sv_verify_noalloc.restype = ctypes.c_int
    lib.sv_verify_noalloc.argtypes = [ctypes.c_void_p] * 8 + [ctypes.POINTER(_lib.SvConfig)]
    lib.sv_noalloc_scratch_bytes.restype = ctypes.c_size_t
    return lib


def test_noalloc_matches_verify_twice(lib):
    import torch

    dev = torch.device("cuda:0")
    # a large call (every sampler class, nucleus rows included), then smaller
    # ones of other shapes on the same scratch: 1500 short rows (the plan's
    # rows over several workgroups, one unit per wave in the row pass), and
    # a small bf16 batch
    cases = [workloads.make("mixed_samplers_b1024", batch=256, vocab=60013),
             workloads.make("tiny_v1000", batch=1500),
             workloads.make("mixed_greedy_b64", batch=24, vocab=20011)]
    for wl in cases:
        print(f"[gpu] noalloc {wl.name} B={wl.B} K={wl.K} V={wl.V} {wl.dtype}", flush=True)
        ref = _run(lib, lib.sv_verify, wl, dev, True)
        got = _run(lib, lib.sv_verify_noalloc, wl, dev, False)
        for a, b in zip(ref, got):
            assert np.array_equal(a, b, equal_nan=True)
        assert (got[1] >= 0).all()


def test_noalloc_rejects_shapes_beyond_its_scratch(lib):
    cap = lib.sv_noalloc_scratch_bytes()
    assert cap == 128 << 20
    # a shape whose workspace exceeds the static scratch: refused before any
    # launch, with its own error code
    B, K, V = 4096, 3, 151936
    assert lib.sv_workspace_bytes(B, K, V, 0) > cap
    cfg = _cfg(B, K, V, 0, None)
    dummy = ctypes.c_void_p(0x1000)
    rc = lib.sv_verify_noalloc(*([dummy] * 8), ctypes.byref(cfg))
    assert rc == -4
    assert b"scratch" in lib.sv_strerror(rc)
