"""ssm_scan_fwd_noalloc (the allocation-free scan: segment carries in the library's static
scratch) against ssm_scan_fwd with a caller workspace, through the C ABI, on long, narrow inputs
whose automatic plan splits L into segments (so the scratch is used): two calls in a row, the
second smaller, each bit-equal to the workspace entry point (same plan, same kernels)."""
import ctypes

import numpy as np
import pytest
import torch

from selective_state_space_37_amd import inputs, ssm
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

SCRATCH = 4 << 20


def _run(lib, inp, noalloc):
    d = {k: gu.dev(getattr(inp, k)) for k in ("x", "delta", "A", "Bm", "Cm", "delta_bias", "Dskip", "z", "h0")}
    Bsz, L, D, N = inp.shape
    io = ssm.SSM_F32 if inp.dtype == "f32" else ssm.SSM_BF16
    y = torch.empty_like(d["x"])
    hl = torch.empty((Bsz, D, N), dtype=torch.float32, device="cuda")
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    args = [Bsz, L, D, N, io, p(d["x"]), p(d["delta"]), p(d["delta_bias"]), int(inp.delta_softplus), p(d["A"]),
            p(d["Bm"]), p(d["Cm"]), p(d["Dskip"]), p(d["z"]), p(d["h0"]), p(y), p(hl)]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if noalloc:
        st = lib.ssm_scan_fwd_noalloc(*args, stream)
    else:
        nb = lib.ssm_scan_fwd_workspace_bytes(Bsz, L, D, N, io)
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
        st = lib.ssm_scan_fwd(*args, p(ws), nb, stream)
    assert st == 0, lib.ssm_last_error_detail()
    torch.cuda.synchronize()
    return gu.host(y), gu.host(hl)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_noalloc_equals_workspace_entry(dtype):
    lib = ssm.load()
    for seed, L, D in ((70, 65536, 64), (71, 20000, 32)):   # second call smaller
        inp = inputs.scan_small(seed=seed, Bsz=1, L=L, D=D, N=16, dtype=dtype, h0=True)
        nb = lib.ssm_scan_fwd_workspace_bytes(1, L, D, 16, ssm.SSM_F32 if dtype == "f32" else ssm.SSM_BF16)
        assert 0 < nb <= SCRATCH   # a segmented plan: the scratch is in use
        y0, h0 = _run(lib, inp, noalloc=False)
        y1, h1 = _run(lib, inp, noalloc=True)
        assert np.isfinite(y1).all() and np.isfinite(h1).all()
        assert np.array_equal(y0, y1) and np.array_equal(h0, h1)
        print("noalloc L %d D %d (%s): %d bytes of scratch, bit-equal" % (L, D, dtype, nb))


def test_noalloc_empty_sequence():
    lib = ssm.load()
    # L == 0: h_last receives h0 (by a kernel, no memory-set node)
    h0 = torch.randn(2, 64, 16, device="cuda")
    hl = torch.full_like(h0, 7.0)
    st = lib.ssm_scan_fwd_noalloc(2, 0, 64, 16, ssm.SSM_F32, None, None, None, 0,
                                  ctypes.c_void_p(torch.empty(64 * 16, device="cuda").data_ptr()), None, None, None,
                                  None, ctypes.c_void_p(h0.data_ptr()), None, ctypes.c_void_p(hl.data_ptr()),
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(hl, h0)
