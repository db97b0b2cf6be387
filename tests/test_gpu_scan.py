"""GPU parity of ssm_scan_fwd against the fp64 oracle (same seeded stored inputs).

Sizes span several 64-channel tiles and 16-token tiles with ragged tails, every supported state
size, the optional arguments, the segmented (long-sequence) plan at several segment lengths, the
oracle-sized workload, and the two full-size workloads (checked on sampled channels, which the
oracle computes one by one)."""
import ctypes

import numpy as np
import pytest
import torch

from selective_state_space_37_amd import inputs, ssm
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _case(seed=10, Bsz=2, L=100, D=136, N=16, dtype="f32", **kw):
    return inputs.scan_small(seed=seed, Bsz=Bsz, L=L, D=D, N=N, dtype=dtype, **kw)


def test_oracle_sized_fp32():
    inp = inputs.scan_small(seed=0)  # batch 1, L=256, D=64, N=16, fp32, gated
    err = gu.scan_parity(inp, gu.scan_on_gpu(inp))
    print("1x256x64x16 fp32 err", err)
    assert err <= gu.TOL["f32"]


def test_oracle_sized_bf16():
    inp = inputs.scan_small(seed=0, dtype="bf16")
    assert gu.scan_parity(inp, gu.scan_on_gpu(inp)) <= gu.TOL["bf16"]


@pytest.mark.parametrize("N", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_state_sizes_ragged(N, dtype):
    # D = 136: two full 64-channel tiles and an 8-channel tail; L = 100: ragged 16-token tail
    inp = _case(seed=11 + N, N=N, dtype=dtype, h0=True)
    err = gu.scan_parity(inp, gu.scan_on_gpu(inp))
    print("N", N, dtype, "err", err)
    assert err <= gu.TOL[dtype]


@pytest.mark.parametrize("opts", [
    dict(gate=False), dict(dskip=False), dict(gate=False, dskip=False), dict(h0=True)])
def test_optional_arguments(opts):
    inp = _case(seed=20, **opts)
    assert gu.scan_parity(inp, gu.scan_on_gpu(inp)) <= gu.TOL["f32"]


def test_no_bias_no_softplus():
    inp = _case(seed=21)
    inp.delta = np.abs(inp.delta) * 0.2 + 0.01
    inp.delta_bias = None
    inp.delta_softplus = False
    assert gu.scan_parity(inp, gu.scan_on_gpu(inp)) <= gu.TOL["f32"]


def test_no_final_state():
    inp = _case(seed=22)
    y, hl = gu.scan_on_gpu(inp, return_state=False)
    assert hl is None
    ry, _ = gu.scan_oracle(inp)
    assert gu.rel_err(y, ry) <= gu.TOL["f32"]


@pytest.mark.parametrize("seg", [16, 48, 100, 333, 1000])
def test_segmented_plan(seg):
    """Only state passes between segments: any split gives the oracle's result."""
    inp = _case(seed=23, Bsz=2, L=1000, D=72, h0=True)
    err = gu.scan_parity(inp, gu.scan_on_gpu(inp, segment_len=seg))
    print("segment", seg, "err", err)
    assert err <= gu.TOL["f32"]


@pytest.mark.parametrize("N", [1, 4, 8])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("seg", [37, 200])
def test_segmented_plan_small_states(N, dtype, seg):
    """The segmented plan for the smaller state sizes (64-channel tiles at N <= 4, element-wise
    B/C loads at N = 1 and 4 in bf16): segment ends that fall inside a 16-token tile, a ragged
    sequence end and a ragged channel tail (D = 136)."""
    inp = _case(seed=25 + N, Bsz=2, L=517, D=136, N=N, dtype=dtype, h0=True)
    err = gu.scan_parity(inp, gu.scan_on_gpu(inp, segment_len=seg))
    print("N", N, dtype, "segment", seg, "err", err)
    assert err <= gu.TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_segmented_correction_stops_early(dtype):
    """Large steps (0.05 .. 0.5): the entering state's part of the outputs falls below the
    output precision a few hundred tokens into each 1024-token segment, where the correction
    stops; outputs past that point and the final state still match the oracle."""
    inp = inputs.scan_steps(31, 2, 4096, 96, 16, dtype, 0.05, 0.5, h0=True)
    err = gu.scan_parity(inp, gu.scan_on_gpu(inp, segment_len=1024))
    print(dtype, "err", err)
    assert err <= gu.TOL[dtype]


def test_segmented_negative_steps():
    """Negative step sizes (no softplus) in some channels of one segment: the state can grow
    again along a segment, so those channels' correction runs to the segment end."""
    inp = inputs.scan_steps(32, 1, 3000, 136, 16, "f32", 0.05, 0.5, h0=True)
    d = inp.delta.copy()
    d[0, 1500:1520, 3:40] = -0.02
    inp.delta = d
    err = gu.scan_parity(inp, gu.scan_on_gpu(inp, segment_len=512))
    print("err", err)
    assert err <= gu.TOL["f32"]


def test_segmented_slow_state():
    """One state per channel that barely decays (A = -1e-4): its entering value stays visible
    over the whole segment, so the correction never stops early."""
    inp = inputs.scan_steps(33, 1, 2048, 64, 16, "f32", 0.01, 0.1, A_kind="random", h0=True)
    A = inp.A.copy()
    A[:, 5] = -1e-4
    inp.A = A
    err = gu.scan_parity(inp, gu.scan_on_gpu(inp, segment_len=400))
    print("err", err)
    assert err <= gu.TOL["f32"]


def test_segmented_zero_entering_state():
    """x = 0 and no h0: every entering state is zero and the correction adds nothing."""
    inp = _case(seed=34, Bsz=1, L=700, D=64)
    inp.x = np.zeros_like(inp.x)
    y, hl = gu.scan_on_gpu(inp, segment_len=160)
    ry, rh = gu.scan_oracle(inp)
    assert np.abs(y).max() == 0.0 and np.abs(ry).max() == 0.0
    assert np.abs(hl).max() == 0.0


def test_split_handoff_matches_whole():
    inp = _case(seed=24, Bsz=1, L=300, D=64, h0=True)
    y, hl = gu.scan_on_gpu(inp)
    L1 = 123
    first = inputs.ScanInputs(**{**inp.__dict__, "x": inp.x[:, :L1], "delta": inp.delta[:, :L1],
                                 "Bm": inp.Bm[:, :L1], "Cm": inp.Cm[:, :L1], "z": inp.z[:, :L1]})
    y1, h1 = gu.scan_on_gpu(first)
    second = inputs.ScanInputs(**{**inp.__dict__, "x": inp.x[:, L1:], "delta": inp.delta[:, L1:],
                                  "Bm": inp.Bm[:, L1:], "Cm": inp.Cm[:, L1:], "z": inp.z[:, L1:],
                                  "h0": h1.astype(np.float32)})
    y2, h2 = gu.scan_on_gpu(second)
    assert gu.rel_err(np.concatenate([y1, y2], axis=1), y) <= 1e-6
    assert gu.rel_err(h2, hl) <= 1e-6


def test_single_token_and_empty():
    inp = _case(seed=25, L=1, h0=True)
    assert gu.scan_parity(inp, gu.scan_on_gpu(inp)) <= gu.TOL["f32"]
    # L == 0: h_last receives h0; B == 0: no-op
    h0 = torch.randn(2, 64, 16, device="cuda")
    x = torch.empty(2, 0, 64, device="cuda")
    bc = torch.empty(2, 0, 16, device="cuda")
    y, hl = ssm.scan_fwd(x, x, torch.full((64, 16), -1.0, device="cuda"), bc, bc, h0=h0)
    torch.cuda.synchronize()
    assert y.shape == (2, 0, 64) and torch.equal(hl, h0)
    x0 = torch.empty(0, 5, 64, device="cuda")
    bc0 = torch.empty(0, 5, 16, device="cuda")
    y0, _ = ssm.scan_fwd(x0, x0, torch.full((64, 16), -1.0, device="cuda"), bc0, bc0)
    assert y0.shape == (0, 5, 64)


def test_final_state_in_place():
    """h_last may be the same buffer as h0."""
    inp = _case(seed=26, h0=True)
    lib = ssm.load()
    t = {k: gu.dev(getattr(inp, k)) for k in ("x", "delta", "A", "Bm", "Cm", "delta_bias", "Dskip", "z", "h0")}
    y = torch.empty_like(t["x"])
    Bsz, L, D, N = inp.shape
    st = lib.ssm_scan_fwd(Bsz, L, D, N, ssm.SSM_F32, *(ctypes.c_void_p(t[k].data_ptr()) for k in ("x", "delta", "delta_bias")),
                          1, *(ctypes.c_void_p(t[k].data_ptr()) for k in ("A", "Bm", "Cm", "Dskip", "z", "h0")),
                          ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(t["h0"].data_ptr()), None, 0,
                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    ry, rh = gu.scan_oracle(inp)
    assert gu.rel_err(gu.host(y), ry) <= gu.TOL["f32"]
    assert gu.rel_err(gu.host(t["h0"]), rh) <= gu.TOL["f32"]


def test_deterministic():
    inp = _case(seed=27, Bsz=2, L=700, D=128)
    a = gu.scan_on_gpu(inp, segment_len=128)
    b = gu.scan_on_gpu(inp, segment_len=128)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_causal():
    inp = _case(seed=28, L=200)
    y1, _ = gu.scan_on_gpu(inp)
    inp.x = inp.x.copy()
    inp.x[:, 150:] += 3.0
    y2, _ = gu.scan_on_gpu(inp)
    assert np.array_equal(y1[:, :150], y2[:, :150])


@pytest.mark.slow
def test_layer_full_size_bf16():
    """Mamba-2.8B-layer-shaped forward, 8 x 2048 x 5120, N = 16, bf16: the benchmark's workload,
    in the launch configuration the benchmark times; every output and final state against the
    oracle (run over channel blocks)."""
    inp = inputs.scan_layer()
    out = gu.scan_on_gpu(inp)
    ay, ah = gu.scan_parity_blocks(inp, out, 1280)
    print("layer 8x2048x5120 bf16 whole tensors: y err %.3e (%s), h_last err %.3e (%s)"
          % (ay.err(), ay.diag(), ah.err(), ah.diag()))
    assert ay.err() <= gu.TOL["bf16"] and ah.err() <= gu.TOL["bf16"]


@pytest.mark.slow
def test_long_narrow_full_size_fp32():
    """Long, narrow sequence, 1 x 1,048,576 x 256, N = 16, fp32: the automatic plan splits L
    into segments; every output and final state against the oracle over the whole length (run
    over channel blocks)."""
    inp = inputs.scan_long()
    out = gu.scan_on_gpu(inp)
    ay, ah = gu.scan_parity_blocks(inp, out, 64)
    print("long 1x1048576x256 fp32 whole tensors: y err %.3e (%s), h_last err %.3e (%s)"
          % (ay.err(), ay.diag(), ah.err(), ah.diag()))
    assert ay.err() <= gu.TOL["f32"] and ah.err() <= gu.TOL["f32"]
