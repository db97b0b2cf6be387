"""GPU parity of ssd_chunk_fwd (Mamba-2, scalar A per head) against the fp64 oracle's plain
recurrence: every chunk length (chunk-size invariance), both state sizes, ragged L, the optional
arguments, the state carried in and out, float32 I/O, and the full-size layer."""
import ctypes

import numpy as np
import pytest
import torch

from selective_state_space_37_amd import inputs, ssm
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("chunk", [64, 128, 256])
@pytest.mark.parametrize("N", [64, 128])
def test_chunk_sizes_ragged(chunk, N):
    inp = inputs.ssd_layer(seed=70, Bsz=2, L=600, H=3, N=N, gate=True, dskip=True, h0=True)
    err = gu.ssd_parity(inp, gu.ssd_on_gpu(inp, chunk=chunk))
    print("chunk", chunk, "N", N, "err", err)
    assert err <= gu.TOL["bf16"]


@pytest.mark.parametrize("opts", [dict(), dict(gate=True), dict(dskip=True), dict(h0=True)])
def test_optional_arguments(opts):
    inp = inputs.ssd_layer(seed=71, Bsz=1, L=512, H=2, **opts)
    assert gu.ssd_parity(inp, gu.ssd_on_gpu(inp)) <= gu.TOL["bf16"]


def test_softplus_and_bias():
    inp = inputs.ssd_layer(seed=72, Bsz=1, L=300, H=2, N=64)
    inp.delta = inputs.store(np.random.default_rng(1).standard_normal((1, 300, 2)).astype(np.float32) - 3.0, "bf16")
    inp.delta_bias = np.array([0.2, -0.4], dtype=np.float32)
    inp.delta_softplus = True
    assert gu.ssd_parity(inp, gu.ssd_on_gpu(inp, chunk=64)) <= gu.TOL["bf16"]


@pytest.mark.parametrize("chunk", [64, 128])
def test_initial_state_with_segments(chunk):
    """h0 with slow decays (A = -0.5 .. -4, small steps) and 64- or 128-token chunks: the state pass
    runs in L-segments (4 heads of one row: 8 segments), the first from h0 and the others from
    zero, so h0 must enter the composition once (through the first segment's end state). Counted
    twice, it adds about exp(a S) h0 again to the outputs of the second segment's chunks."""
    inp = inputs.ssd_layer(seed=79, Bsz=1, L=700, H=4, N=64, h0=True)
    inp.A = np.array([-0.5, -1.0, -2.0, -4.0], dtype=np.float32)
    err = gu.ssd_parity(inp, gu.ssd_on_gpu(inp, chunk=chunk))
    print("chunk", chunk, "err", err)
    assert err <= gu.TOL["bf16"]


@pytest.mark.parametrize("chunk", [64, 128])
def test_segments_with_head_runs_per_xcd(chunk):
    """16 heads of one row with the state pass in L-segments (16 chains: 8 segments): with the head
    count a multiple of 8 the segmented pass hands each XCD a run of adjacent heads (here 2 per run,
    not the identity order), so a head mapped twice or not at all would show in its outputs."""
    inp = inputs.ssd_layer(seed=81, Bsz=1, L=1024, H=16, N=64, gate=True, dskip=True, h0=True)
    err = gu.ssd_parity(inp, gu.ssd_on_gpu(inp, chunk=chunk))
    print("chunk", chunk, "err", err)
    assert err <= gu.TOL["bf16"]


def test_short_sequences():
    for L in (1, 17, 64):
        inp = inputs.ssd_layer(seed=73, Bsz=1, L=L, H=2, h0=True)
        assert gu.ssd_parity(inp, gu.ssd_on_gpu(inp, chunk=64)) <= gu.TOL["bf16"], L


def test_chunk_invariance_between_gpu_runs():
    inp = inputs.ssd_layer(seed=74, Bsz=1, L=1024, H=2, h0=True)
    outs = [gu.ssd_on_gpu(inp, chunk=q) for q in (64, 128, 256)]
    for y, hl in outs[1:]:
        assert gu.rel_err(y, outs[0][0]) <= gu.TOL["bf16"]
        assert gu.rel_err(hl, outs[0][1]) <= gu.TOL["bf16"]


@pytest.mark.parametrize("chunk", [64, 256])
@pytest.mark.parametrize("grouped", [False, True])
def test_float32_io(chunk, grouped):
    """float32 per-token tensors: x, z, B and C become bf16 copies in the workspace (the
    matrix-core operands), delta is read as float32 and y written as float32. The accuracy is
    that of bf16 operands, so the bar is the bf16 one."""
    inp = inputs.ssd_layer(seed=76, Bsz=2, L=700, H=4, N=128, dtype="f32", gate=True, dskip=not grouped, h0=True,
                           groups=2 if grouped else None, dskip_per_channel=grouped)
    y, hl = gu.ssd_on_gpu(inp, chunk=chunk)
    assert np.isfinite(y).all()
    err = gu.ssd_parity(inp, (y, hl))
    print("f32 io chunk", chunk, "grouped", grouped, "err", err)
    assert err <= gu.TOL["bf16"]


@pytest.mark.parametrize("chunk", [64, 256])
def test_float32_io_equals_bf16_io_on_bf16_values(chunk):
    """Inputs whose values are bf16 numbers, given once as float32 and once as bf16: the kernels
    see the same operands and step sizes, so y (float32: the widened bf16 result) and the final
    state agree bit for bit."""
    b16 = inputs.ssd_layer(seed=78, Bsz=2, L=700, H=4, N=128, gate=True, dskip=True, h0=True)
    f32 = inputs.ssd_layer(seed=78, Bsz=2, L=700, H=4, N=128, gate=True, dskip=True, h0=True)
    f32.dtype = "f32"
    for k in ("x", "delta", "Bm", "Cm", "z"):
        setattr(f32, k, inputs.widen(getattr(b16, k), "bf16").astype(np.float32))
    ya, ha = gu.ssd_on_gpu(b16, chunk=chunk)
    yb, hb = gu.ssd_on_gpu(f32, chunk=chunk)
    print("chunk", chunk, "max |dy|", np.abs(ya - yb).max(), "max |dh|", np.abs(ha - hb).max())
    assert np.array_equal(ya, yb) and np.array_equal(ha, hb)


def test_float32_io_step_sizes_kept_in_float32():
    """Large step sizes (softplus of N(0, 1) + 0.5, about 0.1 .. 3.5) with A = -16 on every other
    head: rounding each step size to bf16 would move the decay between neighbouring tokens by
    about |A| Delta 2^-9 (3 % at Delta = 1), past the bar; delta read in float32 stays within it."""
    inp = inputs.ssd_layer(seed=77, Bsz=1, L=512, H=2, N=64, dtype="f32", gate=True, dskip=True, h0=True)
    inp.delta = inputs.store(np.random.default_rng(7).standard_normal((1, 512, 2)), "f32")
    inp.delta_bias = np.full((2,), 0.5, dtype=np.float32)
    inp.delta_softplus = True
    inp.A = np.array([-16.0, -1.0], dtype=np.float32)
    y, hl = gu.ssd_on_gpu(inp, chunk=128)
    assert np.isfinite(y).all()
    err = gu.ssd_parity(inp, (y, hl))
    print("f32 io large steps err", err)
    assert err <= gu.TOL["bf16"]


def test_final_state_in_place():
    inp = inputs.ssd_layer(seed=75, Bsz=1, L=300, H=2, h0=True)
    t = {k: gu.dev(getattr(inp, k)) for k in ("x", "delta", "A", "Bm", "Cm", "h0")}
    y = torch.empty_like(t["x"])
    Bsz, L, H, P, N = inp.shape
    lib = ssm.load()
    nb = lib.ssd_chunk_fwd_workspace_bytes(Bsz, L, H, P, N, 128, ssm.SSM_BF16)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    p = lambda v: ctypes.c_void_p(v.data_ptr())
    st = lib.ssd_chunk_fwd(Bsz, L, H, P, N, 128, ssm.SSM_BF16, p(t["x"]), p(t["delta"]), None, 0, p(t["A"]),
                           p(t["Bm"]), p(t["Cm"]), None, None, p(t["h0"]), p(y), p(t["h0"]), p(ws), nb,
                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    ry, rh = gu.ssd_oracle(inp)
    assert gu.rel_err(gu.host(y), ry) <= gu.TOL["bf16"]
    assert gu.rel_err(gu.host(t["h0"]), rh) <= gu.TOL["bf16"]


@pytest.mark.slow
def test_layer_full_size():
    """Mamba-2 layer, batch 2, L 8192, 80 heads x 64, N 128, chunk 256, bf16: every output and
    final state against the oracle (run over blocks of heads)."""
    inp = inputs.ssd_layer()
    out = gu.ssd_on_gpu(inp, chunk=256)
    ay, ah = gu.ssd_parity_blocks(inp, out, 16)
    print("ssd 2x8192x80x64 N128 whole tensors: y err %.3e (%s), h_last err %.3e (%s)"
          % (ay.err(), ay.diag(), ah.err(), ah.diag()))
    assert ay.err() <= gu.TOL["bf16"] and ah.err() <= gu.TOL["bf16"]
