"""GPU parity of ssd_chunk_bwd (the Mamba-2 layer's gradients) against the fp64 oracle's reverse
mode, itself pinned by finite differences of the forward oracle and by the scan backward.

Every gradient (dx, ddelta, dz, dA, dB, dC, dD, dbias, dh0) is compared with the forward's metric
and bf16 bar. Sizes span several 64-token chunks with ragged tails, both state sizes, grouped B
and C, per-head and per-channel D, the optional inputs, short sequences, run-to-run bit equality,
and a full-size layer on sampled heads."""
import numpy as np
import pytest

from selective_state_space_37_amd import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _run(inp, seed=7, dh_last=True, heads=None):
    Bsz, L, H, P, N = inp.shape
    dy, dhl = inputs.ssd_grads(seed, Bsz, L, H, P, N, dh_last=dh_last)
    gpu = gu.ssd_bwd_on_gpu(inp, dy, dhl)
    ref = gu.ssd_bwd_oracle(inp, dy, dhl, heads=heads)
    return gu.ssd_bwd_errors(gpu, ref, heads=heads), gpu


def _check(errs):
    print({k: "%.2e" % v for k, v in errs.items()})
    bad = {k: v for k, v in errs.items() if not v <= gu.TOL["bf16"]}
    assert not bad, bad


@pytest.mark.parametrize("N", [64, 128])
def test_ssd_bwd_ragged(N):
    # L = 150: two full 64-token chunks and a ragged one
    inp = inputs.ssd_layer(seed=90, Bsz=2, L=150, H=2, N=N, gate=True, dskip=True, h0=True)
    inp.delta_bias = np.array([0.3, -0.2], dtype=np.float32)
    inp.delta_softplus = True
    inp.delta = inputs.store(np.random.default_rng(2).standard_normal((2, 150, 2)).astype(np.float32) - 3.0, "bf16")
    errs, _ = _run(inp)
    _check(errs)


@pytest.mark.parametrize("G", [2, 4])
def test_ssd_bwd_groups_per_channel_d(G):
    inp = inputs.ssd_layer(seed=91, Bsz=1, L=200, H=4, N=64, gate=True, h0=True, groups=G,
                           dskip_per_channel=True)
    errs, _ = _run(inp, seed=8)
    _check(errs)


@pytest.mark.parametrize("opts", [dict(), dict(gate=True), dict(dskip=True), dict(h0=True)])
def test_ssd_bwd_optional_arguments(opts):
    inp = inputs.ssd_layer(seed=92, Bsz=1, L=130, H=2, N=64, **opts)
    errs, _ = _run(inp, seed=9, dh_last=False)
    _check(errs)


def test_ssd_bwd_short_sequences():
    for L in (1, 17, 64):
        inp = inputs.ssd_layer(seed=93, Bsz=2, L=L, H=2, N=128, gate=True, dskip=True, h0=True)
        errs, _ = _run(inp, seed=10)
        print("L", L)
        _check(errs)


def test_ssd_bwd_deterministic():
    inp = inputs.ssd_layer(seed=94, Bsz=2, L=300, H=4, N=64, gate=True, dskip=True, groups=2)
    dy, dhl = inputs.ssd_grads(11, 2, 300, 4, 64, 64)
    a = gu.ssd_bwd_on_gpu(inp, dy, dhl)
    b = gu.ssd_bwd_on_gpu(inp, dy, dhl)
    for k in gu.BWD_KEYS:
        if a.get(k) is not None:
            assert np.array_equal(a[k], b[k]), k


@pytest.mark.slow
def test_ssd_bwd_layer_full_size_sampled():
    """Mamba-2 layer, batch 2, L 8192, 80 heads x 64, N 128, bf16, 8 groups and per-channel D:
    sampled heads for every per-head gradient, and dB, dC of group 1 against all its heads."""
    inp = inputs.ssd_layer(seed=95, groups=8, gate=True, dskip_per_channel=True)
    Bsz, L, H, P, N = inp.shape
    dy, dhl = inputs.ssd_grads(12, Bsz, L, H, P, N)
    gpu = gu.ssd_bwd_on_gpu(inp, dy, dhl)
    heads = np.array([0, 9, 10, 39, 40, 79])
    errs = gu.ssd_bwd_errors(gpu, gu.ssd_bwd_oracle(inp, dy, dhl, heads=heads), heads=heads)
    _check(errs)


@pytest.mark.parametrize("H,G", [(8, 2), (8, 1), (16, 1)])
def test_ssd_bwd_head_blocks(H, G):
    """Heads per group a multiple of 4 and a grid too small for more: the main pass sums dB and dC
    over 4 heads per workgroup and the reduction adds the head blocks of a group (1, 2 and 4
    blocks per group here). The full-size case above takes 10 heads per workgroup."""
    inp = inputs.ssd_layer(seed=96 + H + G, Bsz=2, L=333, H=H, N=128, gate=True, dskip=True, h0=True,
                           groups=G if G > 1 else None)
    errs, _ = _run(inp, seed=13)
    _check(errs)
