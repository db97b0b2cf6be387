"""GPU parity of ssm_scan_fwd_conv (the prefill: causal depthwise convolution fused in front of
the scan) against the fp64 oracle (conv1d then scan, pinned against numpy.convolve and against the
decode step run token by token).

Covers every convolution width 1-4, with and without bias and an incoming register, every state
size, fp32 and bf16, ragged L and channel tiles, the segmented plan (segments read the three x rows
before them), a prefill continued by decode steps through ssm_state_update on the returned
register and state, and the layer shape on sampled channels. The returned register holds raw
inputs and is compared bit for bit."""
import numpy as np
import pytest
import torch

from selective_state_space_37_amd import inputs, ssm
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _conv_params(seed, Bsz, D, W, dtype, bias=True, history=True):
    w = inputs.draw_param(seed, 60, (D, W), scale=0.5)
    b = inputs.draw_param(seed, 61, (D,), scale=0.3) if bias else None
    reg = inputs.conv_register(seed, Bsz, D, W, dtype) if history else None
    return w, b, reg


def _check(inp, w, b, reg, segment_len=0, channels=None):
    y, hl, r = gu.scan_conv_on_gpu(inp, w, b, reg, segment_len=segment_len)
    ry, rh, rr = gu.scan_conv_oracle(inp, w, b, reg, channels=channels)
    if channels is not None:
        y, hl = y[:, :, channels], hl[:, channels]
        r = None if r is None else r[:, channels]
    err = max(gu.rel_err(y, ry), gu.rel_err(hl, rh))
    print("err %.3e" % err)
    assert err <= gu.TOL[inp.dtype]
    # the register is a copy of raw inputs: exact (none is returned without one)
    if reg is None:
        assert r is None
    else:
        assert np.array_equal(r, rr)


@pytest.mark.parametrize("W", [1, 2, 3, 4])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_conv_widths(W, dtype):
    inp = inputs.scan_small(seed=50 + W, Bsz=2, L=100, D=136, dtype=dtype, h0=True)
    _check(inp, *_conv_params(51 + W, 2, 136, W, dtype))


@pytest.mark.parametrize("N", [1, 2, 4, 8])
def test_conv_state_sizes(N):
    inp = inputs.scan_small(seed=60 + N, Bsz=2, L=77, D=72, N=N, h0=True)
    _check(inp, *_conv_params(61 + N, 2, 72, 4, "f32"))


@pytest.mark.parametrize("opts", [dict(bias=False), dict(history=False), dict(bias=False, history=False)])
def test_conv_optional(opts):
    inp = inputs.scan_small(seed=70, Bsz=2, L=64, D=40)
    _check(inp, *_conv_params(71, 2, 40, 4, "f32", **opts))


def test_conv_short_sequence():
    # L < W: the register keeps part of the incoming one
    inp = inputs.scan_small(seed=72, Bsz=2, L=2, D=40)
    _check(inp, *_conv_params(73, 2, 40, 4, "f32"))


@pytest.mark.parametrize("seg", [16, 48, 333])
def test_conv_segmented(seg):
    inp = inputs.scan_small(seed=74, Bsz=2, L=1000, D=72, h0=True)
    _check(inp, *_conv_params(75, 2, 72, 4, "f32"), segment_len=seg)


def test_prefill_then_decode():
    """One sequence split into a fused prefill and decode steps on the returned register and
    state equals the oracle over the whole sequence."""
    Bsz, L, K, D, N, W = 2, 96, 12, 64, 16, 4
    full = inputs.scan_small(seed=76, Bsz=Bsz, L=L + K, D=D, dtype="bf16")
    w, b, reg0 = _conv_params(77, Bsz, D, W, "bf16")
    pre = inputs.ScanInputs(dtype="bf16", x=full.x[:, :L], delta=full.delta[:, :L], A=full.A,
                            Bm=full.Bm[:, :L], Cm=full.Cm[:, :L], delta_bias=full.delta_bias,
                            delta_softplus=True, Dskip=full.Dskip, z=full.z[:, :L])
    regd = gu.dev(reg0)
    y, hl = ssm.scan_fwd_conv(gu.dev(pre.x), gu.dev(pre.delta), gu.dev(pre.A), gu.dev(pre.Bm),
                              gu.dev(pre.Cm), gu.dev(w), conv_b=gu.dev(b), conv_state=regd,
                              delta_bias=gu.dev(pre.delta_bias), delta_softplus=True,
                              Dskip=gu.dev(pre.Dskip), z=gu.dev(pre.z))
    ys = [gu.host(y)]
    A, Dk, cw, cb = gu.dev(full.A), gu.dev(full.Dskip), gu.dev(w), gu.dev(b)
    bias = gu.dev(full.delta_bias)
    for t in range(L, L + K):
        yt = ssm.state_update(gu.dev(np.ascontiguousarray(full.x[:, t])), gu.dev(np.ascontiguousarray(full.delta[:, t])),
                              A, gu.dev(np.ascontiguousarray(full.Bm[:, t])), gu.dev(np.ascontiguousarray(full.Cm[:, t])),
                              hl, delta_bias=bias, delta_softplus=True, Dskip=Dk,
                              z=gu.dev(np.ascontiguousarray(full.z[:, t])), conv_state=regd, conv_w=cw, conv_b=cb)
        ys.append(gu.host(yt)[:, None])
    torch.cuda.synchronize()
    ry, rh, rr = gu.scan_conv_oracle(full, w, b, reg0)
    err = max(gu.rel_err(np.concatenate(ys, axis=1), ry), gu.rel_err(gu.host(hl), rh))
    print("prefill+decode err %.3e" % err)
    assert err <= gu.TOL["bf16"]
    assert np.array_equal(gu.host(regd), rr)


def test_conv_layer_full_size_sampled():
    inp = inputs.scan_layer(seed=1)
    Bsz, L, D, N = inp.shape
    w, b, reg = _conv_params(78, Bsz, D, 4, "bf16")
    ch = np.sort(np.random.default_rng(6).choice(D, 48, replace=False))
    _check(inp, w, b, reg, channels=ch)
