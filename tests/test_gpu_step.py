"""GPU parity of ssm_state_update (one decode token) against the fp64 oracle, and the decode
workload end to end: a raw 2,048-token prompt through the fused-convolution prefill
(ssm_scan_fwd_conv), then 128 single-token steps at batch 128, d_inner 4096, N = 16, bf16 with
float32 state, every output and state compared on all channels."""
import numpy as np
import pytest
import torch

import oracle
from selective_state_space_37_amd import inputs, ssm
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("conv", [True, False])
def test_step_matches_oracle(dtype, N, conv):
    Bsz, D, W, seed = 3, 136, 4, 40 + N
    prm = inputs.decode_params(seed=seed, D=D, N=N, W=W)
    h0 = inputs.draw_param(seed, 50, (Bsz, D, N), scale=0.5)
    bias = inputs.draw_param(seed, 51, (D,), scale=0.3)
    cb = inputs.draw_param(seed, 52, (D,), scale=0.1)
    reg = inputs.conv_register(seed, Bsz, D, W, dtype) if conv else None
    st = inputs.decode_step(seed, 0, Bsz, D, N, dtype)
    h = gu.dev(h0)
    creg = gu.dev(reg) if conv else None
    y = gu.step_on_gpu(st, gu.dev(prm["A"]), h, Dskip=gu.dev(prm["Dskip"]), conv_state=creg,
                       conv_w=gu.dev(prm["conv_w"]) if conv else None, conv_b=gu.dev(cb) if conv else None,
                       delta_bias=gu.dev(bias), delta_softplus=True)
    torch.cuda.synchronize()
    w = lambda a: inputs.widen(a, dtype)
    ry, rh, rc = oracle.step(w(st.x), w(st.delta), prm["A"], w(st.Bm), w(st.Cm), h0,
                             delta_bias=bias, delta_softplus=True, Dskip=prm["Dskip"], z=w(st.z),
                             conv_state=w(reg) if conv else None, conv_w=prm["conv_w"] if conv else None,
                             conv_b=cb if conv else None)
    tol = gu.TOL[dtype]
    assert gu.rel_err(gu.host(y), ry) <= tol
    assert gu.rel_err(gu.host(h), rh) <= tol
    if conv:  # the register holds stored inputs: exact
        assert np.array_equal(gu.host(creg), rc)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [4, 16])
@pytest.mark.parametrize("W", [1, 2, 3, 5, 8])
def test_step_conv_widths(W, N, dtype):
    """Conv registers of every supported width (the width-4 path has its own vector loads; the
    others take the general one). D = 100 leaves a ragged last workgroup."""
    Bsz, D, seed = 2, 100, 70 + W
    prm = inputs.decode_params(seed=seed, D=D, N=N, W=W)
    h0 = inputs.draw_param(seed, 50, (Bsz, D, N), scale=0.5)
    cb = inputs.draw_param(seed, 52, (D,), scale=0.1)
    reg = inputs.conv_register(seed, Bsz, D, W, dtype)
    st = inputs.decode_step(seed, 0, Bsz, D, N, dtype)
    h, creg = gu.dev(h0), gu.dev(reg)
    y = gu.step_on_gpu(st, gu.dev(prm["A"]), h, Dskip=gu.dev(prm["Dskip"]), conv_state=creg,
                       conv_w=gu.dev(prm["conv_w"]), conv_b=gu.dev(cb), delta_softplus=True)
    torch.cuda.synchronize()
    w = lambda a: inputs.widen(a, dtype)
    ry, rh, rc = oracle.step(w(st.x), w(st.delta), prm["A"], w(st.Bm), w(st.Cm), h0,
                             delta_softplus=True, Dskip=prm["Dskip"], z=w(st.z), conv_state=w(reg),
                             conv_w=prm["conv_w"], conv_b=cb)
    tol = gu.TOL[dtype]
    assert gu.rel_err(gu.host(y), ry) <= tol
    assert gu.rel_err(gu.host(h), rh) <= tol
    assert np.array_equal(gu.host(creg), rc)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [2, 16])
def test_step_optional_inputs_absent(N, dtype):
    """No gate, no D term, no step-size bias, no conv bias, no softplus: the kernel reads stand-in
    addresses for absent tensors and must drop those values."""
    Bsz, D, W, seed = 3, 72, 4, 80 + N
    prm = inputs.decode_params(seed=seed, D=D, N=N, W=W)
    h0 = inputs.draw_param(seed, 50, (Bsz, D, N), scale=0.5)
    reg = inputs.conv_register(seed, Bsz, D, W, dtype)
    st = inputs.decode_step(seed, 0, Bsz, D, N, dtype)
    h, creg = gu.dev(h0), gu.dev(reg)
    y = ssm.state_update(gu.dev(st.x), gu.dev(st.delta), gu.dev(prm["A"]), gu.dev(st.Bm), gu.dev(st.Cm), h,
                         conv_state=creg, conv_w=gu.dev(prm["conv_w"]))
    torch.cuda.synchronize()
    w = lambda a: inputs.widen(a, dtype)
    ry, rh, _ = oracle.step(w(st.x), w(st.delta), prm["A"], w(st.Bm), w(st.Cm), h0,
                            conv_state=w(reg), conv_w=prm["conv_w"])
    tol = gu.TOL[dtype]
    assert gu.rel_err(gu.host(y), ry) <= tol
    assert gu.rel_err(gu.host(h), rh) <= tol


def test_repeated_steps_equal_scan():
    """L decode steps without the conv register equal one scan over the L tokens."""
    inp = inputs.scan_small(seed=60, Bsz=2, L=37, D=64, h0=True)
    y_scan, h_scan = gu.scan_on_gpu(inp)
    h = gu.dev(inp.h0).clone()
    A = gu.dev(inp.A)
    ys = []
    for t in range(inp.x.shape[1]):
        y = ssm.state_update(gu.dev(inp.x[:, t]), gu.dev(inp.delta[:, t]), A, gu.dev(inp.Bm[:, t]),
                             gu.dev(inp.Cm[:, t]), h, delta_bias=gu.dev(inp.delta_bias),
                             delta_softplus=True, Dskip=gu.dev(inp.Dskip), z=gu.dev(inp.z[:, t]))
        ys.append(gu.host(y))
    torch.cuda.synchronize()
    assert gu.rel_err(np.stack(ys, axis=1), y_scan) <= 1e-5
    assert gu.rel_err(gu.host(h), h_scan) <= 1e-5


@pytest.mark.slow
def test_decode_workload_end_to_end():
    """The generation workload end to end at batch 128, d_inner 4096, N 16, bf16 I/O, float32 state
    ("Mamba and state space models", section "how much faster": a 2,048-token prompt, then 128
    generated tokens). The raw prompt goes through the prefill (ssm_scan_fwd_conv: the decode
    register's width-4 causal convolution fused in front of the scan) from an empty register, which
    returns the state and the register; then 128 ssm_state_update steps with fresh inputs carry
    both. Every prefill output, the prefill's state and register, every step's output, and the final
    state and register are compared with the oracle on all channels (the prefill oracle over channel
    blocks)."""
    Bsz, L, D, N, W, seed, steps = 128, 2048, 4096, 16, 4, 3, 128
    prm = inputs.decode_params(seed=seed, D=D, N=N, W=W)
    pre = inputs.scan_layer(seed=seed, Bsz=Bsz, L=L, D=D, N=N)
    creg = gu.dev(np.zeros((Bsz, D, W), np.uint16))           # empty register (bf16 zeros)
    y_pre, h = ssm.scan_fwd_conv(gu.dev(pre.x), gu.dev(pre.delta), gu.dev(pre.A), gu.dev(pre.Bm), gu.dev(pre.Cm),
                                 gu.dev(prm["conv_w"]), conv_state=creg, Dskip=gu.dev(pre.Dskip), z=gu.dev(pre.z))
    torch.cuda.synchronize()
    yh, hh, regh = gu.host(y_pre), gu.host(h), gu.host(creg)
    del y_pre
    w = lambda a: inputs.widen(a, "bf16")
    ay, ah = gu.Accum(), gu.Accum()
    rh = np.empty((Bsz, D, N), np.float64)
    rreg = np.empty((Bsz, D, W), np.float64)
    for c0 in range(0, D, 512):
        ch = slice(c0, c0 + 512)
        ry, rh[:, ch], rreg[:, ch] = oracle.scan_conv(
            w(pre.x[:, :, ch]), w(pre.delta[:, :, ch]), pre.A[ch], w(pre.Bm), w(pre.Cm), prm["conv_w"][ch],
            Dskip=pre.Dskip[ch], z=w(pre.z[:, :, ch]))
        ay.add(yh[:, :, ch], ry)
        ah.add(hh[:, ch], rh[:, ch])
    del pre, yh
    print("prefill 128x2048x4096: y err %.3e (%s), h err %.3e" % (ay.err(), ay.diag(), ah.err()))
    assert ay.err() <= gu.TOL["bf16"] and ah.err() <= gu.TOL["bf16"]
    assert np.array_equal(regh, rreg)
    A, Dk, cw = gu.dev(prm["A"]), gu.dev(prm["Dskip"]), gu.dev(prm["conv_w"])
    astep = gu.Accum()
    for s in range(steps):
        st = inputs.decode_step(seed, s, Bsz, D, N, "bf16")
        y = gu.step_on_gpu(st, A, h, Dskip=Dk, conv_state=creg, conv_w=cw)
        ry, rh, rreg = oracle.step(w(st.x), w(st.delta), prm["A"], w(st.Bm), w(st.Cm), rh,
                                   Dskip=prm["Dskip"], z=w(st.z), conv_state=rreg, conv_w=prm["conv_w"])
        astep.add(gu.host(y), ry)
    torch.cuda.synchronize()
    eh = gu.rel_err(gu.host(h), rh)
    print("decode 128 steps: y err %.3e (%s), final h err %.3e" % (astep.err(), astep.diag(), eh))
    assert astep.err() <= gu.TOL["bf16"] and eh <= gu.TOL["bf16"]
    assert np.array_equal(gu.host(creg), rreg)
