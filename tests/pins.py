"""Pins for the fp64 oracle: each check compares an oracle function with something fixed by the
pages or by mathematics -- never with a retyped copy of the oracle's own formula.

Each ``check_*`` takes the oracle callable(s) as arguments and returns the worst relative error,
so the same checks also run against deliberately broken copies of the oracle (the mutation
suite in ``test_oracle_pins.py``), which shows that each planted mistake fails at least one pin.

Pages cited (titles as given):
  [BA] "Beyond attention: exploring Mamba and state space models" -- continuous SSM, ZOH
       discretisation, recurrence/readout (state-space basics section); softplus step size and
       per-token B, C (selective SSM section).
  [MS] "Mamba and state space models" -- LTI convolution view ("every step the same"),
       Delta large resets / small keeps and Theorem 1 gate ("decided by the token"),
       fixed-size decode state with the last 4 inputs ("fixed-size state"), Mamba-2 matrix
       form ("Mamba-2: two algorithms").
"""
from __future__ import annotations

import numpy as np
import scipy.integrate
import scipy.linalg
import scipy.special

RNG = np.random.default_rng


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(float(np.max(np.abs(b))), 1e-300)
    return float(np.max(np.abs(a - b))) / scale


def tiny_scan_case(seed, Bsz=2, L=7, D=3, N=4, a_zero=True, softplus=True, gate=True, dskip=True,
                   h0=True):
    g = RNG(seed)
    A = -g.uniform(0.2, 3.0, (D, N))
    if a_zero:
        A[0, 1] = 0.0  # the a -> 0 limit of the ZOH scale
    case = dict(
        x=g.standard_normal((Bsz, L, D)),
        delta=g.standard_normal((Bsz, L, D)) * 0.7 if softplus else g.uniform(0.05, 0.8, (Bsz, L, D)),
        A=A,
        Bm=g.standard_normal((Bsz, L, N)),
        Cm=g.standard_normal((Bsz, L, N)),
        delta_bias=g.standard_normal(D) * 0.3 if softplus else None,
        delta_softplus=softplus,
        Dskip=g.standard_normal(D) if dskip else None,
        z=g.standard_normal((Bsz, L, D)) if gate else None,
        h0=g.standard_normal((Bsz, D, N)) if h0 else None,
    )
    return case


def _step_sizes(case):
    u = case["delta"] + (0.0 if case["delta_bias"] is None else case["delta_bias"][None, None, :])
    # softplus via numpy's logaddexp: log(e^0 + e^u)
    return np.logaddexp(0.0, u) if case["delta_softplus"] else u


def check_ode(scan, case):
    """[BA] continuous system h' = A h + B x held constant over each step of length Delta_t
    (zero-order hold), integrated numerically; y_t = C_t h(t) + D x_t, then the gate z*sigmoid(z).
    Pins the ZOH discretisation, the softplus step size, the recurrence, the readout, D and gate."""
    dt = _step_sizes(case)
    x, A, Bm, Cm = case["x"], case["A"], case["Bm"], case["Cm"]
    Bsz, L, D = x.shape
    N = A.shape[1]
    h = np.zeros((Bsz, D, N)) if case["h0"] is None else case["h0"].copy()
    y_ref = np.zeros((Bsz, L, D))
    for b in range(Bsz):
        for t in range(L):
            for d in range(D):
                drive = Bm[b, t, :] * x[b, t, d]
                a = A[d, :]
                sol = scipy.integrate.solve_ivp(lambda s, hh: a * hh + drive, (0.0, dt[b, t, d]),
                                                h[b, d, :], method="DOP853", rtol=1e-13, atol=1e-15)
                h[b, d, :] = sol.y[:, -1]
                out = float(Cm[b, t, :] @ h[b, d, :])
                if case["Dskip"] is not None:
                    out += case["Dskip"][d] * x[b, t, d]
                if case["z"] is not None:
                    zz = case["z"][b, t, d]
                    out *= zz * scipy.special.expit(zz)
                y_ref[b, t, d] = out
    y, h_last = scan(**case)
    return max(rel_err(y, y_ref), rel_err(h_last, h))


def _zoh_pair_expm(dt, a_vec, b_vec):
    """Abar, Bbar for diagonal A from the matrix exponential of [[dt A, dt B], [0, 0]]
    (Van Loan's block form of the zero-order hold), via scipy.linalg.expm."""
    N = len(a_vec)
    M = np.zeros((N + 1, N + 1))
    M[:N, :N] = dt * np.diag(a_vec)
    M[:N, N] = dt * b_vec
    E = scipy.linalg.expm(M)
    return np.diag(E[:N, :N]).copy(), E[:N, N].copy()


def check_lti_convolution(scan, seed=1, L=24, D=3, N=5):
    """[MS] 'every step the same': with Delta, B, C constant the output is the convolution of x
    with the kernel K_k = sum_n C_n Abar_n^k Bbar_n (plus D x), computed by O(L^2) brute force
    with Abar, Bbar from the matrix exponential."""
    g = RNG(seed)
    A = -g.uniform(0.1, 2.0, (D, N))
    dts = g.uniform(0.05, 0.6, D)
    Bc = g.standard_normal(N)
    Cc = g.standard_normal(N)
    x = g.standard_normal((1, L, D))
    Dp = g.standard_normal(D)
    delta = np.broadcast_to(dts[None, None, :], (1, L, D)).copy()
    Bm = np.broadcast_to(Bc[None, None, :], (1, L, N)).copy()
    Cm = np.broadcast_to(Cc[None, None, :], (1, L, N)).copy()
    y_ref = np.zeros((1, L, D))
    for d in range(D):
        Ab, Bb = _zoh_pair_expm(dts[d], A[d], Bc)
        K = np.array([np.sum(Cc * Ab ** k * Bb) for k in range(L)])
        for t in range(L):
            y_ref[0, t, d] = sum(K[k] * x[0, t - k, d] for k in range(t + 1)) + Dp[d] * x[0, t, d]
    y, _ = scan(x=x, delta=delta, A=A, Bm=Bm, Cm=Cm, Dskip=Dp)
    return rel_err(y, y_ref)


def check_theorem1_gate(scan, seed=2, L=50):
    """[MS] Theorem 1: one state, A = -1, B = C = 1, softplus step size: the update is the RNN gate
    h <- (1 - g) h + g x with g = sigmoid(delta)."""
    g = RNG(seed)
    x = g.standard_normal((1, L, 1))
    delta = g.standard_normal((1, L, 1)) * 2.0
    ones = np.ones((1, L, 1))
    y, _ = scan(x=x, delta=delta, A=-np.ones((1, 1)), Bm=ones, Cm=ones, delta_softplus=True)
    h = 0.0
    ref = np.zeros(L)
    for t in range(L):
        gt = scipy.special.expit(delta[0, t, 0])
        h = (1.0 - gt) * h + gt * x[0, t, 0]
        ref[t] = h
    return rel_err(y[0, :, 0], ref)


def check_zero_input_decay(scan, seed=3, L=40, D=3, N=6):
    """With x = 0 the state only decays: h_t = exp(A * sum_{s<=t} Delta_s) h0 and y_t = C_t . h_t."""
    g = RNG(seed)
    A = -g.uniform(0.1, 4.0, (D, N))
    delta = g.uniform(0.01, 0.3, (2, L, D))
    Cm = g.standard_normal((2, L, N))
    h0 = g.standard_normal((2, D, N))
    y, h_last = scan(x=np.zeros((2, L, D)), delta=delta, A=A, Bm=g.standard_normal((2, L, N)),
                     Cm=Cm, h0=h0)
    S = np.cumsum(delta, axis=1)                        # [2, L, D]
    h_t = np.exp(A[None, None] * S[..., None]) * h0[:, None]  # [2, L, D, N]
    y_ref = np.einsum("bln,bldn->bld", Cm, h_t)
    return max(rel_err(y, y_ref), rel_err(h_last, h_t[:, -1]))


def check_delta_limits(scan, seed=4, L=12, D=2, N=5):
    """[MS] Delta large resets the state to the current input: h_t = -B_t x_t / A.
    Delta tiny keeps the state: h_t = h0."""
    g = RNG(seed)
    A = -g.uniform(0.5, 3.0, (D, N))
    x = g.standard_normal((1, L, D))
    Bm = g.standard_normal((1, L, N))
    Cm = g.standard_normal((1, L, N))
    h0 = g.standard_normal((1, D, N))
    _, hl = scan(x=x, delta=np.full((1, L, D), 1e3), A=A, Bm=Bm, Cm=Cm, h0=h0)
    reset_ref = -Bm[0, -1][None, :] * x[0, -1][:, None] / A
    e1 = rel_err(hl[0], reset_ref)
    y2, hl2 = scan(x=x, delta=np.full((1, L, D), 1e-15), A=A, Bm=Bm, Cm=Cm, h0=h0)
    e2 = rel_err(hl2, h0)
    y2_ref = np.einsum("ln,dn->ld", Cm[0], h0[0])[None]
    return max(e1, e2, rel_err(y2, y2_ref))


def check_fixed_point(scan, seed=5, L=30, D=3, N=4):
    """Zero-order hold is exact for constant input: with x_t = x0, B_t = B0 and random Delta_t,
    the state h0 = -B0 x0 / A (the equilibrium of h' = A h + B x) never moves."""
    g = RNG(seed)
    A = -g.uniform(0.2, 5.0, (D, N))
    x0 = g.standard_normal(D)
    B0 = g.standard_normal(N)
    h0 = -(B0[None, :] * x0[:, None]) / A
    x = np.broadcast_to(x0[None, None, :], (1, L, D)).copy()
    Bm = np.broadcast_to(B0[None, None, :], (1, L, N)).copy()
    _, hl = scan(x=x, delta=g.uniform(0.001, 2.0, (1, L, D)), A=A, Bm=Bm,
                 Cm=g.standard_normal((1, L, N)), h0=h0[None])
    return rel_err(hl[0], h0)


def check_split_handoff(scan, seed=6, L=33, L1=14):
    """The state is the whole context: scanning L tokens equals scanning L1 tokens and then the
    remaining ones from the carried state."""
    c = tiny_scan_case(seed, L=L)
    y, hl = scan(**c)
    first = {k: (v[:, :L1] if k in ("x", "delta", "Bm", "Cm", "z") and v is not None else v)
             for k, v in c.items()}
    y1, h1 = scan(**first)
    second = {k: (v[:, L1:] if k in ("x", "delta", "Bm", "Cm", "z") and v is not None else v)
              for k, v in c.items()}
    second["h0"] = h1
    y2, h2 = scan(**second)
    return max(rel_err(np.concatenate([y1, y2], axis=1), y), rel_err(h2, hl))


def check_linearity_causality(scan, seed=7, L=20):
    """Before the gate the layer is linear in (x, h0) and causal."""
    c1 = tiny_scan_case(seed, L=L, gate=False)
    c2 = tiny_scan_case(seed + 100, L=L, gate=False)
    c2.update({k: c1[k] for k in ("delta", "A", "Bm", "Cm", "delta_bias", "Dskip")})
    a, b = 0.7, -1.3
    c3 = dict(c1)
    c3["x"] = a * c1["x"] + b * c2["x"]
    c3["h0"] = a * c1["h0"] + b * c2["h0"]
    y1, _ = scan(**c1)
    y2, _ = scan(**c2)
    y3, _ = scan(**c3)
    e_lin = rel_err(y3, a * y1 + b * y2)
    c4 = dict(c1)
    c4["x"] = c1["x"].copy()
    t0 = L // 2
    c4["x"][:, t0:] += 5.0
    y4, _ = scan(**c4)
    e_causal = rel_err(y4[:, :t0], y1[:, :t0])
    return max(e_lin, e_causal)


def check_gate_and_skip(scan, seed=8):
    """D adds D * x to each output; the gate multiplies the output by z * sigmoid(z)."""
    c = tiny_scan_case(seed, gate=False, dskip=False)
    y0, _ = scan(**c)
    cd = dict(c)
    cd["Dskip"] = RNG(seed + 1).standard_normal(c["x"].shape[2])
    yd, _ = scan(**cd)
    e1 = rel_err(yd - y0, cd["Dskip"][None, None, :] * c["x"])
    cz = dict(cd)
    cz["z"] = RNG(seed + 2).standard_normal(c["x"].shape) * 2.0
    yz, _ = scan(**cz)
    e2 = rel_err(yz, yd * cz["z"] * scipy.special.expit(cz["z"]))
    return max(e1, e2)


SCAN_CHECKS = [
    ("ode_zoh", lambda s: max(check_ode(s, tiny_scan_case(11)),
                              check_ode(s, tiny_scan_case(12, softplus=False, h0=False)))),
    ("lti_convolution", check_lti_convolution),
    ("theorem1_gate", check_theorem1_gate),
    ("zero_input_decay", check_zero_input_decay),
    ("delta_limits", check_delta_limits),
    ("fixed_point", check_fixed_point),
    ("split_handoff", check_split_handoff),
    ("linearity_causality", check_linearity_causality),
    ("gate_and_skip", check_gate_and_skip),
]
SCAN_TOL = {"ode_zoh": 1e-9}
DEFAULT_TOL = 1e-11


# ----------------------------------------------------------------------------- decode step
def check_step_equals_scan(step, scan, seed=20, L=9):
    """Without the conv register, L decode steps equal one scan over the L tokens."""
    c = tiny_scan_case(seed, L=L)
    y_scan, h_scan = scan(**c)
    h = c["h0"].copy()
    ys = []
    for t in range(L):
        y, h, _ = step(x=c["x"][:, t], delta=c["delta"][:, t], A=c["A"], Bm=c["Bm"][:, t],
                       Cm=c["Cm"][:, t], h=h, delta_bias=c["delta_bias"],
                       delta_softplus=c["delta_softplus"], Dskip=c["Dskip"], z=c["z"][:, t])
        ys.append(y)
    return max(rel_err(np.stack(ys, axis=1), y_scan), rel_err(h, h_scan))


def check_step_conv(step, scan, seed=21, L=11, W=4):
    """[MS] the decode state keeps the last 4 inputs: after each step the register holds the last W
    raw inputs, and the outputs equal a scan over the causal depthwise convolution of the raw
    inputs (numpy.convolve, zero history), with the convolution output as the SSM input."""
    c = tiny_scan_case(seed, L=L, h0=False)
    Bsz, _, D = c["x"].shape
    g = RNG(seed + 1)
    w = g.standard_normal((D, W))
    cb = g.standard_normal(D)
    u = np.zeros_like(c["x"])
    for b in range(Bsz):
        for d in range(D):
            # causal conv: u_t = sum_k w[d, W-1-k] x_{t-k}; numpy.convolve flips its second operand
            u[b, :, d] = np.convolve(c["x"][b, :, d], w[d, ::-1])[:L] + cb[d]
    cu = dict(c)
    cu["x"] = u
    y_ref, h_ref = scan(**cu)
    h = np.zeros((Bsz, D, c["A"].shape[1]))
    reg = np.zeros((Bsz, D, W))
    ys = []
    e_reg = 0.0
    for t in range(L):
        y, h, reg = step(x=c["x"][:, t], delta=c["delta"][:, t], A=c["A"], Bm=c["Bm"][:, t],
                         Cm=c["Cm"][:, t], h=h, delta_bias=c["delta_bias"],
                         delta_softplus=c["delta_softplus"], Dskip=c["Dskip"], z=c["z"][:, t],
                         conv_state=reg, conv_w=w, conv_b=cb)
        ys.append(y)
        hist = np.zeros((Bsz, D, W))
        for k in range(W):
            src = t - (W - 1) + k
            if src >= 0:
                hist[:, :, k] = c["x"][:, src]
        e_reg = max(e_reg, float(np.max(np.abs(reg - hist))))
    return max(rel_err(np.stack(ys, axis=1), y_ref), rel_err(h, h_ref), e_reg)


def check_conv_prefill(conv1d, scan_conv, step, seed=22, L=13, W=4):
    """The prefill's convolution is the decode state's convolution run over the sequence:
    (i) with zero history it is numpy.convolve of the raw inputs with the weights reversed;
    (ii) with a register of earlier inputs it equals the tail of the zero-history convolution of
        those inputs followed by the sequence (the register carries the history exactly);
    (iii) conv then scan equals L decode steps (the step oracle, pinned on its own) started from
        the same register and state, for y, the final state and the final register;
    (iv) with L < W the final register mixes the old register and the new inputs."""
    c = tiny_scan_case(seed, L=L)
    Bsz, _, D = c["x"].shape
    g = RNG(seed + 1)
    w = g.standard_normal((D, W))
    cb = g.standard_normal(D)
    hist = g.standard_normal((Bsz, D, W))
    e = 0.0
    u0, _ = conv1d(c["x"], w, conv_b=cb)
    ref = np.zeros_like(c["x"])
    for b in range(Bsz):
        for d in range(D):
            ref[b, :, d] = np.convolve(c["x"][b, :, d], w[d, ::-1])[:L] + cb[d]
    e = max(e, rel_err(u0, ref))
    u1, r1 = conv1d(c["x"], w, conv_b=cb, conv_state=hist)
    xx = np.concatenate([np.moveaxis(hist, 2, 1), c["x"]], axis=1)
    u2, r2 = conv1d(xx, w, conv_b=cb)
    e = max(e, rel_err(u1, u2[:, W:]), rel_err(r1, r2))
    y, hl, reg = scan_conv(conv_w=w, conv_b=cb, conv_state=hist, **c)
    h, rg = c["h0"].copy(), hist.copy()
    ys = []
    for t in range(L):
        yt, h, rg = step(x=c["x"][:, t], delta=c["delta"][:, t], A=c["A"], Bm=c["Bm"][:, t],
                         Cm=c["Cm"][:, t], h=h, delta_bias=c["delta_bias"],
                         delta_softplus=c["delta_softplus"], Dskip=c["Dskip"], z=c["z"][:, t],
                         conv_state=rg, conv_w=w, conv_b=cb)
        ys.append(yt)
    e = max(e, rel_err(y, np.stack(ys, axis=1)), rel_err(hl, h), rel_err(reg, rg))
    _, r3 = conv1d(c["x"][:, :2], w, conv_state=hist)
    want = np.concatenate([hist[:, :, 2:], np.moveaxis(c["x"][:, :2], 1, 2)], axis=2)
    e = max(e, rel_err(r3, want))
    return e


# ----------------------------------------------------------------------------- SSD
def tiny_ssd_case(seed, Bsz=2, L=20, H=2, P=3, N=4, gate=True, dskip=True, softplus=True, groups=None,
                  dskip_per_channel=False):
    g = RNG(seed)
    bc = (Bsz, L, N) if groups is None else (Bsz, L, groups, N)
    return dict(
        x=g.standard_normal((Bsz, L, H, P)),
        delta=g.standard_normal((Bsz, L, H)) * 0.6,
        A=-g.uniform(0.3, 4.0, H),
        Bm=g.standard_normal(bc),
        Cm=g.standard_normal(bc),
        delta_bias=g.standard_normal(H) * 0.2,
        delta_softplus=softplus,
        Dskip=(g.standard_normal((H, P)) if dskip_per_channel else g.standard_normal(H)) if dskip else None,
        z=g.standard_normal((Bsz, L, H, P)) if gate else None,
    )


def check_ssd_quadratic(ssd, ssd_quadratic, seed=30):
    """[MS] Mamba-2: the recurrence equals multiplication by the lower-triangular matrix."""
    e = 0.0
    for s, kw in ((seed, {}), (seed + 1, dict(gate=False, dskip=False, L=33, N=6, P=2)),
                  (seed + 2, dict(H=6, groups=3, dskip_per_channel=True)),
                  (seed + 3, dict(H=4, groups=4, L=17))):
        c = tiny_ssd_case(s, **kw)
        y, _ = ssd(**c)
        e = max(e, rel_err(y, ssd_quadratic(**c)))
    return e


def check_ssd_groups(ssd, seed=32):
    """G groups of heads each with their own B, C: every group's heads give the same outputs and
    states as a layer holding only those heads with that group's B, C shared by all of them; D per
    channel equals per-head D where it is constant over a head's channels."""
    c = tiny_ssd_case(seed, H=6, groups=3, dskip_per_channel=True)
    Bsz, L, H, P = c["x"].shape
    g = RNG(seed + 1)
    h0 = g.standard_normal((Bsz, H, P, c["Bm"].shape[3]))
    y, hl = ssd(h0=h0, **c)
    e = 0.0
    per = H // 3
    for grp in range(3):
        hs = slice(grp * per, (grp + 1) * per)
        cg = dict(c, x=c["x"][:, :, hs], delta=c["delta"][:, :, hs], A=c["A"][hs], Bm=c["Bm"][:, :, grp],
                  Cm=c["Cm"][:, :, grp], delta_bias=c["delta_bias"][hs], Dskip=c["Dskip"][hs], z=c["z"][:, :, hs])
        yg, hg = ssd(h0=h0[:, hs], **cg)
        e = max(e, rel_err(y[:, :, hs], yg), rel_err(hl[:, hs], hg))
    d1 = dict(c, Dskip=c["Dskip"][:, 0])
    d2 = dict(c, Dskip=np.repeat(c["Dskip"][:, :1], P, axis=1))
    e = max(e, rel_err(ssd(**d1)[0], ssd(**d2)[0]))
    return e


def check_ssd_equals_scan(ssd, scan, seed=31):
    """[MS] Mamba-2 restricts A to a scalar times the identity: the SSD layer equals the selective
    scan with A[d, n] = A_h and Delta[b, t, d] = Delta[b, t, h] for every channel d = (h, p)."""
    c = tiny_ssd_case(seed)
    Bsz, L, H, P = c["x"].shape
    N = c["Bm"].shape[2]
    g = RNG(seed + 5)
    h0 = g.standard_normal((Bsz, H, P, N))
    y, hl = ssd(h0=h0, **c)
    sc = dict(
        x=c["x"].reshape(Bsz, L, H * P),
        delta=np.repeat(c["delta"], P, axis=2),
        A=np.repeat(c["A"], P)[:, None] * np.ones((1, N)),
        Bm=c["Bm"], Cm=c["Cm"],
        delta_bias=np.repeat(c["delta_bias"], P),
        delta_softplus=c["delta_softplus"],
        Dskip=np.repeat(c["Dskip"], P),
        z=c["z"].reshape(Bsz, L, H * P),
        h0=h0.reshape(Bsz, H * P, N),
    )
    ys, hs = scan(**sc)
    return max(rel_err(y.reshape(Bsz, L, H * P), ys), rel_err(hl.reshape(Bsz, H * P, N), hs))


# ----------------------------------------------------------------------------- scan gradients
_GRAD_OF = (("x", "dx"), ("delta", "ddelta"), ("A", "dA"), ("Bm", "dBm"), ("Cm", "dCm"),
            ("Dskip", "dDskip"), ("delta_bias", "ddelta_bias"), ("z", "dz"), ("h0", "dh0"))


def _fd_loss(scan, case, dy, dh_last):
    y, hl = scan(**case)
    return float(np.sum(y * dy)) + (float(np.sum(hl * dh_last)) if dh_last is not None else 0.0)


def check_bwd_finite_differences(scan_bwd, scan, seed=40, eps=1e-6):
    """The gradients are the derivative of the forward map. For the loss
    sum(dy * y) + sum(dh_last * h_last), every gradient entry must equal the central difference
    (loss(v + eps) - loss(v - eps)) / (2 eps) of the forward oracle: brute force, accurate to about
    1e-9 relative at eps = 1e-6 in fp64. Cases: (i) softplus with bias, gate, D term, h0, dh_last
    and one A entry of exactly zero (the limit of the ZOH scale); (ii) plain Delta with none of the
    optional inputs -- there the gradients of the absent bias, D and h0 are compared with the
    differences taken at explicit zeros, where the forward map is the same."""
    worst = 0.0
    for k, kw in enumerate((dict(), dict(softplus=False, gate=False, dskip=False, h0=False, a_zero=False))):
        case = tiny_scan_case(seed + k, Bsz=2, L=6, D=3, N=3, **kw)
        g = RNG(seed + 10 + k)
        dy = g.standard_normal(case["x"].shape)
        dh_last = g.standard_normal((2, 3, 3)) if k == 0 else None
        grads = scan_bwd(dy=dy, dh_last=dh_last, **case)
        full = dict(case)
        Bsz, L, D = case["x"].shape
        N = case["A"].shape[1]
        for key, shape in (("delta_bias", (D,)), ("Dskip", (D,)), ("h0", (Bsz, D, N))):
            if full[key] is None:
                full[key] = np.zeros(shape)
        for key, gkey in _GRAD_OF:
            if full.get(key) is None:
                continue
            arr = full[key] = np.array(full[key], dtype=np.float64)
            fd = np.zeros_like(arr)
            for idx in np.ndindex(arr.shape):
                v = arr[idx]
                arr[idx] = v + eps
                lp = _fd_loss(scan, full, dy, dh_last)
                arr[idx] = v - eps
                lm = _fd_loss(scan, full, dy, dh_last)
                arr[idx] = v
                fd[idx] = (lp - lm) / (2 * eps)
            worst = max(worst, rel_err(grads[gkey], fd))
    return worst


BWD_FD_TOL = 1e-7


# ----------------------------------------------------------------------------- SSD gradients
def check_ssd_bwd_finite_differences(ssd_bwd, ssd, seed=50, eps=3e-6):
    """The SSD gradients are the derivative of the forward map: every entry of every gradient
    equals the central difference of the forward oracle's loss sum(dy * y) + sum(dh_last * h_last).
    Cases: (i) 4 heads in 2 groups, per-channel D, softplus with bias, gate, h0, dh_last, one A of
    exactly zero, and L = 70 so that the state is rebuilt from more than one checkpoint (every 64
    steps); (ii) one group given as [B, L, N], plain Delta, per-head D, no gate, h0 or dh_last --
    the gradients of the absent bias and h0 are compared with differences taken at zeros.
    eps = 3e-6: the loss sums hundreds of outputs, and at 1e-6 its fp64 rounding over 2 eps reaches
    1e-8 of the small dA of case (ii); agreement is then within SSD_BWD_FD_TOL."""
    worst = 0.0
    cases = (dict(L=70, H=4, P=2, N=3, groups=2, dskip_per_channel=True),
             dict(L=9, H=2, P=3, N=2, gate=False, softplus=False))
    for k, kw in enumerate(cases):
        case = tiny_ssd_case(seed + k, Bsz=2, **kw)
        Bsz, L, H, P = case["x"].shape
        N = case["Bm"].shape[-1]
        g = RNG(seed + 10 + k)
        if k == 0:
            case["A"][1] = 0.0
            case["h0"] = g.standard_normal((Bsz, H, P, N))
        else:
            case["delta"] = np.abs(case["delta"]) * 0.3 + 0.05
            case["delta_bias"] = None
        dy = g.standard_normal(case["x"].shape)
        dh_last = g.standard_normal((Bsz, H, P, N)) if k == 0 else None
        grads = ssd_bwd(dy=dy, dh_last=dh_last, **case)
        full = dict(case)
        for key, shape in (("delta_bias", (H,)), ("h0", (Bsz, H, P, N))):
            if full.get(key) is None:
                full[key] = np.zeros(shape)
        for key, gkey in _GRAD_OF:
            if full.get(key) is None:
                continue
            arr = full[key] = np.array(full[key], dtype=np.float64)
            fd = np.zeros_like(arr)
            for idx in np.ndindex(arr.shape):
                v = arr[idx]
                arr[idx] = v + eps
                lp = _fd_loss(ssd, full, dy, dh_last)
                arr[idx] = v - eps
                lm = _fd_loss(ssd, full, dy, dh_last)
                arr[idx] = v
                fd[idx] = (lp - lm) / (2 * eps)
            worst = max(worst, rel_err(grads[gkey], fd))
    return worst


def check_ssd_bwd_equals_scan_bwd(ssd_bwd, scan_bwd, seed=52):
    """The SSD layer is the selective scan with A[d, n] = A_h and Delta[b, t, d] = Delta[b, t, h]
    for the channels d = (h, p) of head h, so its gradients are the scan's gathered per head:
    dx, dz, dB, dC, dh0 equal; ddelta, dA, ddelta_bias, dD (per head) are the scan's sums over the
    head's channels (and over the N states for dA)."""
    c = tiny_ssd_case(seed, L=23)
    Bsz, L, H, P = c["x"].shape
    N = c["Bm"].shape[2]
    g = RNG(seed + 1)
    h0 = g.standard_normal((Bsz, H, P, N))
    dy = g.standard_normal(c["x"].shape)
    dhl = g.standard_normal((Bsz, H, P, N))
    gs = ssd_bwd(h0=h0, dy=dy, dh_last=dhl, **c)
    sc = dict(x=c["x"].reshape(Bsz, L, H * P), delta=np.repeat(c["delta"], P, axis=2),
              A=np.repeat(c["A"], P)[:, None] * np.ones((1, N)), Bm=c["Bm"], Cm=c["Cm"],
              delta_bias=np.repeat(c["delta_bias"], P), delta_softplus=c["delta_softplus"],
              Dskip=np.repeat(c["Dskip"], P), z=c["z"].reshape(Bsz, L, H * P), h0=h0.reshape(Bsz, H * P, N))
    gc = scan_bwd(dy=dy.reshape(Bsz, L, H * P), dh_last=dhl.reshape(Bsz, H * P, N), **sc)
    per_head = lambda a, ax: a.reshape(a.shape[:ax] + (H, P) + a.shape[ax + 1:]).sum(axis=ax + 1)
    return max(
        rel_err(gs["dx"].reshape(Bsz, L, H * P), gc["dx"]),
        rel_err(gs["dz"].reshape(Bsz, L, H * P), gc["dz"]),
        rel_err(gs["dBm"], gc["dBm"]), rel_err(gs["dCm"], gc["dCm"]),
        rel_err(gs["dh0"].reshape(Bsz, H * P, N), gc["dh0"]),
        rel_err(gs["ddelta"], per_head(gc["ddelta"], 2)),
        rel_err(gs["dA"], per_head(gc["dA"].sum(axis=1), 0)),
        rel_err(gs["ddelta_bias"], per_head(gc["ddelta_bias"], 0)),
        rel_err(gs["dDskip"], per_head(gc["dDskip"], 0)))


SSD_BWD_FD_TOL = 2e-7


# ----------------------------------------------------------------------------- Mamba block
def tiny_block_weights(seed, Dm=8, Di=12, N=4, W=4, R=3):
    g = RNG(seed)
    return dict(ln_w=1 + 0.1 * g.standard_normal(Dm), ln_b=0.1 * g.standard_normal(Dm),
                W_x=g.standard_normal((Di, Dm)) / np.sqrt(Dm), W_z=g.standard_normal((Di, Dm)) / np.sqrt(Dm),
                conv_w=0.5 * g.standard_normal((Di, W)), conv_b=0.1 * g.standard_normal(Di),
                W_dtin=g.standard_normal((R, Di)) / np.sqrt(Di), W_B=g.standard_normal((N, Di)) / np.sqrt(Di),
                W_C=g.standard_normal((N, Di)) / np.sqrt(Di), W_dt=g.standard_normal((Di, R)) / np.sqrt(R),
                b_dt=-2.0 + 0.3 * g.standard_normal(Di), A=-np.tile(np.arange(1.0, N + 1), (Di, 1)),
                D=g.standard_normal(Di), W_out=g.standard_normal((Dm, Di)) / np.sqrt(Di))


def check_layernorm_closed_form(layernorm, eps=1e-5):
    """Rows mu + sigma * s with s = (+1, -1, +1, ...) have mean mu and variance sigma^2 exactly, so
    LayerNorm gives s sigma / sqrt(sigma^2 + eps) * w + b."""
    g = RNG(60)
    Dm = 10
    s = np.array([1.0, -1.0] * (Dm // 2))
    mu, sig = g.standard_normal((3, 1)) * 3, np.array([[0.5], [2.0], [1e-3]])
    w, b = g.standard_normal(Dm), g.standard_normal(Dm)
    want = s * sig / np.sqrt(sig ** 2 + eps) * w + b
    return rel_err(layernorm(mu + sig * s, w, b, eps), want)


def check_block_step_equals_sequence(block_step, block_seq, seed=61):
    """The block's state is the convolution register and the SSM state: L single-token steps from
    a given register and state give the sequence form's outputs, register and state (the sequence
    form uses the pinned full-sequence convolution and scan, the steps the pinned decode step)."""
    g = RNG(seed)
    Bsz, L, Dm, Di, N, W = 2, 9, 8, 12, 4, 4
    wts = tiny_block_weights(seed)
    hid = g.standard_normal((Bsz, L, Dm))
    reg0 = g.standard_normal((Bsz, Di, W))
    h0 = g.standard_normal((Bsz, Di, N))
    out, reg, hl = block_seq(hid, reg0, h0, wts)
    r, h = reg0, h0
    outs = []
    for t in range(L):
        o, r, h = block_step(hid[:, t], r, h, wts)
        outs.append(o)
    return max(rel_err(np.stack(outs, axis=1), out), rel_err(r, reg), rel_err(h, hl))

