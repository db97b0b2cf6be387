"""Helpers for the GPU parity tests: move seeded inputs to the device, run the HIP path through
the C ABI (via the ctypes binding), run the fp64 oracle on the same stored inputs, compare.

Error metric (the tolerance the parity bar states, read as a norm): per output tensor,
max_i |gpu_i - ref_i| / max_i |ref_i|, in fp64. Bar: 1e-5 for fp32 inputs, 2e-2 for bf16
inputs (float32 state and accumulation in both)."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from selective_state_space_37_amd import inputs, ssm

TOL = {"f32": 1e-5, "bf16": 2e-2}


def dev(a, dtype: str = "f32"):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def host(t):
    return None if t is None else t.float().cpu().numpy().astype(np.float64)


def rel_err(a, ref) -> float:
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(a - ref))) / max(float(np.max(np.abs(ref))), 1e-30)


def elementwise_diag(a, ref):
    """Element-wise relative error |a - ref| / (|ref| + 1e-3 max|ref|): its median, 99.9th
    percentile and maximum (a diagnostic printed beside the max-norm metric, not a gate)."""
    a = np.asarray(a, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    if ref.size == 0:
        return 0.0, 0.0, 0.0
    r = np.abs(a - ref) / (np.abs(ref) + 1e-3 * float(np.max(np.abs(ref))) + 1e-300)
    q = np.quantile(r, [0.5, 0.999])
    return float(q[0]), float(q[1]), float(np.max(r))


def diag_str(a, ref) -> str:
    m, p, x = elementwise_diag(a, ref)
    return "elementwise median %.2e p99.9 %.2e max %.2e" % (m, p, x)


class Accum:
    """Max-norm error and element-wise diagnostic accumulated over blocks of one output tensor.

    The diagnostic's normaliser needs max|ref| over the whole tensor, so the blocks' |a - ref| and
    |ref| are kept (float32) and reduced at the end."""

    def __init__(self):
        self.maxdiff = 0.0
        self.maxref = 0.0
        self.diffs, self.refs = [], []

    def add(self, a, ref):
        a = np.asarray(a, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        assert np.isfinite(a).all(), "non-finite output"
        d = np.abs(a - ref)
        self.maxdiff = max(self.maxdiff, float(d.max(initial=0.0)))
        self.maxref = max(self.maxref, float(np.abs(ref).max(initial=0.0)))
        self.diffs.append(d.astype(np.float32).ravel())
        self.refs.append(np.abs(ref).astype(np.float32).ravel())

    def err(self) -> float:
        return self.maxdiff / max(self.maxref, 1e-30)

    def diag(self) -> str:
        d = np.concatenate(self.diffs).astype(np.float64)
        r = d / (np.concatenate(self.refs).astype(np.float64) + 1e-3 * self.maxref + 1e-300)
        q = np.quantile(r, [0.5, 0.999])
        return "elementwise median %.2e p99.9 %.2e max %.2e" % (q[0], q[1], r.max())


# ----------------------------------------------------------------------------- scan
def scan_on_gpu(inp: inputs.ScanInputs, segment_len=None, return_state=True):
    y, hl = ssm.scan_fwd(dev(inp.x), dev(inp.delta), dev(inp.A), dev(inp.Bm), dev(inp.Cm),
                         delta_bias=dev(inp.delta_bias), delta_softplus=inp.delta_softplus,
                         Dskip=dev(inp.Dskip), z=dev(inp.z), h0=dev(inp.h0),
                         return_state=return_state, segment_len=segment_len)
    torch.cuda.synchronize()
    return host(y), host(hl)


def scan_oracle(inp: inputs.ScanInputs, channels=None):
    w = lambda a: inputs.widen(a, inp.dtype)
    sel = (lambda a, ax: a if a is None or channels is None else np.take(a, channels, axis=ax))
    return oracle.scan(sel(w(inp.x), 2), sel(w(inp.delta), 2), sel(inp.A, 0), w(inp.Bm), w(inp.Cm),
                       delta_bias=sel(inp.delta_bias, 0), delta_softplus=inp.delta_softplus,
                       Dskip=sel(inp.Dskip, 0), z=sel(w(inp.z), 2), h0=sel(inp.h0, 1))


def scan_parity(inp, gpu_out, channels=None) -> float:
    y, hl = gpu_out
    ry, rh = scan_oracle(inp, channels)
    if channels is not None:
        y = y[:, :, channels]
        hl = None if hl is None else hl[:, channels]
    e = rel_err(y, ry)
    if hl is not None:
        e = max(e, rel_err(hl, rh))
    return e


def scan_parity_blocks(inp, gpu_out, block: int):
    """Whole-tensor parity of a scan result, the oracle run over channel blocks of `block` (the
    channels' recurrences are independent, so each block is the full problem's exact answer on
    those channels). Returns (Accum for y, Accum for h_last or None)."""
    y, hl = gpu_out
    D = inp.x.shape[2]
    ay, ah = Accum(), (Accum() if hl is not None else None)
    for c0 in range(0, D, block):
        ch = np.arange(c0, min(D, c0 + block))
        ry, rh = scan_oracle(inp, ch)
        ay.add(y[:, :, ch], ry)
        if ah is not None:
            ah.add(hl[:, ch], rh)
    return ay, ah


# ----------------------------------------------------------------------------- prefill with conv
def scan_conv_on_gpu(inp: inputs.ScanInputs, conv_w, conv_b=None, conv_state=None, segment_len=0):
    """ssm_scan_fwd_conv; conv_state (storage type) is updated in place. Returns (y, h_last,
    register) on the host; the register as raw storage values (bf16 bits widened exactly)."""
    reg = dev(conv_state) if conv_state is not None else None
    y, hl = ssm.scan_fwd_conv(dev(inp.x), dev(inp.delta), dev(inp.A), dev(inp.Bm), dev(inp.Cm),
                              dev(conv_w), conv_b=dev(conv_b), conv_state=reg,
                              delta_bias=dev(inp.delta_bias), delta_softplus=inp.delta_softplus,
                              Dskip=dev(inp.Dskip), z=dev(inp.z), h0=dev(inp.h0),
                              segment_len=segment_len)
    torch.cuda.synchronize()
    return host(y), host(hl), host(reg)


def scan_conv_oracle(inp: inputs.ScanInputs, conv_w, conv_b=None, conv_state=None, channels=None):
    w = lambda a: inputs.widen(a, inp.dtype)
    sel = (lambda a, ax: a if a is None or channels is None else np.take(a, channels, axis=ax))
    return oracle.scan_conv(sel(w(inp.x), 2), sel(w(inp.delta), 2), sel(inp.A, 0), w(inp.Bm), w(inp.Cm),
                            sel(conv_w, 0), conv_b=sel(conv_b, 0), conv_state=sel(w(conv_state), 1),
                            delta_bias=sel(inp.delta_bias, 0), delta_softplus=inp.delta_softplus,
                            Dskip=sel(inp.Dskip, 0), z=sel(w(inp.z), 2), h0=sel(inp.h0, 1))


# ----------------------------------------------------------------------------- scan backward
BWD_KEYS = ("dx", "ddelta", "dz", "dA", "dBm", "dCm", "dDskip", "ddelta_bias", "dh0")


def scan_bwd_on_gpu(inp: inputs.ScanInputs, dy, dh_last=None, segment_len=None):
    out = ssm.scan_bwd(dev(inp.x), dev(inp.delta), dev(inp.A), dev(inp.Bm), dev(inp.Cm), dev(dy),
                       delta_bias=dev(inp.delta_bias), delta_softplus=inp.delta_softplus,
                       Dskip=dev(inp.Dskip), z=dev(inp.z), h0=dev(inp.h0), dh_last=dev(dh_last),
                       segment_len=segment_len)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in out.items()}


def scan_bwd_oracle(inp: inputs.ScanInputs, dy, dh_last=None, channels=None, rows=None):
    """Oracle gradients; channels restricts to a channel subset (everything but dBm, dCm then
    matches the full problem's values on those channels), rows to a batch-row subset (everything
    but dA, dDskip, ddelta_bias then matches on those rows)."""
    w = lambda a: inputs.widen(a, inp.dtype)
    ch = (lambda a, ax: a if a is None or channels is None else np.take(a, channels, axis=ax))
    rw = (lambda a: a if a is None or rows is None else np.take(a, rows, axis=0))
    return oracle.scan_bwd(rw(ch(w(inp.x), 2)), rw(ch(w(inp.delta), 2)), ch(inp.A, 0),
                           rw(w(inp.Bm)), rw(w(inp.Cm)), rw(ch(w(dy), 2)),
                           delta_bias=ch(inp.delta_bias, 0), delta_softplus=inp.delta_softplus,
                           Dskip=ch(inp.Dskip, 0), z=rw(ch(w(inp.z), 2)), h0=rw(ch(inp.h0, 1)),
                           dh_last=rw(ch(dh_last, 1)))


def scan_bwd_errors(gpu: dict, ref: dict, channels=None, rows=None) -> dict:
    """Per-gradient error (the parity metric); with channels / rows, only the entries that the
    restricted oracle call determines are compared."""
    errs = {}
    for k in BWD_KEYS:
        g, r = gpu.get(k), ref.get(k)
        if r is None or g is None:
            continue
        if channels is not None:
            if k in ("dBm", "dCm"):
                continue
            ax = {"dx": 2, "ddelta": 2, "dz": 2, "dA": 0, "dDskip": 0, "ddelta_bias": 0, "dh0": 1}[k]
            g = np.take(g, channels, axis=ax)
        if rows is not None:
            if k in ("dA", "dDskip", "ddelta_bias"):
                continue
            g = np.take(g, rows, axis=0)
        errs[k] = rel_err(g, r)
    return errs


# ----------------------------------------------------------------------------- decode step
def step_on_gpu(step: inputs.DecodeStep, A, h, *, Dskip=None, conv_state=None, conv_w=None,
                conv_b=None, delta_bias=None, delta_softplus=False):
    """Runs one ssm_state_update; h / conv_state are device tensors updated in place."""
    return ssm.state_update(dev(step.x), dev(step.delta), A, dev(step.Bm), dev(step.Cm), h,
                            delta_bias=delta_bias, delta_softplus=delta_softplus, Dskip=Dskip,
                            z=dev(step.z), conv_state=conv_state, conv_w=conv_w, conv_b=conv_b)


def step_smoke(Bsz=4, D=64, N=16, dtype="bf16", seed=3):
    prm = inputs.decode_params(seed=seed, D=D, N=N)
    reg = inputs.conv_register(seed, Bsz, D, 4, dtype)
    h0 = inputs.draw_param(seed, 50, (Bsz, D, N), scale=0.5)
    st = inputs.decode_step(seed, 0, Bsz, D, N, dtype)
    h = dev(h0)
    conv = dev(reg)
    y = step_on_gpu(st, dev(prm["A"]), h, Dskip=dev(prm["Dskip"]), conv_state=conv,
                    conv_w=dev(prm["conv_w"]))
    torch.cuda.synchronize()
    w = lambda a: inputs.widen(a, dtype)
    ry, rh, rc = oracle.step(w(st.x), w(st.delta), prm["A"], w(st.Bm), w(st.Cm), h0,
                             Dskip=prm["Dskip"], z=w(st.z), conv_state=w(reg), conv_w=prm["conv_w"])
    return max(rel_err(host(y), ry), rel_err(host(h), rh), rel_err(host(conv), rc))


# ----------------------------------------------------------------------------- SSD
def ssd_on_gpu(inp: inputs.SSDInputs, chunk=256, return_state=True, grouped=None):
    """grouped=None: ssd_chunk_fwd_grouped for grouped B/C or per-channel D, else ssd_chunk_fwd."""
    if grouped is None:
        grouped = inp.Bm.ndim == 4 or (inp.Dskip is not None and inp.Dskip.ndim == 2)
    Bm, Cm = inp.Bm, inp.Cm
    if grouped and Bm.ndim == 3:
        Bm, Cm = Bm[:, :, None], Cm[:, :, None]
    fn = ssm.ssd_chunk_fwd_grouped if grouped else ssm.ssd_chunk_fwd
    y, hl = fn(dev(inp.x), dev(inp.delta), dev(inp.A), dev(Bm), dev(Cm),
               chunk=chunk, delta_bias=dev(inp.delta_bias),
               delta_softplus=inp.delta_softplus, Dskip=dev(inp.Dskip), z=dev(inp.z),
               h0=dev(inp.h0), return_state=return_state)
    torch.cuda.synchronize()
    return host(y), host(hl)


def ssd_oracle(inp: inputs.SSDInputs, heads=None):
    """The oracle on every head, or on the listed heads only (each with its own group's B, C)."""
    w = lambda a: inputs.widen(a, inp.dtype)
    H = inp.x.shape[2]
    hs = np.arange(H) if heads is None else np.asarray(heads)
    G = inp.groups
    if heads is None or G == 1:
        sel = (lambda a, ax: a if a is None or heads is None else np.take(a, hs, axis=ax))
        Bm, Cm = w(inp.Bm), w(inp.Cm)
        return oracle.ssd(sel(w(inp.x), 2), sel(w(inp.delta), 2), sel(inp.A, 0), Bm, Cm,
                          delta_bias=sel(inp.delta_bias, 0), delta_softplus=inp.delta_softplus,
                          Dskip=sel(inp.Dskip, 0), z=sel(w(inp.z), 2), h0=sel(inp.h0, 1))
    ys, hls = [], []
    for h in hs:
        grp = h // (H // G)
        one = lambda a, ax: None if a is None else np.take(a, [h], axis=ax)
        y, hl = oracle.ssd(one(w(inp.x), 2), one(w(inp.delta), 2), one(inp.A, 0),
                           w(inp.Bm)[:, :, grp], w(inp.Cm)[:, :, grp],
                           delta_bias=one(inp.delta_bias, 0), delta_softplus=inp.delta_softplus,
                           Dskip=one(inp.Dskip, 0), z=one(w(inp.z), 2), h0=one(inp.h0, 1))
        ys.append(y)
        hls.append(hl)
    return np.concatenate(ys, axis=2), np.concatenate(hls, axis=1)


def ssd_bwd_on_gpu(inp: inputs.SSDInputs, dy, dh_last=None):
    out = ssm.ssd_chunk_bwd(dev(inp.x), dev(inp.delta), dev(inp.A), dev(inp.Bm), dev(inp.Cm), dev(dy),
                            delta_bias=dev(inp.delta_bias), delta_softplus=inp.delta_softplus,
                            Dskip=dev(inp.Dskip), z=dev(inp.z), h0=dev(inp.h0), dh_last=dev(dh_last))
    torch.cuda.synchronize()
    return {k: host(v) for k, v in out.items()}


def ssd_bwd_oracle(inp: inputs.SSDInputs, dy, dh_last=None, heads=None):
    """Oracle gradients; heads restricts to a head subset, each run with its own group's B and C
    (everything but dBm, dCm then matches the full problem's values on those heads)."""
    w = lambda a: inputs.widen(a, inp.dtype)
    H = inp.x.shape[2]
    kw = dict(delta_softplus=inp.delta_softplus)
    if heads is None:
        return oracle.ssd_bwd(w(inp.x), w(inp.delta), inp.A, w(inp.Bm), w(inp.Cm), w(dy),
                              delta_bias=inp.delta_bias, Dskip=inp.Dskip, z=w(inp.z), h0=inp.h0,
                              dh_last=dh_last, **kw)
    G = inp.groups
    outs = []
    for h in heads:
        grp = h // (H // G)
        one = lambda a, ax: None if a is None else np.take(a, [h], axis=ax)
        Bm = w(inp.Bm)[:, :, grp] if inp.Bm.ndim == 4 else w(inp.Bm)
        Cm = w(inp.Cm)[:, :, grp] if inp.Cm.ndim == 4 else w(inp.Cm)
        outs.append(oracle.ssd_bwd(one(w(inp.x), 2), one(w(inp.delta), 2), one(inp.A, 0), Bm, Cm,
                                   one(w(dy), 2), delta_bias=one(inp.delta_bias, 0), Dskip=one(inp.Dskip, 0),
                                   z=one(w(inp.z), 2), h0=one(inp.h0, 1), dh_last=one(dh_last, 1), **kw))
    ax = {"dx": 2, "ddelta": 2, "dz": 2, "dA": 0, "dDskip": 0, "ddelta_bias": 0, "dh0": 1}
    return {k: (None if outs[0][k] is None else np.concatenate([o[k] for o in outs], axis=a))
            for k, a in ax.items()}


def ssd_bwd_errors(gpu: dict, ref: dict, heads=None) -> dict:
    errs = {}
    ax = {"dx": 2, "ddelta": 2, "dz": 2, "dA": 0, "dDskip": 0, "ddelta_bias": 0, "dh0": 1}
    for k in BWD_KEYS:
        g, r = gpu.get(k), ref.get(k)
        if r is None or g is None:
            continue
        if heads is not None:
            if k in ("dBm", "dCm"):
                continue
            g = np.take(g, heads, axis=ax[k])
        errs[k] = rel_err(g, r)
    return errs


def ssd_parity_blocks(inp, gpu_out, block: int):
    """Whole-tensor parity of an SSD result, the oracle run over blocks of `block` heads (each head
    is independent given its group's B and C). Returns (Accum for y, Accum for h_last or None)."""
    y, hl = gpu_out
    H = inp.x.shape[2]
    ay, ah = Accum(), (Accum() if hl is not None else None)
    for h0 in range(0, H, block):
        hs = np.arange(h0, min(H, h0 + block))
        ry, rh = ssd_oracle(inp, hs)
        ay.add(y[:, :, hs], ry)
        if ah is not None:
            ah.add(hl[:, hs], rh)
    return ay, ah


def ssd_parity(inp, gpu_out, heads=None) -> float:
    y, hl = gpu_out
    ry, rh = ssd_oracle(inp, heads)
    if heads is not None:
        y = y[:, :, heads]
        hl = None if hl is None else hl[:, heads]
    e = rel_err(y, ry)
    if hl is not None:
        e = max(e, rel_err(hl, rh))
    return e
