"""Helpers of the GPU parity tests: run the HIP path and the CPU oracle on the
same seeded inputs and compare them row by row.

Row error (the decode tolerance): max_c |o_gpu[c] - o_orc[c]| / ||o_orc||_2 <= 1e-4
for every (group, head, step) row.  Rows where the aggregate rectifier's
decision sits within rounding of its threshold (|far_den| < 1e-5 * sum|gain Z^|)
may take either branch: there the GPU row must match the oracle's output under
one of the two branches.
"""
from __future__ import annotations

import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle as O
import streaming_nystr_attention_amd as P
from streaming_nystr_attention_amd import workloads as W

DECODE_TOL = 1e-4
AMBIG_REL = 1e-5
THREADS = min(16, os.cpu_count() or 1)


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu(x):
    return x.detach().to("cpu").numpy()


def oracle_prefill(wl, qh, kh, vh, frozen=None, rect=O.RECT_AGGREGATE):
    """One oracle group per sampled group: qh [n][hpk][T][d], kh [n][T][d], vh [n][T][dv]."""
    def one(i):
        g = O.Group(wl.m, wl.w, wl.sink, wl.hpk, rect)
        fz = None if frozen is None else frozen[i]
        g.prefill(qh[i], kh[i], vh[i], frozen=fz)
        return g

    with ThreadPoolExecutor(THREADS) as ex:
        return list(ex.map(one, range(len(qh))))


def oracle_decode(groups, qs, ks, vs):
    """Step every oracle group through its inputs qs [steps][n][hpk][d] ...

    Returns (out, alt, ambiguous) with out/alt [steps][n][hpk][dv] f64 and
    ambiguous [steps][n][hpk] bool."""
    steps, n = qs.shape[0], qs.shape[1]
    hpk, dv = qs.shape[2], vs.shape[2]
    out = np.zeros((steps, n, hpk, dv))
    alt = np.zeros((steps, n, hpk, dv))
    amb = np.zeros((steps, n, hpk), bool)

    def one(i):
        g = groups[i]
        o, a, dg = g.step_many(np.ascontiguousarray(qs[:, i]), np.ascontiguousarray(ks[:, i]),
                               np.ascontiguousarray(vs[:, i]), with_alt=True)
        out[:, i] = o
        alt[:, i] = a
        fd = np.ctypeslib.as_array(dg).reshape(steps, hpk)
        amb[:, i] = (fd["have_far"] != 0) & (np.abs(fd["far_den"]) < AMBIG_REL * fd["far_abs"])

    with ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(one, range(n)))
    return out, alt, amb


def row_errors(gpu, out, alt, amb):
    """Per-row relative max error; ambiguous rows take the better branch."""
    nrm = np.linalg.norm(out, axis=-1)
    e = np.abs(gpu - out).max(-1) / np.maximum(nrm, 1e-300)
    alt_ok = np.isfinite(alt).all(-1)
    nrm_a = np.linalg.norm(np.where(np.isfinite(alt), alt, 0.0), axis=-1)
    ea = np.abs(gpu - np.where(np.isfinite(alt), alt, 0.0)).max(-1) / np.maximum(nrm_a, 1e-300)
    e = np.where(amb & alt_ok, np.minimum(e, ea), e)
    return e


def oracle_frozen_arrays(wl, groups):
    """Per sampled group, the oracle's f32 K~, Q~, M (as the oracle stores them)."""
    res = []
    for g in groups:
        st = g.state()
        res.append(O.Frozen(k_tilde=st["k_tilde"], q_tilde=st["q_tilde"], mu=st["mu"]))
    return res


class DecodeRun:
    """GPU decode over `steps` steps of a workload with sampled groups gathered."""

    def __init__(self, wl, sample, steps, dev="cuda"):
        self.wl, self.sample, self.steps = wl, sample, steps
        self.idx = torch.tensor(sample, device=dev, dtype=torch.long)
        n = len(sample)
        self.q = torch.empty(steps, n, wl.hpk, wl.d, device=dev)
        self.k = torch.empty(steps, n, wl.d, device=dev)
        self.v = torch.empty(steps, n, wl.dv, device=dev)
        self.out = torch.empty(steps, n, wl.hpk, wl.dv, device=dev)

    def run(self, grp, dev="cuda", to_host=True):
        """Step `grp` through every step's inputs, keeping the sampled groups' inputs
        and outputs on the device; with `to_host` returns them all as host arrays."""
        wl = self.wl
        G = wl.groups
        qb = torch.empty(G, wl.hpk, wl.d, device=dev)
        kb = torch.empty(G, wl.d, device=dev)
        vb = torch.empty(G, wl.dv, device=dev)
        ob = torch.empty(G, wl.hpk, wl.dv, device=dev)
        t0 = time.time()
        for t in range(self.steps):
            W.decode_inputs(wl, t, dev, out=(qb, kb, vb))
            grp.step(qb, kb, vb, ob)
            self.q[t] = qb.index_select(0, self.idx)
            self.k[t] = kb.index_select(0, self.idx)
            self.v[t] = vb.index_select(0, self.idx)
            self.out[t] = ob.index_select(0, self.idx)
        torch.cuda.synchronize()
        say(f"  gpu decode {self.steps} steps x {G} groups: {time.time() - t0:.2f}s")
        if to_host:
            return self.host(0, len(self.sample))

    def host(self, c0, c1):
        """Host copies of sampled groups c0..c1-1: q, k, v (f32) and the outputs (f64)."""
        s = slice(c0, c1)
        return (cpu(self.q[:, s]), cpu(self.k[:, s]), cpu(self.v[:, s]),
                cpu(self.out[:, s]).astype(np.float64))


def frozen_tensors_with_oracle(grp, wl, sample, orc_groups, dev="cuda"):
    """Full-size frozen (K~, Q~, M) tensors: the GPU's own prefill values, with the
    sampled groups' entries replaced by the oracle's."""
    G, H, m, d = wl.groups, wl.hpk, wl.m_eff, wl.d
    kt = grp.read(P.FIELD_K_TILDE, device=dev).view(G, m, d).clone()
    qt = grp.read(P.FIELD_Q_TILDE, device=dev).view(G, H, m, d).clone()
    mu = grp.read(P.FIELD_MU, device=dev).view(G, H, m, m).clone()
    for i, g in enumerate(sample):
        st = orc_groups[i].state()
        kt[g] = torch.from_numpy(st["k_tilde"]).to(dev)
        qt[g] = torch.from_numpy(st["q_tilde"]).to(dev)
        mu[g] = torch.from_numpy(st["mu"]).to(dev)
    return kt.contiguous(), qt.contiguous(), mu.contiguous()


# ---- whole parity runs shared by the GPU test modules -------------------

DEV = "cuda"
RESID_TOL = 1e-3
CHUNK_BYTES = 1 << 29


def stack_frozen(orc_groups):
    sts = [g.state() for g in orc_groups]
    kt = torch.from_numpy(np.stack([s["k_tilde"] for s in sts])).to(DEV)
    qt = torch.from_numpy(np.stack([s["q_tilde"] for s in sts])).to(DEV)
    mu = torch.from_numpy(np.stack([s["mu"] for s in sts])).to(DEV)
    return kt, qt, mu


def decode_parity(wl, sample=None, steps=None, rect=O.RECT_AGGREGATE, frozen_override=None):
    steps = wl.steps if steps is None else steps
    G = wl.groups
    sample = list(range(G)) if sample is None else sample
    say(f"[decode] {wl.name}: G={G} hpk={wl.hpk} d={wl.d} m={wl.m} w={wl.w} sink={wl.sink} "
        f"T={wl.T} steps={steps} rect={rect} sampled={len(sample)}")
    q, k, v = W.prompt(wl, DEV)
    si = torch.tensor(sample, device=DEV)
    qh, kh, vh = cpu(q[si]), cpu(k[si]), cpu(v[si])
    fz_orc = None
    if frozen_override is not None:
        fz_orc = [O.Frozen(mu=frozen_override) for _ in sample]
    orc = oracle_prefill(wl, qh, kh, vh, frozen=fz_orc, rect=rect)
    cfg = wl.config
    cfg = P.Config(**{**cfg.__dict__, "rect": rect})
    grp = P.O1Groups(cfg)
    if len(sample) == G:
        frozen = stack_frozen(orc)
    else:
        grp.prefill(q, k, v)
        frozen = frozen_tensors_with_oracle(grp, wl, sample, orc)
    grp.prefill(q, k, v, frozen=frozen)
    del q, k, v, frozen
    run = DecodeRun(wl, sample, steps)
    run.run(grp, to_host=False)
    # compare in chunks of groups so the host holds at most ~CHUNK_BYTES of f64 outputs
    n = len(sample)
    per_group = max(1, steps * wl.hpk * wl.dv * 8)
    cg = max(1, min(n, CHUNK_BYTES // per_group))
    errs, n_amb, t0 = [], 0, time.time()
    for c0 in range(0, n, cg):
        c1 = min(n, c0 + cg)
        qs, ks, vs, gout = run.host(c0, c1)
        out, alt, amb = oracle_decode(orc[c0:c1], qs, ks, vs)
        errs.append(row_errors(gout, out, alt, amb))
        n_amb += int(amb.sum())
        del qs, ks, vs, gout, out, alt, amb
    del run
    err = np.concatenate(errs, axis=1)
    say(f"  rows={err.size} max_err={err.max():.3e} median={np.median(err):.3e} "
        f"ambiguous={n_amb} oracle decode {time.time() - t0:.1f}s")

    # counters of every group, bit-exact
    E = wl.T - wl.sink - wl.w + steps
    far_len = grp.read(P.FIELD_FAR_LEN).numpy()
    win_head = grp.read(P.FIELD_WIN_HEAD).numpy()
    assert (far_len == E).all(), "far_len must equal the eviction count for every head"
    assert (win_head == E % wl.w).all()
    for i in range(len(sample)):
        assert orc[i].far_len(0) == E and orc[i].win_head == E % wl.w

    # ring and sink rows of the sampled groups, bit-exact
    R = wl.sink + wl.w
    nk = grp.read(P.FIELD_NEAR_K).view(G, R, wl.d)[sample].numpy()
    nv = grp.read(P.FIELD_NEAR_V).view(G, R, wl.dv)[sample].numpy()
    for i in range(len(sample)):
        st = orc[i].state()
        np.testing.assert_array_equal(nk[i, : wl.sink], st["sink_k"])
        np.testing.assert_array_equal(nv[i, : wl.sink], st["sink_v"])
        np.testing.assert_array_equal(nk[i, wl.sink:], st["win_k"])
        np.testing.assert_array_equal(nv[i, wl.sink:], st["win_v"])
    grp.close()
    assert err.max() <= DECODE_TOL, f"max row error {err.max():.3e}"
    return err


def ulp_diff(a, b):
    ai = a.view(np.int32).astype(np.int64)
    bi = b.view(np.int32).astype(np.int64)
    return np.abs(ai - bi).max() if a.size else 0


def prefill_parity(wl, sample=None):
    G, H, m, d, dv = wl.groups, wl.hpk, wl.m_eff, wl.d, wl.dv
    sample = list(range(G)) if sample is None else sample
    say(f"[prefill] {wl.name}: G={G} hpk={H} T={wl.T} m_eff={m} sampled={len(sample)}")
    q, k, v = W.prompt(wl, DEV)
    si = torch.tensor(sample, device=DEV)
    qh, kh, vh = cpu(q[si]), cpu(k[si]), cpu(v[si])
    grp = P.O1Groups(wl.config)
    grp.prefill(q, k, v)
    torch.cuda.synchronize()
    info = grp.info()
    assert info.sealed == 1 and info.m_eff == m and info.prompt_len == wl.T
    del q, k, v
    orc = oracle_prefill(wl, qh, kh, vh)

    kt = grp.read(P.FIELD_K_TILDE).view(G, m, d)[sample].numpy()
    qt = grp.read(P.FIELD_Q_TILDE).view(G, H, m, d)[sample].numpy()
    mu = grp.read(P.FIELD_MU).view(G, H, m, m)[sample].numpy().astype(np.float64)
    lam = grp.read(P.FIELD_LAMBDA).view(G, H)[sample].numpy()
    tries = grp.read(P.FIELD_TRIES).view(G, H)[sample].numpy()
    th = grp.read(P.FIELD_T_HAT).view(G, H, m, dv)[sample].numpy().astype(np.float64)
    zh = grp.read(P.FIELD_Z_HAT).view(G, H, m)[sample].numpy()
    mx = grp.read(P.FIELD_M_MAX).view(G, H, m)[sample].numpy().astype(np.float64)
    R = wl.sink + wl.w
    nk = grp.read(P.FIELD_NEAR_K).view(G, R, d)[sample].numpy()
    nv = grp.read(P.FIELD_NEAR_V).view(G, R, dv)[sample].numpy()
    far_len = grp.read(P.FIELD_FAR_LEN).numpy()
    win_head = grp.read(P.FIELD_WIN_HEAD).numpy()
    E = wl.T - wl.sink - wl.w
    assert (far_len == E).all() and (win_head == E % wl.w).all()

    # resid: the GPU M's ||A M A - A||_F / ||A||_F; resid_orc: the oracle's own f32 M
    # on the same A; resid_f64: the unrounded ridge solution (numpy) with the
    # oracle's lambda -- logged so the GPU figure can be read against both.
    worst = {"lm_ulp": 0, "resid": 0.0, "resid_orc": 0.0, "resid_f64": 0.0, "lam": 0.0,
             "far": 0.0, "z": 0.0}
    for i, g in enumerate(orc):
        st = g.state()
        worst["lm_ulp"] = max(worst["lm_ulp"], ulp_diff(kt[i], st["k_tilde"]),
                              ulp_diff(qt[i], st["q_tilde"]))
        np.testing.assert_array_equal(nk[i, : wl.sink], st["sink_k"])
        np.testing.assert_array_equal(nk[i, wl.sink:], st["win_k"])
        np.testing.assert_array_equal(nv[i, : wl.sink], st["sink_v"])
        np.testing.assert_array_equal(nv[i, wl.sink:], st["win_v"])
        for h in range(H):
            A = st["au"][h]
            r = np.linalg.norm(A @ mu[i, h] @ A - A) / np.linalg.norm(A)
            worst["resid"] = max(worst["resid"], r)
            mo = st["mu"][h].astype(np.float64)
            worst["resid_orc"] = max(worst["resid_orc"],
                                     np.linalg.norm(A @ mo @ A - A) / np.linalg.norm(A))
            m64 = np.linalg.solve(A.T @ A + st["lambda"][h] * np.eye(A.shape[0]), A.T)
            worst["resid_f64"] = max(worst["resid_f64"],
                                     np.linalg.norm(A @ m64 @ A - A) / np.linalg.norm(A))
            worst["lam"] = max(worst["lam"], abs(lam[i, h] - st["lambda"][h]) / st["lambda"][h])
            assert tries[i, h] == st["tries"][h]
            # far field at a common scale: the oracle's running max
            shift = np.exp(mx[i, h] - st["m_max"][h])
            tg = th[i, h] * shift[:, None]
            rel = np.abs(tg - st["t_hat"][h]).max(1) / np.maximum(np.linalg.norm(st["t_hat"][h], axis=1), 1e-300)
            worst["far"] = max(worst["far"], rel.max())
            zr = np.abs(zh[i, h] * shift - st["z_hat"][h]) / st["z_hat"][h]
            worst["z"] = max(worst["z"], zr.max())
    say("  " + " ".join(f"{k}={float(v):.4e}" if isinstance(v, float) else f"{k}={v}"
                        for k, v in worst.items()))
    grp.close()
    assert worst["lm_ulp"] <= 1
    assert worst["resid"] <= RESID_TOL
    assert worst["lam"] <= 1e-12
    # the far weights e^{l - max} are f32 values (an f32 exp, as NystromHead::far_insert
    # on the nystrom.rs source page takes them; the gap itself is formed in f64) and
    # T^ is accumulated in f32 as the page accumulates it: T^ rows within 1e-5, Z^
    # (f64 sums of the f32 weights) within 1e-6 relative
    assert worst["far"] <= 1e-5
    assert worst["z"] <= 1e-6
