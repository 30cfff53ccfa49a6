"""Helpers of the GPU parity tests: run the HIP path and the CPU oracle on the
same seeded inputs and compare them row by row.

Row error (the benchmark spec tolerance): max_c |o_gpu[c] - o_orc[c]| / ||o_orc||_2 <= 1e-4
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

    def run(self, grp, dev="cuda"):
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
        return cpu(self.q), cpu(self.k), cpu(self.v), cpu(self.out).astype(np.float64)


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
