"""GPU tests of the prefill's ridge pseudo-inverse on its retry and fallback
paths, of the info record (the page's memory_bytes, the ridge summary), and of
a counter write in the middle of a fold period.

ridge_pinv (nystrom.rs source page) grows lambda tenfold after a failed
Cholesky factorisation, up to 12 attempts, then returns a scaled identity.
Both paths are reached here with inputs whose outcome IEEE arithmetic fixes,
so the device and the oracle must take the same attempt:

  retry     frozen landmarks that make A a 0/1 matrix (logits exactly 0, or so
            negative that exp underflows to 0) with two equal columns: A^T A
            holds the block [[1, 1], [1, 1]] and tr(A^T A) / m = 1.  While
            lambda <= 2^-53 the block's second pivot is 1 - 1*1 = 0 exactly;
            with ridge_rel = 8e-19 the fourth attempt (lambda = 8e-16) factors.
  fallback  a NaN in the frozen key landmarks: every pivot test fails, M is
            I / max(mean diag, DBL_MIN) (in f32, +inf on the diagonal) and
            lambda the initial one times 10^12.
"""
import numpy as np
import pytest
import torch

import oracle as O
import streaming_nystr_attention_amd as P
from streaming_nystr_attention_amd import workloads as W

from parity_util import (DECODE_TOL, RESID_TOL, DecodeRun, cpu, oracle_decode, oracle_prefill,
                         row_errors, say)

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    P.lib()
    yield


def zero_one_landmarks(G, hpk, m, d, big=30000.0):
    """K~ [G][m][d] and Q~ [G][hpk][m][d] with exp(q~_i . k~_j / sqrt d) = A[i][j]:
    A[0][0] = A[0][1] = 1, A[j][j] = 1 for j >= 2, every other entry 0 (row 1
    empty).  k~_0 = k~_1 = e_0 and k~_j = e_{j-1}; q~_i is -big on the components
    0 .. m-2 except the one its ones sit on."""
    assert m <= d + 1
    kt = np.zeros((m, d), np.float32)
    kt[0, 0] = kt[1, 0] = 1.0
    for j in range(2, m):
        kt[j, j - 1] = 1.0
    qt = np.full((m, d), 0.0, np.float32)
    qt[:, : m - 1] = -big
    qt[0, 0] = 0.0
    for i in range(2, m):
        qt[i, i - 1] = 0.0
    A = np.exp(qt.astype(np.float64) @ kt.astype(np.float64).T / np.sqrt(d))
    expect = np.zeros((m, m))
    expect[0, 0] = expect[0, 1] = 1.0
    for j in range(2, m):
        expect[j, j] = 1.0
    assert np.array_equal(A, expect)
    return (np.broadcast_to(kt, (G, m, d)).copy(),
            np.broadcast_to(qt, (G, hpk, m, d)).copy())


def _prefill_both(wl, frozen_np, ridge_rel=0.0):
    """The GPU prefill with `frozen_np` = (K~, Q~) (either may be None) and the
    oracle's, group by group, on the same prompt."""
    q, k, v = W.prompt(wl, DEV)
    kt, qt = frozen_np
    fz = [O.Frozen(k_tilde=None if kt is None else kt[i], q_tilde=None if qt is None else qt[i])
          for i in range(wl.groups)]
    orc = []
    for i in range(wl.groups):
        g = O.Group(wl.m, wl.w, wl.sink, wl.hpk)
        if ridge_rel:
            g.set_ridge_rel(ridge_rel)
        g.prefill(cpu(q[i]), cpu(k[i]), cpu(v[i]), frozen=fz[i])
        orc.append(g)
    cfg = P.Config(**{**wl.config.__dict__, "ridge_rel": ridge_rel})
    grp = P.O1Groups(cfg)
    dev_fz = (None if kt is None else torch.from_numpy(kt).to(DEV),
              None if qt is None else torch.from_numpy(qt).to(DEV), None)
    grp.prefill(q, k, v, frozen=dev_fz)
    torch.cuda.synchronize()
    return grp, orc


def test_ridge_retry_on_device_matches_oracle():
    wl = W.Workload("ridge_retry", 1, 1, 2, 2, 64, 64, 16, 32, 4, T=160, steps=0, seed=41)
    G, H, m = wl.groups, wl.hpk, wl.m_eff
    assert m == 16
    kt, qt = zero_one_landmarks(G, H, m, wl.d)
    grp, orc = _prefill_both(wl, (kt, qt), ridge_rel=8e-19)
    lam = grp.read(P.FIELD_LAMBDA).view(G, H).numpy()
    tries = grp.read(P.FIELD_TRIES).view(G, H).numpy()
    mu = grp.read(P.FIELD_MU).view(G, H, m, m).numpy().astype(np.float64)
    worst_m, worst_r = 0.0, 0.0
    for i, g in enumerate(orc):
        st = g.state()
        for h in range(H):
            assert st["tries"][h] == 4 and tries[i, h] == 4, (tries[i, h], st["tries"][h])
            assert lam[i, h] == st["lambda"][h] == 8e-19 * 10.0 * 10.0 * 10.0
            ref = st["mu"][h].astype(np.float64)
            worst_m = max(worst_m, np.abs(mu[i, h] - ref).max() / np.abs(ref).max())
            A = st["au"][h]
            worst_r = max(worst_r, np.linalg.norm(A @ mu[i, h] @ A - A) / np.linalg.norm(A))
    info = grp.info()
    say(f"  retry: tries 4 on {G * H} heads, M max rel diff {worst_m:.2e}, resid {worst_r:.2e}, "
        f"info tries_max={info.tries_max} retried={info.heads_retried}")
    assert worst_m <= 1e-6
    assert worst_r <= RESID_TOL
    assert info.tries_max == 4 and info.heads_retried == G * H and info.heads_fallback == 0
    assert info.lambda_min == info.lambda_max == info.lambda_median == 8e-19 * 10.0 * 10.0 * 10.0


def test_ridge_fallback_on_device_matches_oracle():
    wl = W.Workload("ridge_fallback", 1, 1, 2, 2, 64, 64, 16, 32, 4, T=160, steps=0, seed=42)
    G, H, m, d = wl.groups, wl.hpk, wl.m_eff, wl.d
    q, k, _ = W.prompt(wl, DEV)
    kt = np.stack([O.seg_means(cpu(k[i]), m).astype(np.float32) for i in range(G)])
    kt[:, 3, 5] = np.nan  # column 3 of A, and with it A^T A's trace, become NaN
    grp, orc = _prefill_both(wl, (kt, None))
    lam = grp.read(P.FIELD_LAMBDA).view(G, H).numpy()
    tries = grp.read(P.FIELD_TRIES).view(G, H).numpy()
    mu = grp.read(P.FIELD_MU).view(G, H, m, m).numpy()
    tiny = np.finfo(np.float64).tiny
    lam_ref = O.RIDGE_REL * tiny
    for _ in range(O.RIDGE_TRIES):
        lam_ref *= 10.0
    for i, g in enumerate(orc):
        st = g.state()
        for h in range(H):
            assert st["tries"][h] == tries[i, h] == O.RIDGE_TRIES + 1
            assert st["lambda"][h] == lam[i, h] == lam_ref
            assert np.array_equal(mu[i, h], st["mu"][h])
    assert np.isposinf(np.diagonal(mu, axis1=-2, axis2=-1)).all()
    info = grp.info()
    assert info.heads_fallback == G * H and info.tries_max == O.RIDGE_TRIES + 1


def test_info_memory_bytes_and_ridge_summary_match_oracle():
    wl = W.Workload("info", 2, 2, 2, 2, 128, 128, 32, 64, 4, T=256, steps=12, q_std=2.0,
                    k_std=2.0, seed=43)
    G, H = wl.groups, wl.hpk
    q, k, v = W.prompt(wl, DEV)
    orc = oracle_prefill(wl, cpu(q), cpu(k), cpu(v))
    grp = P.O1Groups(wl.config)
    info = grp.info()
    assert info.page_bytes == 0 and info.ridge_heads == 0  # nothing sealed yet
    grp.prefill(q, k, v)
    info = grp.info()
    page = sum(g.memory_bytes() for g in orc)
    assert info.page_bytes == page, (info.page_bytes, page)
    lam = np.sort(np.concatenate([g.state()["lambda"] for g in orc]))
    assert info.ridge_heads == G * H == lam.size
    assert info.tries_max == 1 and info.heads_retried == 0 and info.heads_fallback == 0
    for got, ref in ((info.lambda_min, lam[0]), (info.lambda_max, lam[-1]),
                     (info.lambda_median, np.median(lam))):
        assert abs(got - ref) <= 1e-12 * ref, (got, ref)
    m_cap = min(wl.m, 64)
    assert info.fold_bytes == G * 8 * wl.dv * 4 + G * H * 8 * m_cap * 8 + G * H * m_cap * 4
    assert info.ring_logit_bytes == G * wl.w * H * m_cap * 8
    assert info.page_bytes < info.state_bytes
    out = torch.empty(G, H, wl.dv, device=DEV)
    for t in range(wl.steps):
        qq, kk, vv = W.decode_inputs(wl, t, DEV)
        grp.step(qq, kk, vv, out)
        for i, g in enumerate(orc):
            g.step(cpu(qq[i]), cpu(kk[i]), cpu(vv[i]))
    assert grp.info().page_bytes == sum(g.memory_bytes() for g in orc)
    say(f"  page memory_bytes {info.page_bytes} of {info.state_bytes} device bytes "
        f"(fold {info.fold_bytes}, ring logits {info.ring_logit_bytes}); lambda "
        f"{info.lambda_min:.3e} / {info.lambda_median:.3e} / {info.lambda_max:.3e}")


def test_info_memory_bytes_exact_only_matches_oracle():
    wl = W.Workload("info_exact", 2, 1, 2, 2, 64, 64, 8, 16, 2, T=20, steps=5,
                    seed=44)
    G = wl.groups
    q, k, v = W.prompt(wl, DEV)
    orc = oracle_prefill(wl, cpu(q), cpu(k), cpu(v))
    assert all(g.exact_only for g in orc)
    grp = P.O1Groups(P.Config(**{**wl.config.__dict__, "exact_cap": 64}))
    grp.prefill(q, k, v)
    info = grp.info()
    assert info.exact_only == 1 and info.ridge_heads == 0
    assert info.page_bytes == sum(g.memory_bytes() for g in orc) == G * 4 * wl.T * (wl.d + wl.dv)
    out = torch.empty(G, wl.hpk, wl.dv, device=DEV)
    for t in range(wl.steps):
        qq, kk, vv = W.decode_inputs(wl, t, DEV)
        grp.step(qq, kk, vv, out)
        for i, g in enumerate(orc):
            g.step(cpu(qq[i]), cpu(kk[i]), cpu(vv[i]))
        assert grp.info().page_bytes == sum(g.memory_bytes() for g in orc), t


def test_far_len_write_mid_period_keeps_outputs():
    """A write of far_len alone, with evictions held, moves the step at which the
    next fold computes the far-insert logits of newly arrived keys.  far_len
    itself does not enter an output (only far_len > 0 does), so with the logits
    of every ring key recomputed at the write the outputs stay the oracle's
    through the evictions of every key that was in the ring then."""
    wl = W.Workload("far_len_write", 2, 1, 2, 2, 128, 128, 16, 32, 4, T=180, steps=0, q_std=2.0,
                    k_std=2.0, seed=45)
    G, H, dv = wl.groups, wl.hpk, wl.dv
    n1, n2 = 5, wl.w + 2 * P.FOLD_PERIOD
    E = wl.T - wl.sink - wl.w + n1
    assert E % P.FOLD_PERIOD > 3, "the write must land mid-period"
    q, k, v = W.prompt(wl, DEV)
    orc = oracle_prefill(wl, cpu(q), cpu(k), cpu(v))
    frozen = tuple(torch.from_numpy(np.stack([g.state()[n] for g in orc])).to(DEV)
                   for n in ("k_tilde", "q_tilde", "mu"))
    grp = P.O1Groups(wl.config)
    grp.prefill(q, k, v, frozen=frozen)
    steps = [W.decode_inputs(wl, t, DEV) for t in range(n1 + n2)]
    gout = []
    for t in range(n1 + n2):
        if t == n1:
            fl = grp.read(P.FIELD_FAR_LEN, device=DEV)
            assert (fl == E).all()
            grp.write(P.FIELD_FAR_LEN, (fl - 3).contiguous())
        out = torch.empty(G, H, dv, device=DEV)
        grp.step(*steps[t], out)
        gout.append(cpu(out).astype(np.float64))
    qs = np.stack([cpu(s[0]) for s in steps])
    ks = np.stack([cpu(s[1]) for s in steps])
    vs = np.stack([cpu(s[2]) for s in steps])
    out, alt, amb = oracle_decode(orc, qs, ks, vs)
    err = row_errors(np.stack(gout), out, alt, amb)
    say(f"  far_len written mid-period: max row error {err.max():.3e} over {err.size} rows")
    assert err.max() <= DECODE_TOL
    assert (grp.read(P.FIELD_FAR_LEN) == E - 3 + n2).all()
