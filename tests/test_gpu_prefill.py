"""GPU parity of the prefill freeze (o1_prefill computing everything itself)
against the CPU oracle on the same prompts.

  K~, Q~         equal to the oracle's f32 values (both sum the segment in row
                 order in f64 and round once); at most 1 ulp is allowed.
  M              judged by the residual ||A M A - A||_F / ||A||_F <= 1e-3 with the
                 oracle's f64 A, not elementwise (A is ill-conditioned).
  lambda, tries  lambda within 1e-12 relative, attempt number equal.
  far field      T^ e^{m_max} and Z^ e^{m_max} against the oracle's (which uses
                 the oracle's own landmarks), relative 1e-5 of each landmark row.
  ring, sinks,   bit-exact; counters bit-exact for every group.
"""
import numpy as np
import pytest
import torch

import streaming_nystr_attention_amd as P
from streaming_nystr_attention_amd import workloads as W

from parity_util import cpu, oracle_prefill, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
RESID_TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    P.lib()
    yield


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

    worst = {"lm_ulp": 0, "resid": 0.0, "lam": 0.0, "far": 0.0, "z": 0.0}
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
            worst["lam"] = max(worst["lam"], abs(lam[i, h] - st["lambda"][h]) / st["lambda"][h])
            assert tries[i, h] == st["tries"][h]
            # far field at a common scale: the oracle's running max
            shift = np.exp(mx[i, h] - st["m_max"][h])
            tg = th[i, h] * shift[:, None]
            rel = np.abs(tg - st["t_hat"][h]).max(1) / np.maximum(np.linalg.norm(st["t_hat"][h], axis=1), 1e-300)
            worst["far"] = max(worst["far"], rel.max())
            zr = np.abs(zh[i, h] * shift - st["z_hat"][h]) / st["z_hat"][h]
            worst["z"] = max(worst["z"], zr.max())
    say(f"  {worst}")
    grp.close()
    assert worst["lm_ulp"] <= 1
    assert worst["resid"] <= RESID_TOL
    assert worst["lam"] <= 1e-12
    assert worst["far"] <= 1e-5
    assert worst["z"] <= 1e-12


def test_prefill_single_head():
    prefill_parity(W.WORKLOADS["single_head"])


def test_prefill_qwen3_layer():
    prefill_parity(W.WORKLOADS["qwen3_layer"])


@pytest.mark.parametrize("name", ["stress_m8_s0", "stress_m16_s4", "stress_m32_s4"])
def test_prefill_stress(name):
    wl = W.WORKLOADS[name]
    prefill_parity(wl, sample=W.sample_groups(wl, extra=2))


def test_prefill_wide_gqa():
    prefill_parity(W.WORKLOADS["wide_gqa"], sample=[0, 5, 131, 255])


def test_prefill_qwen3_stack_full_size():
    wl = W.WORKLOADS["qwen3_stack_b64"]
    prefill_parity(wl, sample=W.sample_groups(wl, extra=4))


def test_prefill_ragged_segments():
    prefill_parity(W.Workload("ragged", 3, 1, 2, 2, 128, 128, 32, 16, 2, T=100, steps=0, seed=11))


def test_prefill_prompt_longer_than_budget():
    # T / 8 above the budget: m_eff clamps to m (the warn-once case of the page)
    prefill_parity(W.Workload("clamped", 2, 1, 2, 2, 64, 64, 16, 32, 4, T=300, steps=0, seed=21))


@pytest.mark.parametrize("wl", [
    W.Workload("max_window_hpk4", 2, 1, 2, 4, 128, 128, 64, 1000, 24, T=1100, steps=0, q_std=2.0,
               k_std=2.0, seed=16),
    W.Workload("max_heads_d64", 2, 1, 2, 8, 64, 64, 64, 500, 12, T=700, steps=0, seed=17),
], ids=["max_window_hpk4", "max_heads_d64"])
def test_prefill_maximum_sizes(wl):
    """The largest compiled near block (sink + w = 1024) and head count (hpk 8),
    both with m = 64."""
    prefill_parity(wl)
