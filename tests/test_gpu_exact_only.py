"""GPU parity of the exact-only mode (NystromGroup::prefill_shared on the
nystrom.rs source page): a prompt of T <= w + sink + 8 tokens builds no
skeleton, every key stays exact and each decode step appends one key.  The HIP
path (o1_prefill / o1_step on a handle with exact_cap > 0) is compared with the
oracle's exact-only groups step by step; the stored window and the counters are
compared bit for bit."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
import streaming_nystr_attention_amd as P
from streaming_nystr_attention_amd import workloads as W

from parity_util import DECODE_TOL, cpu, oracle_decode, oracle_prefill, row_errors, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    P.lib()
    yield


def _wl(name, n_seq, n_layer, n_kv, hpk, d, m, w, sink, T, steps, seed, dv=None):
    return W.Workload(name, n_seq, n_layer, n_kv, hpk, d, d if dv is None else dv, m, w, sink, T=T,
                      steps=steps, q_std=2.0, k_std=2.0, seed=seed)


# (workload, exact_cap).  T runs from one key to the mode's upper bound
# w + sink + 8; the last case has one group, so its key range is split over
# work-groups (ceil(n / 128) of them) and the keys cross 1024 while it runs.
CASES = [
    (_wl("x_d64_h1_T1", 2, 1, 2, 1, 64, 8, 16, 2, T=1, steps=30, seed=41), 31),
    (_wl("x_d64_h1_T26", 2, 1, 2, 1, 64, 8, 16, 2, T=26, steps=20, seed=42), 64),
    (_wl("x_d128_h2_T140", 1, 2, 4, 2, 128, 32, 128, 4, T=140, steps=24, seed=43), 200),
    (_wl("x_d128_h8_T268", 2, 1, 2, 8, 128, 64, 256, 4, T=268, steps=8, seed=44), 276),
    (_wl("x_d64_h4_split", 1, 1, 1, 4, 64, 16, 1000, 8, T=1010, steps=30, seed=45), 1040),
    (_wl("x_d128_h3_T100", 2, 1, 3, 3, 128, 16, 96, 4, T=100, steps=12, seed=46), 120),
    (_wl("x_d64_h6_split", 1, 1, 1, 6, 64, 8, 500, 2, T=505, steps=16, seed=47), 530),
    (_wl("x_d96_h2_T60", 2, 1, 2, 2, 96, 16, 64, 4, T=60, steps=20, seed=48), 80),
    (_wl("x_d96_h8_split", 1, 1, 1, 8, 96, 32, 500, 4, T=510, steps=12, seed=49), 530),
    (_wl("x_d256_h2_T60", 2, 1, 2, 2, 256, 16, 64, 4, T=60, steps=20, seed=50), 80),
    (_wl("x_d256_h4_split", 1, 1, 1, 4, 256, 32, 500, 4, T=510, steps=12, seed=51), 530),
    (_wl("x_d128_h12_T140", 2, 1, 2, 12, 128, 32, 128, 4, T=140, steps=24, seed=52), 200),
    (_wl("x_d64_h16_split", 1, 1, 1, 16, 64, 8, 500, 2, T=505, steps=16, seed=53), 530),
    # keys of 192 floats with values of 128
    (_wl("x_d192_h2_T60", 2, 1, 2, 2, 192, 16, 64, 4, T=60, steps=20, seed=54, dv=128), 80),
    (_wl("x_d192_h8_split", 1, 1, 1, 8, 192, 32, 500, 4, T=510, steps=12, seed=55, dv=128), 530),
    # 32 heads over one KV head: four blocks
    (_wl("x_d128_h32_split", 1, 1, 1, 32, 128, 16, 500, 4, T=510, steps=12, seed=56), 530),
]


def _run_exact(wl, cap, grp=None):
    """Exact-only prefill + wl.steps decode steps on the GPU.  Returns the
    handle, host copies of the inputs and the outputs [steps][G][hpk][dv]."""
    cfg = dataclasses.replace(wl.config, exact_cap=cap)
    if grp is None:
        grp = P.O1Groups(cfg)
    q, k, v = W.prompt(wl, DEV)
    grp.prefill(q, k, v)
    G, H = wl.groups, wl.hpk
    qs = torch.empty(wl.steps, G, H, wl.d, device=DEV)
    ks = torch.empty(wl.steps, G, wl.d, device=DEV)
    vs = torch.empty(wl.steps, G, wl.dv, device=DEV)
    outs = torch.empty(wl.steps, G, H, wl.dv, device=DEV)
    for t in range(wl.steps):
        W.decode_inputs(wl, t, DEV, out=(qs[t], ks[t], vs[t]))
        grp.step(qs[t], ks[t], vs[t], outs[t])
    torch.cuda.synchronize()
    return grp, (cpu(q), cpu(k), cpu(v)), (cpu(qs), cpu(ks), cpu(vs)), cpu(outs).astype(np.float64)


@pytest.mark.parametrize("wl,cap", CASES, ids=[c[0].name for c in CASES])
def test_exact_only_decode_matches_oracle(wl, cap):
    say(f"exact-only {wl.name}: G={wl.groups} hpk={wl.hpk} d={wl.d} T={wl.T} steps={wl.steps} cap={cap}")
    assert wl.T <= wl.w + wl.sink + 8
    grp, (qh, kh, vh), (qs, ks, vs), gpu = _run_exact(wl, cap)
    orc = oracle_prefill(wl, qh, kh, vh)
    assert all(g.exact_only for g in orc)
    out, alt, amb = oracle_decode(orc, qs, ks, vs)
    assert not amb.any()  # no far field, so no rectifier decision
    err = row_errors(gpu, out, alt, amb)
    say(f"  max row error {err.max():.3e} over {err.size} rows")
    assert err.max() <= DECODE_TOL

    # the window holds the prompt and then every appended key, bit for bit
    G, T, S = wl.groups, wl.T, wl.steps
    ek = grp.read(P.FIELD_EXACT_K).view(G, cap, wl.d).numpy()
    ev = grp.read(P.FIELD_EXACT_V).view(G, cap, wl.dv).numpy()
    assert np.array_equal(ek[:, :T], kh) and np.array_equal(ev[:, :T], vh)
    assert np.array_equal(ek[:, T:T + S], ks.transpose(1, 0, 2))
    assert np.array_equal(ev[:, T:T + S], vs.transpose(1, 0, 2))
    for i, g in enumerate(orc):
        assert g.win_len == T + S
        st = g.state()
        assert np.array_equal(st["win_k"], ek[i, :T + S])
    assert torch.count_nonzero(grp.read(P.FIELD_FAR_LEN)) == 0
    assert torch.count_nonzero(grp.read(P.FIELD_WIN_HEAD)) == 0
    info = grp.info()
    assert (info.sealed, info.exact_only, info.m_eff, info.prompt_len) == (1, 1, 0, T)
    assert info.exact_keys == T + S and info.steps == S
    with pytest.raises(P.O1Error) as e:
        grp.read(P.FIELD_T_HAT)
    assert e.value.status == P.O1_ESTATE
    grp.close()


def test_exact_only_full_window_is_refused_and_changes_nothing():
    wl, _ = CASES[1]
    wl = wl.with_(steps=3)
    cap = wl.T + wl.steps
    grp, _, _, _ = _run_exact(wl, cap)
    ek = grp.read(P.FIELD_EXACT_K, device=DEV)
    q, k, v = W.decode_inputs(wl, 99, DEV)
    out = torch.full((wl.groups, wl.hpk, wl.dv), float("nan"), device=DEV)
    with pytest.raises(P.O1Error) as e:
        grp.step(q, k, v, out)
    assert e.value.status == P.O1_EFULL
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
    assert torch.equal(grp.read(P.FIELD_EXACT_K, device=DEV), ek)
    info = grp.info()
    assert info.steps == wl.steps and info.exact_keys == cap
    # a prompt longer than the buffers is refused at prefill
    small = dataclasses.replace(wl.config, exact_cap=wl.T - 1)
    with P.O1Groups(small) as g2:
        pq, pk, pv = W.prompt(wl, DEV)
        with pytest.raises(P.O1Error) as e:
            g2.prefill(pq, pk, pv)
        assert e.value.status == P.O1_EFULL
        assert g2.info().sealed == 0
    grp.close()


def test_exact_only_prefill_ignores_queries():
    wl, cap = CASES[2]
    wl = wl.with_(steps=4)
    grp, _, (qs, ks, vs), ref = _run_exact(wl, cap)
    # same prompt keys, no queries: identical outputs
    cfg = dataclasses.replace(wl.config, exact_cap=cap)
    with P.O1Groups(cfg) as g2:
        _, k, v = W.prompt(wl, DEV)
        g2.prefill(None, k, v)
        out = torch.empty(wl.groups, wl.hpk, wl.dv, device=DEV)
        for t in range(wl.steps):
            g2.step(torch.from_numpy(qs[t]).to(DEV), torch.from_numpy(ks[t]).to(DEV),
                    torch.from_numpy(vs[t]).to(DEV), out)
            assert np.array_equal(cpu(out).astype(np.float64), ref[t])
    grp.close()


def test_mode_switch_on_one_handle():
    """skeleton -> exact-only -> skeleton prefills on the same handle, each
    followed by decode steps checked against a fresh oracle group."""
    base = W.Workload("x_switch", 1, 2, 2, 2, 128, 128, 16, 32, 4, T=180, steps=12, q_std=2.0,
                      k_std=2.0, seed=46)
    cap = 80
    cfg = dataclasses.replace(base.config, exact_cap=cap)
    grp = P.O1Groups(cfg)
    for wl in (base, base.with_(T=30, seed=47), base.with_(T=200, seed=48)):
        exact = wl.T <= wl.w + wl.sink + 8
        q, k, v = W.prompt(wl, DEV)
        grp.prefill(q, k, v)
        G, H = wl.groups, wl.hpk
        qs = torch.empty(wl.steps, G, H, wl.d, device=DEV)
        ks = torch.empty(wl.steps, G, wl.d, device=DEV)
        vs = torch.empty(wl.steps, G, wl.dv, device=DEV)
        outs = torch.empty(wl.steps, G, H, wl.dv, device=DEV)
        for t in range(wl.steps):
            W.decode_inputs(wl, t, DEV, out=(qs[t], ks[t], vs[t]))
            grp.step(qs[t], ks[t], vs[t], outs[t])
        torch.cuda.synchronize()
        orc = oracle_prefill(wl, cpu(q), cpu(k), cpu(v))
        out, alt, amb = oracle_decode(orc, cpu(qs), cpu(ks), cpu(vs))
        err = row_errors(cpu(outs).astype(np.float64), out, alt, amb)
        info = grp.info()
        say(f"  T={wl.T} exact_only={info.exact_only} max row error {err.max():.3e}")
        assert info.exact_only == int(exact)
        assert info.exact_keys == (wl.T + wl.steps if exact else wl.sink + wl.w)
        assert err.max() <= DECODE_TOL
        if not exact:
            far = grp.read(P.FIELD_FAR_LEN).view(G, H).numpy()
            assert (far == wl.T - wl.sink - wl.w + wl.steps).all()
    grp.close()
