"""GPU tests of the state interface: field copies, partial frozen prefills,
re-prefill on a handle, and the info record."""
import numpy as np
import pytest
import torch

import oracle as O
import streaming_nystr_attention_amd as P
from streaming_nystr_attention_amd import workloads as W

from parity_util import DECODE_TOL, DecodeRun, cpu, oracle_decode, oracle_prefill, row_errors, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    P.lib()
    yield


WL = W.Workload("state", 2, 1, 3, 2, 128, 128, 16, 32, 4, T=180, steps=40, q_std=2.0, k_std=2.0,
                seed=31)


# keys wider than values: every field's size follows its own width
WL192 = W.Workload("state_d192", 2, 1, 3, 3, 192, 128, 16, 32, 4, T=180, steps=40, q_std=2.0, k_std=2.0,
                   seed=32)


@pytest.mark.parametrize("wl", [WL, WL192], ids=["d128", "d192_dv128"])
def test_field_roundtrip_bit_exact(wl):
    G, H, m, R = wl.groups, wl.hpk, wl.m_eff, wl.sink + wl.w
    q, k, v = W.prompt(wl, DEV)
    grp = P.O1Groups(wl.config)
    grp.prefill(q, k, v)
    for field in range(12):
        a = grp.read(field, device=DEV)
        grp.write(field, torch.zeros_like(a))
        assert torch.count_nonzero(grp.read(field, device=DEV)) == 0
        grp.write(field, a)
        assert torch.equal(grp.read(field, device=DEV), a), field
        # host-side copies go through the same entry points
        h = grp.read(field, device="cpu")
        assert torch.equal(h.to(DEV), a)
    with pytest.raises(P.O1Error) as e:
        grp.write(P.FIELD_T_HAT, torch.zeros(3, device=DEV))
    assert e.value.status == P.O1_EINVAL
    # element counts: key-width fields d wide, value-width fields dv wide
    sizes = {P.FIELD_NEAR_K: G * R * wl.d, P.FIELD_NEAR_V: G * R * wl.dv, P.FIELD_K_TILDE: G * m * wl.d,
             P.FIELD_Q_TILDE: G * H * m * wl.d, P.FIELD_T_HAT: G * H * m * wl.dv, P.FIELD_MU: G * H * m * m}
    for field, n in sizes.items():
        assert grp.read(field, device=DEV).numel() == n, field
    grp.close()


@pytest.mark.parametrize("wl", [WL, WL192], ids=["d128", "d192_dv128"])
def test_decode_from_uploaded_oracle_far_field(wl):
    """Decode parity with the whole far field (T^, Z^, running max) taken from
    the oracle's sequential replay, so the decode kernel is checked apart from
    the prefill's far-field kernel."""
    G, H, m = wl.groups, wl.hpk, wl.m_eff
    q, k, v = W.prompt(wl, DEV)
    orc = oracle_prefill(wl, cpu(q), cpu(k), cpu(v))
    sts = [g.state() for g in orc]
    frozen = tuple(torch.from_numpy(np.stack([s[n] for s in sts])).to(DEV)
                   for n in ("k_tilde", "q_tilde", "mu"))
    grp = P.O1Groups(wl.config)
    grp.prefill(q, k, v, frozen=frozen)
    th = torch.from_numpy(np.stack([s["t_hat"] for s in sts]).astype(np.float32)).to(DEV)
    zh = torch.from_numpy(np.stack([s["z_hat"] for s in sts])).to(DEV)
    mx = torch.from_numpy(np.stack([s["m_max"] for s in sts]).astype(np.float32)).to(DEV)
    # the f32 running max must stay consistent with T^ and Z^: rescale them to it
    corr = torch.exp(torch.from_numpy(np.stack([s["m_max"] for s in sts])).to(DEV) - mx.double())
    grp.write(P.FIELD_T_HAT, (th.double() * corr[..., None]).float().contiguous().view(-1))
    grp.write(P.FIELD_Z_HAT, (zh * corr).contiguous().view(-1))
    grp.write(P.FIELD_M_MAX, mx.contiguous().view(-1))
    run = DecodeRun(wl, list(range(G)), wl.steps)
    qs, ks, vs, gout = run.run(grp)
    out, alt, amb = oracle_decode(orc, qs, ks, vs)
    err = row_errors(gout, out, alt, amb)
    say(f"  uploaded far field: max_err={err.max():.3e}")
    assert err.max() <= DECODE_TOL


def test_frozen_mixing_matrix_only():
    """frozen = (None, None, M): landmarks computed on the device, M given."""
    wl = WL
    G, H, m = wl.groups, wl.hpk, wl.m_eff
    q, k, v = W.prompt(wl, DEV)
    rng = np.random.default_rng(5)
    mu = (rng.standard_normal((G, H, m, m)) * 0.1).astype(np.float32)
    orc = oracle_prefill(wl, cpu(q), cpu(k), cpu(v), frozen=[O.Frozen(mu=mu[i]) for i in range(G)])
    grp = P.O1Groups(wl.config)
    grp.prefill(q, k, v, frozen=(None, None, torch.from_numpy(mu).to(DEV)))
    assert torch.equal(grp.read(P.FIELD_MU).view(G, H, m, m), torch.from_numpy(mu))
    kt = grp.read(P.FIELD_K_TILDE).view(G, m, wl.d).numpy()
    for i, g in enumerate(orc):
        np.testing.assert_array_equal(kt[i], g.state()["k_tilde"])
    tries = grp.read(P.FIELD_TRIES).numpy()
    assert (tries == 0).all()
    run = DecodeRun(wl, list(range(G)), 20)
    qs, ks, vs, gout = run.run(grp)
    out, alt, amb = oracle_decode(orc, qs, ks, vs)
    err = row_errors(gout, out, alt, amb)
    say(f"  frozen M only: max_err={err.max():.3e}")
    assert err.max() <= DECODE_TOL


def test_reprefill_resets_state_and_info():
    wl = WL
    G = wl.groups
    grp = P.O1Groups(wl.config)
    info = grp.info()
    assert info.sealed == 0 and info.m_eff == 0 and info.state_bytes > 0
    q, k, v = W.prompt(wl, DEV)
    grp.prefill(q, k, v)
    out = torch.empty(G, wl.hpk, wl.dv, device=DEV)
    for t in range(5):
        grp.step(*W.decode_inputs(wl, t, DEV), out)
    info = grp.info()
    assert info.sealed == 1 and info.steps == 5 and info.prompt_len == wl.T and info.m_eff == wl.m_eff
    # a second, shorter prompt on the same handle: state as if freshly created
    wl2 = wl.with_(T=120, seed=32)
    q2, k2, v2 = W.prompt(wl2, DEV)
    grp.prefill(q2, k2, v2)
    info = grp.info()
    assert info.steps == 0 and info.prompt_len == 120 and info.m_eff == wl2.m_eff
    fresh = P.O1Groups(wl.config)
    fresh.prefill(q2, k2, v2)
    for field in range(12):
        assert torch.equal(grp.read(field), fresh.read(field)), field


def _stepped(wl, steps, dev=DEV):
    """A prefilled handle stepped `steps` times, with every step's output."""
    q, k, v = W.prompt(wl, dev)
    grp = P.O1Groups(wl.config)
    grp.prefill(q, k, v)
    outs = []
    for t in range(steps):
        out = torch.empty(wl.groups, wl.hpk, wl.dv, device=dev)
        grp.step(*W.decode_inputs(wl, t, dev), out)
        outs.append(out)
    return grp, outs


def test_t_hat_read_between_folds_matches_oracle_and_changes_nothing():
    """Read while evictions are held (far_len mod FOLD_PERIOD != 0), T^ is the
    oracle's far numerator (compared at a common scale, as for the prefill),
    and the read leaves the state as it was: later outputs equal, bit for bit,
    those of an identical handle that was not read."""
    wl = WL
    G, H, m, dv = wl.groups, wl.hpk, wl.m_eff, wl.dv
    n1, n2 = 13, 2 * P.FOLD_PERIOD + 3
    E = wl.T - wl.sink - wl.w + n1
    assert E % P.FOLD_PERIOD != 0, "the read must see held evictions"
    a, _ = _stepped(wl, n1)
    b, _ = _stepped(wl, n1)
    th = a.read(P.FIELD_T_HAT).view(G, H, m, dv).numpy().astype(np.float64)
    mx = a.read(P.FIELD_M_MAX).view(G, H, m).numpy().astype(np.float64)

    q, k, v = W.prompt(wl, DEV)
    orc = oracle_prefill(wl, cpu(q), cpu(k), cpu(v))
    qs = np.stack([cpu(W.decode_inputs(wl, t, DEV)[0]) for t in range(n1)])
    ks = np.stack([cpu(W.decode_inputs(wl, t, DEV)[1]) for t in range(n1)])
    vs = np.stack([cpu(W.decode_inputs(wl, t, DEV)[2]) for t in range(n1)])
    oracle_decode(orc, qs, ks, vs)
    worst = 0.0
    for i, g in enumerate(orc):
        st = g.state()
        for h in range(H):
            tg = th[i, h] * np.exp(mx[i, h] - st["m_max"][h])[:, None]
            ref = st["t_hat"][h]
            rel = np.abs(tg - ref).max(1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-300)
            worst = max(worst, rel.max())
    say(f"  T^ read between folds: max row error {worst:.3e}")
    assert worst <= 1e-5

    # the read changed nothing: both handles continue identically past a fold
    for t in range(n1, n1 + n2):
        oa = torch.empty(G, H, dv, device=DEV)
        ob = torch.empty(G, H, dv, device=DEV)
        qq, kk, vv = W.decode_inputs(wl, t, DEV)
        a.step(qq, kk, vv, oa)
        b.step(qq, kk, vv, ob)
        assert torch.equal(oa, ob), t
    for f in range(12):
        assert torch.equal(a.read(f), b.read(f)), f


def test_state_upload_between_folds_continues_the_same_outputs():
    """Every field read from a handle with evictions held, written into a fresh
    sealed handle (each write first adds that handle's own held evictions to
    its T^), continues with the same outputs to within rounding."""
    wl = WL
    G, H, dv = wl.groups, wl.hpk, wl.dv
    n1, n2 = 13, 2 * P.FOLD_PERIOD + 3
    a, _ = _stepped(wl, n1)
    b, _ = _stepped(wl.with_(seed=wl.seed + 100), 5)  # another state, its own held set
    for f in range(12):
        b.write(f, a.read(f))
    for f in range(12):
        assert torch.equal(a.read(f), b.read(f)), f
    worst = 0.0
    for t in range(n1, n1 + n2):
        oa = torch.empty(G, H, dv, device=DEV)
        ob = torch.empty(G, H, dv, device=DEV)
        qq, kk, vv = W.decode_inputs(wl, t, DEV)
        a.step(qq, kk, vv, oa)
        b.step(qq, kk, vv, ob)
        oa64, ob64 = oa.double(), ob.double()
        worst = max(worst, ((oa64 - ob64).abs().amax(-1) / oa64.norm(dim=-1)).max().item())
    say(f"  uploaded state: max row difference {worst:.3e}")
    assert worst <= 1e-5
