"""GPU parity at head width d = dv = 80 against the oracle: the prefill freeze,
the decode steps, the exact comparator and the exact-only mode.  A row of 80
floats is 20 float4, whose largest power-of-two factor is 4: the row dots split
a key row over 4 lanes (5 float4 each), so one launch serves at most 4 query
heads and groups of more are stepped in blocks of 4 (8 heads in two, 6 in a
block of 4 and one of 2); the column passes give each value row 32 lanes, the
last 12 of which read its last column again and store nothing.  The shapes
cover 1 to 12 heads, m up to 64, windows below, at and above the fold period,
a 1024-group grid and the Fm rectifier."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
import streaming_nystr_attention_amd as P
from streaming_nystr_attention_amd import workloads as W

from parity_util import DECODE_TOL, cpu, decode_parity, oracle_decode, oracle_prefill, prefill_parity, \
    row_errors, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
D = 80


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    P.lib()
    yield


def _wl(name, n_seq, n_layer, n_kv, hpk, m, w, sink, T, steps, seed, std=1.0):
    return W.Workload(name, n_seq, n_layer, n_kv, hpk, D, D, m, w, sink, T=T, steps=steps,
                      q_std=std, k_std=std, seed=seed)


SHAPES = [
    # one head per KV head (multi-head attention), the page's default budget
    _wl("d80_h1_m32_w128", 2, 1, 8, 1, 32, 128, 4, T=256, steps=3 * P.FOLD_PERIOD, seed=801),
    _wl("d80_h2_m16_w7", 2, 1, 3, 2, 16, 7, 2, T=120, steps=20, seed=802, std=2.0),
    _wl("d80_h3_m24_w100", 1, 2, 2, 3, 24, 100, 3, T=200, steps=16, seed=803),
    _wl("d80_h4_m64_w64", 2, 1, 2, 4, 64, 64, 4, T=600, steps=20, seed=804, std=2.0),
    # more heads than one launch serves: blocks of 4
    _wl("d80_h6_m32_w9", 2, 1, 2, 6, 32, 9, 0, T=150, steps=3 * P.FOLD_PERIOD + 5, seed=805),
    _wl("d80_h8_m32_w64", 2, 1, 2, 8, 32, 64, 4, T=300, steps=20, seed=806, std=2.0),
    _wl("d80_h12_m40_w32", 1, 1, 3, 12, 40, 32, 2, T=400, steps=16, seed=807),
]


@pytest.mark.parametrize("wl", SHAPES, ids=[w.name for w in SHAPES])
def test_prefill_d80(wl):
    prefill_parity(wl)


@pytest.mark.parametrize("wl", SHAPES, ids=[w.name for w in SHAPES])
def test_decode_d80(wl):
    decode_parity(wl)


def test_decode_d80_fm_rectifier():
    decode_parity(_wl("d80_h2_fm", 2, 1, 2, 2, 16, 32, 2, T=120, steps=20, seed=808, std=2.0),
                  rect=O.RECT_FM)


def test_d80_large_grid():
    # 1024 groups: the 256-thread decode work-groups
    wl = _wl("d80_grid", 128, 1, 8, 4, 32, 64, 4, T=160, steps=12, seed=809)
    assert wl.groups >= 1024
    prefill_parity(wl, sample=W.groups_of_sequences(wl, W.sample_sequences(wl)))
    decode_parity(wl, sample=W.sample_groups(wl))


@pytest.mark.parametrize("G,H,cap,n,first,std", [
    (3, 1, 1000, 1000, 0, 2.0),      # split key range + combine
    (2048, 2, 200, 200, 0, 3.0),     # many groups: one work-group per group
    (2, 4, 400, 300, 100, 1.0),      # four heads, sliding-window start, ragged tail
    (5, 8, 300, 211, 7, 1.0),        # eight heads: two blocks of four
    (2, 7, 900, 900, 0, 1.0),        # blocks of 4 and 3, split key range
])
def test_exact_attend_d80(G, H, cap, n, first, std):
    say(f"[exact] G={G} hpk={H} d={D} cap={cap} n_keys={n} first={first}")
    g = torch.Generator(device=DEV).manual_seed(G * 13 + n)
    q = (std * torch.randn(G, H, D, device=DEV, generator=g)).contiguous()
    k = (std * torch.randn(G, cap, D, device=DEV, generator=g)).contiguous()
    v = torch.randn(G, cap, D, device=DEV, generator=g).contiguous()
    out = torch.empty(G, H, D, device=DEV)
    P.o1_exact_attend(q, k, v, out, n, first)
    torch.cuda.synchronize()
    qh, kh, vh, oh = q.cpu().numpy(), k.cpu().numpy(), v.cpu().numpy(), out.cpu().numpy()
    scale = O.f32_scale(D)
    check = range(G) if G <= 16 else [0, 1, G // 2, G - 1]
    worst = 0.0
    for gi in check:
        for h in range(H):
            ref = O.exact_attention(qh[gi, h], kh[gi, first:n], vh[gi, first:n], scale)
            worst = max(worst, np.abs(oh[gi, h] - ref).max() / np.linalg.norm(ref))
    say(f"  max row error {worst:.3e}")
    assert worst <= 1e-6


@pytest.mark.parametrize("hpk", [2, 6])
def test_exact_only_d80(hpk):
    """A prompt of T <= w + sink + 8 keeps every key; each step appends one."""
    wl = _wl(f"x_d80_h{hpk}", 2, 1, 2, hpk, 16, 64, 4, T=60, steps=20, seed=810 + hpk, std=2.0)
    cap = 80
    grp = P.O1Groups(dataclasses.replace(wl.config, exact_cap=cap))
    q, k, v = W.prompt(wl, DEV)
    grp.prefill(q, k, v)
    G, H = wl.groups, wl.hpk
    qs = torch.empty(wl.steps, G, H, D, device=DEV)
    ks = torch.empty(wl.steps, G, D, device=DEV)
    vs = torch.empty(wl.steps, G, D, device=DEV)
    outs = torch.empty(wl.steps, G, H, D, device=DEV)
    for t in range(wl.steps):
        W.decode_inputs(wl, t, DEV, out=(qs[t], ks[t], vs[t]))
        grp.step(qs[t], ks[t], vs[t], outs[t])
    torch.cuda.synchronize()
    orc = oracle_prefill(wl, cpu(q), cpu(k), cpu(v))
    assert all(g.exact_only for g in orc)
    out, alt, amb = oracle_decode(orc, cpu(qs), cpu(ks), cpu(vs))
    err = row_errors(cpu(outs).astype(np.float64), out, alt, amb)
    say(f"  max row error {err.max():.3e} over {err.size} rows")
    assert err.max() <= DECODE_TOL
    grp.close()
