"""GPU parity with long exact windows (sink + w up to 4096) against the oracle.
The near logits of a launch's heads sit in LDS (compiled heads x (sink + w)
doubles, at most 32 KB), so a window of 4092 keys runs one head per block and
one of 2040 two; every other pass loops over the window's rows.  The cases
check the prefill freeze (the window's keys span many landmark segments) and
the decode steps, a window at the limit for two heads, and the exact-only mode
of a prompt shorter than such a window (its keys split over work-groups)."""
import dataclasses

import numpy as np
import pytest
import torch

import streaming_nystr_attention_amd as P
from streaming_nystr_attention_amd import workloads as W

from parity_util import DECODE_TOL, cpu, decode_parity, oracle_decode, oracle_prefill, prefill_parity, \
    row_errors, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    P.lib()
    yield


def _wl(name, n_kv, hpk, d, m, w, sink, T, steps, seed, std=1.0):
    return W.Workload(name, 1, 1, n_kv, hpk, d, d, m, w, sink, T=T, steps=steps, q_std=std, k_std=std,
                      seed=seed)


CASES = [
    _wl("w4092_h1_d128", 2, 1, 128, 32, 4092, 4, T=4400, steps=20, seed=901, std=2.0),
    _wl("w2040_h2_d64", 2, 2, 64, 32, 2040, 8, T=2300, steps=20, seed=902),
    _wl("w1020_h3_d96", 1, 3, 96, 16, 1020, 4, T=1200, steps=12, seed=903),  # run as 4 heads: 4 x 1024
]


@pytest.mark.parametrize("wl", CASES, ids=[c.name for c in CASES])
def test_long_window_prefill_and_decode(wl):
    prefill_parity(wl)
    decode_parity(wl)


def test_long_window_exact_only():
    wl = _wl("x_w4000_h1", 2, 1, 128, 32, 4000, 4, T=3000, steps=10, seed=904, std=2.0)
    assert wl.T <= wl.w + wl.sink + 8
    cap = 3100
    grp = P.O1Groups(dataclasses.replace(wl.config, exact_cap=cap))
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
    assert all(g.exact_only for g in orc)
    out, alt, amb = oracle_decode(orc, cpu(qs), cpu(ks), cpu(vs))
    err = row_errors(cpu(outs).astype(np.float64), out, alt, amb)
    say(f"  max row error {err.max():.3e} over {err.size} rows")
    assert err.max() <= DECODE_TOL
    grp.close()
