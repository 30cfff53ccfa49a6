"""GPU parity at more than 8 query heads per KV head (9 to 16: e.g. 96 or 128
query heads over 8 KV heads; 24 to 64: attention with one or two KV heads).  The library steps such a group in blocks of at
most 8 heads, one launch each on the caller's stream; every block reads the
ring's old row for the evicted key, and the last block alone writes the new row,
the held value row and the ring position.  Each case checks the prefill freeze
and every decode step against the oracle as the fixed-shape tests do, on both
launch paths (512-thread work-groups for small grids, 256-thread ones from 1024
groups up, where 8-head blocks run two heads per wave)."""
import gc

import pytest
import torch

import streaming_nystr_attention_amd as P
from streaming_nystr_attention_amd import workloads as W

from parity_util import decode_parity, prefill_parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    P.lib()
    yield


def _wl(name, n_seq, n_kv, hpk, d, m, w, sink, T, steps, std, seed, dv=None):
    return W.Workload(name, n_seq, 1, n_kv, hpk, d, d if dv is None else dv, m, w, sink, T=T,
                      steps=steps, q_std=std, k_std=std, seed=seed)


CASES = [
    _wl("h12_d128", 2, 2, 12, 128, 32, 64, 4, 300, 40, 2.0, 81),    # blocks of 8 and 4 heads
    _wl("h16_d64", 2, 2, 16, 64, 16, 32, 2, 200, 30, 1.0, 82),      # two blocks of 8
    _wl("h9_d128_w7", 2, 2, 9, 128, 32, 7, 2, 200, 30, 2.0, 83),    # 8 + 1 heads; no per-slot logits
    _wl("h13_d96_m64", 2, 2, 13, 96, 64, 256, 4, 600, 24, 1.0, 84), # 8 + 5 (placeholders), m = 64
    _wl("h32_d128_kv1", 2, 1, 32, 128, 32, 64, 4, 300, 24, 2.0, 86),  # four blocks, one KV head
    _wl("h64_d64_kv1", 2, 1, 64, 64, 16, 32, 2, 200, 20, 1.0, 87),    # eight blocks
    _wl("h40_d128_w7", 2, 2, 40, 128, 32, 7, 2, 200, 20, 2.0, 88),    # five blocks; no per-slot logits
    _wl("h24_d192", 2, 1, 24, 192, 32, 64, 4, 300, 20, 1.0, 89, dv=128),  # three blocks, keys wider than values
]


@pytest.mark.parametrize("wl", CASES, ids=[c.name for c in CASES])
def test_many_heads_prefill_and_decode(wl):
    prefill_parity(wl)
    decode_parity(wl)


def test_many_heads_large_grid_sampled():
    """1024 groups of 16 heads at d = 128: 256-thread work-groups for both
    blocks; a declared sample of sequences is compared."""
    wl = _wl("h16_grid1024", 64, 16, 16, 128, 32, 64, 4, 300, 20, 2.0, 85)
    sample = W.groups_of_sequences(wl, W.sample_sequences(wl))
    prefill_parity(wl, sample=sample)
    decode_parity(wl, sample=sample)


@pytest.mark.parametrize("hpk,d", [(12, 128), (6, 80)], ids=["h12_d128", "h6_d80"])
def test_graph_replay_of_head_block_steps_matches_eager(hpk, d):
    """A whole-handle step of a group stepped in head blocks (8 + 4 heads at
    d = 128, 4 + 2 at d = 80) captured in a HIP graph and replayed, with eager
    input copies and synchronisation between the replays; every replay must
    equal the eager steps of a twin handle, and so must the state after."""
    wl = _wl(f"graph_h{hpk}_d{d}", 2, 2, hpk, d, 16, 32, 4, 120, 2 * 8 + 3, 2.0, 90 + hpk)
    G = wl.groups
    q, k, v = W.prompt(wl, "cuda")
    qs = torch.empty(wl.steps, G, hpk, d, device="cuda")
    ks = torch.empty(wl.steps, G, d, device="cuda")
    vs = torch.empty(wl.steps, G, d, device="cuda")
    for t in range(wl.steps):
        W.decode_inputs(wl, t, "cuda", out=(qs[t], ks[t], vs[t]))
    eager, graphed = P.O1Groups(wl.config), P.O1Groups(wl.config)
    eager.prefill(q, k, v)
    graphed.prefill(q, k, v)
    sq, sk, sv = torch.empty_like(qs[0]), torch.empty_like(ks[0]), torch.empty_like(vs[0])
    out_g = torch.empty(G, hpk, d, device="cuda")
    out_e = torch.empty_like(out_g)
    with P.O1Groups(wl.config) as warm:  # first launches of these kernels outside the capture
        warm.prefill(q, k, v)
        warm.step(qs[0], ks[0], vs[0], out_e)
        torch.cuda.synchronize()
    gc.collect()  # finalise leftover objects now: destroying a graph during a capture aborts
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        graphed.step(sq, sk, sv, out_g)
    for t in range(wl.steps):  # more than two fold periods
        eager.step(qs[t], ks[t], vs[t], out_e)
        sq.copy_(qs[t])
        sk.copy_(ks[t])
        sv.copy_(vs[t])
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), t
    for f in (P.FIELD_NEAR_K, P.FIELD_NEAR_V, P.FIELD_T_HAT, P.FIELD_Z_HAT, P.FIELD_M_MAX,
              P.FIELD_WIN_HEAD, P.FIELD_FAR_LEN):
        assert torch.equal(graphed.read(f, "cuda"), eager.read(f, "cuda")), f
    eager.close()
    graphed.close()
