"""GPU tests of per-layer sealing and stepping (LayerKvCache::o1_seal / o1_step
on the docs.rs LayerKvCache page): o1_prefill_layer reads a model's query
trace and per-KV-head caches in place, o1_step_layer steps one layer of every
sequence.  Both run the same kernels as the whole-handle entry points with a
different group map, so their outputs and state must equal the whole-handle
path's bit for bit; a sampled group is also checked against the oracle."""
import dataclasses
import gc

import numpy as np
import pytest
import torch

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


WL = W.Workload("layers", n_seq=3, n_layer=4, n_kv=2, hpk=2, d=128, dv=128, m=16, w=32, sink=4,
                T=180, steps=12, q_std=2.0, k_std=2.0, seed=61)
# keys wider than values and a partial head group: a stride taken from the
# wrong width, or a head count taken from the compiled one, shows here
WL192 = W.Workload("layers_d192", n_seq=2, n_layer=3, n_kv=2, hpk=3, d=192, dv=128, m=16, w=32, sink=4,
                   T=150, steps=12, q_std=2.0, k_std=2.0, seed=63)


def _layer_groups(wl, layer):
    """State groups of one layer in call order (s, kv)."""
    return [(s * wl.n_layer + layer) * wl.n_kv + kv for s in range(wl.n_seq) for kv in range(wl.n_kv)]


def _model_buffers(wl, q, k, v, layer, cap):
    """The layer's prompt as a model holds it: a query trace [n_seq][T][H][d]
    (position-major) and per-KV-head caches [n_seq][n_kv][cap][d] whose rows
    past T are NaN, so a read outside the prompt would show."""
    B, K, H, T = wl.n_seq, wl.n_kv, wl.hpk, wl.T
    idx = torch.tensor(_layer_groups(wl, layer), device=DEV)
    trace = None
    if q is not None:
        ql = q.index_select(0, idx).view(B, K, H, T, wl.d)         # [s][kv][j][t][c]
        trace = ql.permute(0, 3, 1, 2, 4).reshape(B, T, K * H, wl.d).contiguous()
    kc = torch.full((B, K, cap, wl.d), float("nan"), device=DEV)
    vc = torch.full((B, K, cap, wl.dv), float("nan"), device=DEV)
    kc[:, :, :T] = k.index_select(0, idx).view(B, K, T, wl.d)
    vc[:, :, :T] = v.index_select(0, idx).view(B, K, T, wl.dv)
    return trace, kc, vc


def _seal_layers(grp, wl, q, k, v, frozen=None, cap=None):
    cap = cap or wl.T + 7
    for layer in reversed(range(wl.n_layer)):  # any order
        trace, kc, vc = _model_buffers(wl, q, k, v, layer, cap)
        fz = None
        if frozen is not None:
            idx = torch.tensor(_layer_groups(wl, layer), device=DEV)
            fz = tuple(f.index_select(0, idx).contiguous() for f in frozen)
        qv = None if q is None else trace.permute(0, 2, 1, 3)  # logical [s][head][t][c]
        grp.prefill_layer(layer, qv, kc, vc, T=wl.T, frozen=fz)


def _step_inputs(wl):
    G, H = wl.groups, wl.hpk
    qs = torch.empty(wl.steps, G, H, wl.d, device=DEV)
    ks = torch.empty(wl.steps, G, wl.d, device=DEV)
    vs = torch.empty(wl.steps, G, wl.dv, device=DEV)
    for t in range(wl.steps):
        W.decode_inputs(wl, t, DEV, out=(qs[t], ks[t], vs[t]))
    return qs, ks, vs


def _step_by_layer(grp, wl, qs, ks, vs):
    """Every token: each layer stepped on its own (layer order reversed on odd
    tokens); outputs gathered back into group order [steps][G][hpk][dv]."""
    B, K, H = wl.n_seq, wl.n_kv, wl.hpk
    out = torch.empty(wl.steps, wl.groups, H, wl.dv, device=DEV)
    ob = torch.empty(B, K * H, wl.dv, device=DEV)
    for t in range(wl.steps):
        order = range(wl.n_layer) if t % 2 == 0 else reversed(range(wl.n_layer))
        for layer in order:
            idx = torch.tensor(_layer_groups(wl, layer), device=DEV)
            q = qs[t].index_select(0, idx).view(B, K * H, wl.d).contiguous()
            k = ks[t].index_select(0, idx).view(B, K, wl.d).contiguous()
            v = vs[t].index_select(0, idx).view(B, K, wl.dv).contiguous()
            grp.step_layer(layer, q, k, v, ob)
            out[t].index_copy_(0, idx, ob.view(B * K, H, wl.dv))
    torch.cuda.synchronize()
    return out


def _step_whole(grp, wl, qs, ks, vs):
    out = torch.empty(wl.steps, wl.groups, wl.hpk, wl.dv, device=DEV)
    for t in range(wl.steps):
        grp.step(qs[t], ks[t], vs[t], out[t])
    torch.cuda.synchronize()
    return out


FIELDS = [P.FIELD_NEAR_K, P.FIELD_NEAR_V, P.FIELD_K_TILDE, P.FIELD_Q_TILDE, P.FIELD_MU,
          P.FIELD_T_HAT, P.FIELD_Z_HAT, P.FIELD_M_MAX, P.FIELD_WIN_HEAD, P.FIELD_FAR_LEN,
          P.FIELD_LAMBDA, P.FIELD_TRIES]


@pytest.mark.parametrize("wl", [WL, WL192], ids=["d128_h2", "d192_dv128_h3"])
@pytest.mark.parametrize("with_frozen", [False, True])
def test_layer_path_equals_whole_handle_bitwise(wl, with_frozen):
    q, k, v = W.prompt(wl, DEV)
    qs, ks, vs = _step_inputs(wl)
    whole = P.O1Groups(wl.config)
    frozen = None
    if with_frozen:
        # frozen arrays: the computed landmarks and M, perturbed so they differ
        whole.prefill(q, k, v)
        G, H, m = wl.groups, wl.hpk, wl.m_eff
        frozen = (whole.read(P.FIELD_K_TILDE, DEV).view(G, m, wl.d) * 1.01,
                  whole.read(P.FIELD_Q_TILDE, DEV).view(G, H, m, wl.d) * 0.99,
                  whole.read(P.FIELD_MU, DEV).view(G, H, m, m) * 1.02)
    whole.prefill(q, k, v, frozen=frozen)
    ref = _step_whole(whole, wl, qs, ks, vs)

    layered = P.O1Groups(wl.config)
    _seal_layers(layered, wl, q, k, v, frozen=frozen)
    info = layered.info()
    assert (info.sealed, info.layers_sealed, info.n_layer, info.prompt_len) == (1, wl.n_layer,
                                                                                 wl.n_layer, wl.T)
    got = _step_by_layer(layered, wl, qs, ks, vs)
    assert torch.equal(got, ref)
    for f in FIELDS:
        assert torch.equal(layered.read(f, DEV), whole.read(f, DEV)), f
    info = layered.info()
    assert info.steps == wl.steps and info.max_steps == wl.steps

    # one sampled group against the oracle, independently of the whole-handle path
    if not with_frozen:
        g = _layer_groups(wl, 2)[3]
        sub = wl.with_(n_seq=1, n_layer=1, n_kv=1)
        orc = oracle_prefill(sub, cpu(q[g:g + 1]), cpu(k[g:g + 1]), cpu(v[g:g + 1]))
        out, alt, amb = oracle_decode(orc, cpu(qs[:, g:g + 1]), cpu(ks[:, g:g + 1]),
                                      cpu(vs[:, g:g + 1]))
        err = row_errors(cpu(got[:, g:g + 1]).astype(np.float64), out, alt, amb)
        say(f"  group {g}: max row error {err.max():.3e}")
        assert err.max() <= DECODE_TOL
    whole.close()
    layered.close()


def test_layer_steps_are_counted_per_layer_and_new_prompt_unseals():
    wl = WL.with_(steps=3)
    q, k, v = W.prompt(wl, DEV)
    grp = P.O1Groups(wl.config)
    B, K, H = wl.n_seq, wl.n_kv, wl.hpk
    with pytest.raises(P.O1Error) as e:  # nothing sealed yet
        grp.step_layer(0, torch.zeros(B, K * H, wl.d, device=DEV), torch.zeros(B, K, wl.d, device=DEV),
                       torch.zeros(B, K, wl.dv, device=DEV), torch.empty(B, K * H, wl.dv, device=DEV))
    assert e.value.status == P.O1_ESTATE
    for layer in (0, 1):
        trace, kc, vc = _model_buffers(wl, q, k, v, layer, wl.T)
        grp.prefill_layer(layer, trace.permute(0, 2, 1, 3), kc, vc)
    info = grp.info()
    assert (info.sealed, info.layers_sealed) == (0, 2)
    qb = torch.randn(B, K * H, wl.d, device=DEV)
    kb = torch.randn(B, K, wl.d, device=DEV)
    vb = torch.randn(B, K, wl.dv, device=DEV)
    ob = torch.empty(B, K * H, wl.dv, device=DEV)
    for _ in range(3):
        grp.step_layer(1, qb, kb, vb, ob)
    grp.step_layer(0, qb, kb, vb, ob)
    info = grp.info()
    assert (info.steps, info.max_steps) == (1, 3)
    with pytest.raises(P.O1Error) as e:  # whole-handle step needs every layer
        grp.step(torch.zeros(wl.groups, H, wl.d, device=DEV), torch.zeros(wl.groups, wl.d, device=DEV),
                 torch.zeros(wl.groups, wl.dv, device=DEV), torch.empty(wl.groups, H, wl.dv, device=DEV))
    assert e.value.status == P.O1_ESTATE
    with pytest.raises(P.O1Error) as e:
        grp.step_layer(wl.n_layer, qb, kb, vb, ob)
    assert e.value.status == P.O1_EINVAL
    far = grp.read(P.FIELD_FAR_LEN).view(wl.n_seq, wl.n_layer, K, H).numpy()
    base = wl.T - wl.sink - wl.w
    assert (far[:, 0] == base + 1).all() and (far[:, 1] == base + 3).all()

    # a prompt of another length on layer 0 starts a new prompt: layer 1 is unsealed
    wl2 = wl.with_(T=200, seed=62)
    q2, k2, v2 = W.prompt(wl2, DEV)
    trace, kc, vc = _model_buffers(wl2, q2, k2, v2, 0, wl2.T)
    grp.prefill_layer(0, trace.permute(0, 2, 1, 3), kc, vc)
    info = grp.info()
    assert (info.layers_sealed, info.prompt_len, info.steps) == (1, 200, 0)
    with pytest.raises(P.O1Error) as e:
        grp.step_layer(1, qb, kb, vb, ob)
    assert e.value.status == P.O1_ESTATE
    grp.step_layer(0, qb, kb, vb, ob)
    grp.close()


def test_layer_path_exact_only_equals_whole_handle():
    wl = WL.with_(T=30, steps=9, seed=63)
    cap = wl.T + wl.steps
    cfg = dataclasses.replace(wl.config, exact_cap=cap)
    q, k, v = W.prompt(wl, DEV)
    qs, ks, vs = _step_inputs(wl)
    whole = P.O1Groups(cfg)
    whole.prefill(q, k, v)
    ref = _step_whole(whole, wl, qs, ks, vs)
    layered = P.O1Groups(cfg)
    _seal_layers(layered, wl, None, k, v, cap=wl.T + 3)  # no query trace needed
    info = layered.info()
    assert (info.sealed, info.exact_only, info.m_eff) == (1, 1, 0)
    got = _step_by_layer(layered, wl, qs, ks, vs)
    assert torch.equal(got, ref)
    for f in (P.FIELD_EXACT_K, P.FIELD_EXACT_V, P.FIELD_FAR_LEN, P.FIELD_WIN_HEAD):
        assert torch.equal(layered.read(f, DEV), whole.read(f, DEV)), f
    B, K, H = wl.n_seq, wl.n_kv, wl.hpk
    with pytest.raises(P.O1Error) as e:  # every layer's window is full now
        layered.step_layer(2, torch.zeros(B, K * H, wl.d, device=DEV),
                           torch.zeros(B, K, wl.d, device=DEV), torch.zeros(B, K, wl.dv, device=DEV),
                           torch.empty(B, K * H, wl.dv, device=DEV))
    assert e.value.status == P.O1_EFULL
    whole.close()
    layered.close()


def _layer_slices(wl, layer, q, k, v):
    B, K, H = wl.n_seq, wl.n_kv, wl.hpk
    idx = torch.tensor(_layer_groups(wl, layer), device=DEV)
    return (idx, q.index_select(0, idx).view(B, K * H, wl.d).contiguous(),
            k.index_select(0, idx).view(B, K, wl.d).contiguous(),
            v.index_select(0, idx).view(B, K, wl.dv).contiguous())


def test_exact_only_whole_steps_after_unequal_layers():
    """Exact-only mode: each group's key count lives on the device, so after
    layer 0 alone took a step, whole-handle steps append every group at its own
    count.  They must equal stepping every layer on its own, bit for bit."""
    wl = WL.with_(T=30, steps=4, seed=64)
    cfg = dataclasses.replace(wl.config, exact_cap=wl.T + 8)
    q, k, v = W.prompt(wl, DEV)
    qs, ks, vs = _step_inputs(wl)
    whole, layered = P.O1Groups(cfg), P.O1Groups(cfg)
    B, K, H, L, G = wl.n_seq, wl.n_kv, wl.hpk, wl.n_layer, wl.groups
    ob = torch.empty(B, K * H, wl.dv, device=DEV)
    for grp in (whole, layered):
        grp.prefill(q, k, v)
        _, a, b, c = _layer_slices(wl, 0, qs[0], ks[0], vs[0])
        grp.step_layer(0, a, b, c, ob)  # layer 0 now holds one key more
    out_w = torch.empty(wl.steps, G, H, wl.dv, device=DEV)
    out_l = torch.empty_like(out_w)
    for t in range(1, wl.steps):
        whole.step(qs[t], ks[t], vs[t], out_w[t])
        for layer in range(L):
            idx, a, b, c = _layer_slices(wl, layer, qs[t], ks[t], vs[t])
            layered.step_layer(layer, a, b, c, ob)
            out_l[t].index_copy_(0, idx, ob.view(B * K, H, wl.dv))
    torch.cuda.synchronize()
    assert torch.equal(out_w[1:], out_l[1:])
    cap = cfg.exact_cap
    for f, width in ((P.FIELD_EXACT_K, wl.d), (P.FIELD_EXACT_V, wl.dv)):
        a, b = (h.read(f, DEV).view(G, cap, width) for h in (whole, layered))
        for layer in range(L):  # rows past a group's keys were never written
            held = wl.T + wl.steps - (0 if layer == 0 else 1)
            idx = torch.tensor(_layer_groups(wl, layer), device=DEV)
            assert torch.equal(a.index_select(0, idx)[:, :held], b.index_select(0, idx)[:, :held]), (f, layer)
    info = whole.info()
    assert (info.steps, info.max_steps, info.exact_keys) == (wl.steps - 1, wl.steps, wl.T + wl.steps)
    whole.close()
    layered.close()


def test_exact_only_graph_replays_match_eager_and_stop_at_cap():
    """A whole-handle exact-only step captured in a HIP graph: every replay
    reads the key count from the device, so replays with eager input copies
    and synchronisation between them equal the eager steps of a twin handle;
    once the groups hold exact_cap keys a replay changes nothing and writes no
    output (the eager twin is refused with O1_EFULL)."""
    wl = WL.with_(T=30, steps=5, seed=65)
    room = 3  # keys the cap leaves after the prompt
    cfg = dataclasses.replace(wl.config, exact_cap=wl.T + room)
    q, k, v = W.prompt(wl, DEV)
    qs, ks, vs = _step_inputs(wl)
    G, H = wl.groups, wl.hpk
    eager, graphed = P.O1Groups(cfg), P.O1Groups(cfg)
    eager.prefill(q, k, v)
    graphed.prefill(q, k, v)
    sq, sk, sv = torch.empty_like(qs[0]), torch.empty_like(ks[0]), torch.empty_like(vs[0])
    out_g = torch.empty(G, H, wl.dv, device=DEV)
    out_e = torch.empty_like(out_g)
    with P.O1Groups(cfg) as warm:  # first launch of this shape outside the capture
        warm.prefill(q, k, v)
        warm.step(qs[0], ks[0], vs[0], out_e)
        torch.cuda.synchronize()
    gc.collect()  # finalise leftover objects now: destroying a graph during a capture aborts
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        graphed.step(sq, sk, sv, out_g)
    for t in range(wl.steps):
        status = P.O1_OK
        try:  # (the except target is unbound on exit: no frame cycle keeps the graph alive)
            eager.step(qs[t], ks[t], vs[t], out_e)
        except P.O1Error as err:
            status = err.status
        assert status == (P.O1_OK if t < room else P.O1_EFULL), t
        sq.copy_(qs[t])
        sk.copy_(ks[t])
        sv.copy_(vs[t])
        out_g.fill_(7.0)
        graph.replay()
        torch.cuda.synchronize()
        if t < room:
            assert torch.equal(out_g, out_e), t
        else:
            assert (out_g == 7.0).all(), t
    for f in (P.FIELD_EXACT_K, P.FIELD_EXACT_V):
        assert torch.equal(graphed.read(f, DEV), eager.read(f, DEV)), f
    del graph  # destroyed here, outside any capture
    eager.close()
    graphed.close()


def test_graph_replay_of_layer_steps_matches_eager():
    """One token's o1_step_layer launches captured in a HIP graph and replayed
    several times, with eager input copies and synchronisation between the
    replays; every replay must equal the eager steps of a twin handle."""
    wl = WL.with_(steps=5)
    B, K, H, L = wl.n_seq, wl.n_kv, wl.hpk, wl.n_layer
    q, k, v = W.prompt(wl, DEV)
    qs, ks, vs = _step_inputs(wl)
    eager, graphed = P.O1Groups(wl.config), P.O1Groups(wl.config)
    eager.prefill(q, k, v)
    graphed.prefill(q, k, v)
    idx = [torch.tensor(_layer_groups(wl, l), device=DEV) for l in range(L)]

    def token_inputs(t):
        return (torch.stack([qs[t].index_select(0, i).view(B, K * H, wl.d) for i in idx]),
                torch.stack([ks[t].index_select(0, i).view(B, K, wl.d) for i in idx]),
                torch.stack([vs[t].index_select(0, i).view(B, K, wl.dv) for i in idx]))

    sq, sk, sv = (torch.empty_like(x) for x in token_inputs(0))
    out_g = torch.empty(L, B, K * H, wl.dv, device=DEV)
    out_e = torch.empty_like(out_g)
    with P.O1Groups(wl.config) as warm:  # first launch of this shape outside the capture
        warm.prefill(q, k, v)
        a, b, c = token_inputs(0)
        warm.step_layer(0, a[0], b[0], c[0], out_e[0])
        torch.cuda.synchronize()
    gc.collect()  # finalise leftover objects now: destroying a graph during a capture aborts
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for l in range(L):
            graphed.step_layer(l, sq[l], sk[l], sv[l], out_g[l])
    for t in range(wl.steps):
        a, b, c = token_inputs(t)
        for l in range(L):
            eager.step_layer(l, a[l], b[l], c[l], out_e[l])
        sq.copy_(a)
        sk.copy_(b)
        sv.copy_(c)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), t
    for f in FIELDS:
        assert torch.equal(graphed.read(f, DEV), eager.read(f, DEV)), f
    eager.close()
    graphed.close()
