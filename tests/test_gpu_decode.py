"""GPU parity of the decode step (o1_step) against the CPU oracle.

The GPU prefill runs with the oracle's frozen K~, Q~ and M (the `frozen` hook of
o1_prefill), so the decode outputs are compared at the decode tolerance
(1e-4 of the row norm) without the ill-conditioned pinv's elementwise spread.
Counters (far_len, win_head) are compared bit-exactly for every group, ring and
sink rows bit-exactly for the sampled groups.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
import streaming_nystr_attention_amd as P
from streaming_nystr_attention_amd import workloads as W

from parity_util import decode_parity

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    P.lib()  # raises when the HIP library is missing
    yield
    torch.cuda.synchronize()


def test_decode_single_head():
    decode_parity(W.WORKLOADS["single_head"])


def test_decode_qwen3_layer():
    decode_parity(W.WORKLOADS["qwen3_layer"])


def seq_sample(wl):
    """Every group of sequences {0, 1, B/2, B-1} and 4 seeded ones: all layers, KV
    heads, query heads and steps of those sequences."""
    return W.groups_of_sequences(wl, W.sample_sequences(wl))


@pytest.mark.parametrize("name", [f"stress_m{m}_s{s}" for m in (8, 16, 32) for s in (0, 4)])
def test_decode_stress(name):
    # 64 of 2048 groups, 8192 steps each
    wl = W.WORKLOADS[name]
    decode_parity(wl, sample=seq_sample(wl))


@pytest.mark.parametrize("part", range(4))
def test_decode_wide_gqa_all_groups(part):
    # every group of the wide GQA workload, all 2048 steps, in four parts of 8 sequences
    wl = W.WORKLOADS["wide_gqa"]
    n = wl.groups // 4
    decode_parity(wl, sample=list(range(part * n, (part + 1) * n)))


def test_decode_qwen3_stack_full_size():
    # the bench workload: 64 x 28 x 8 groups, 1024 steps; 8 whole sequences (1792 groups)
    wl = W.WORKLOADS["qwen3_stack_b64"]
    decode_parity(wl, sample=seq_sample(wl))


# ---- edge cases ----------------------------------------------------------

def test_decode_ragged_prompt_and_small_window():
    # T = 100: m_eff = 12 with 8- and 9-row segments; prompt just long enough
    wl = W.Workload("ragged", 3, 1, 2, 2, 128, 128, 32, 16, 2, T=100, steps=70, seed=11)
    decode_parity(wl)


def test_decode_shortest_skeleton_prompt():
    # T = w + sink + 9: the first prompt length with a skeleton (9 evictions)
    wl = W.Workload("shortest", 2, 1, 2, 4, 64, 64, 8, 24, 3, T=36, steps=40, seed=12)
    decode_parity(wl)


def test_decode_d64_hpk8_fm_rectifier():
    wl = W.Workload("d64_hpk8_fm", 2, 1, 3, 8, 64, 64, 16, 32, 4, T=200, steps=50, q_std=2.0,
                    k_std=2.0, seed=13)
    decode_parity(wl, rect=O.RECT_FM)


def test_decode_negative_mixing_drops_far_field():
    wl = W.Workload("neg_mu", 2, 1, 2, 2, 128, 128, 8, 16, 2, T=64, steps=20, seed=14)
    mu = -np.eye(wl.m_eff, dtype=np.float32)[None].repeat(wl.hpk, 0)
    decode_parity(wl, frozen_override=mu)


@pytest.mark.parametrize("w", [P.FOLD_PERIOD - 1, P.FOLD_PERIOD, P.FOLD_PERIOD + 1])
def test_decode_windows_around_the_fold_period(w):
    # w = FOLD_PERIOD is the shortest window whose keys get their far-insert
    # logits on a fold and keep them per ring slot (every slot is rewritten by
    # each fold); one less takes them from q~ at every eviction
    wl = W.Workload(f"w{w}", 2, 1, 2, 2, 128, 128, 16, w, 2, T=133 + w, steps=3 * P.FOLD_PERIOD + 5,
                    q_std=2.0, k_std=2.0, seed=40 + w)
    decode_parity(wl)


def test_decode_hpk1_window1():
    wl = W.Workload("w1", 2, 1, 1, 1, 128, 128, 4, 1, 0, T=40, steps=30, seed=15)
    decode_parity(wl)


MAX_SIZES = [
    # the largest near block compiled, sink + w = 1024, with hpk 4 (the 32 KB of
    # near logits the kernel reserves) and the largest landmark count, m = 64
    W.Workload("max_window_hpk4", 2, 1, 2, 4, 128, 128, 64, 1000, 24, T=1100, steps=40,
               q_std=2.0, k_std=2.0, seed=16),
    # the most heads, hpk 8, at d = 64 with sink + w = 512 and m = 64
    W.Workload("max_heads_d64", 2, 1, 2, 8, 64, 64, 64, 500, 12, T=700, steps=30, seed=17),
]


LARGE_GRIDS = [
    # 2048 groups: 256-thread decode work-groups, and the prefill's ring-key
    # logits take all of a group's heads in one work-group (4 and 8 heads)
    W.Workload("grid_hpk4", 256, 1, 8, 4, 128, 128, 32, 64, 4, T=300, steps=20, q_std=2.0,
               k_std=2.0, seed=18),
    W.Workload("grid_hpk8_d64", 256, 1, 8, 8, 64, 64, 16, 32, 2, T=200, steps=20, seed=19),
]


@pytest.mark.parametrize("wl", LARGE_GRIDS, ids=[w.name for w in LARGE_GRIDS])
def test_decode_large_grid_many_heads(wl):
    assert wl.groups >= 2048
    decode_parity(wl, sample=W.sample_groups(wl))


@pytest.mark.parametrize("wl", MAX_SIZES, ids=[w.name for w in MAX_SIZES])
def test_decode_maximum_sizes(wl):
    assert wl.hpk * (wl.sink + wl.w) * 8 == 32 * 1024 and wl.m_eff == 64
    decode_parity(wl)


def test_gqa_group_equals_single_head_groups_bitwise():
    wl = W.WORKLOADS["qwen3_layer"].with_(n_kv=4, steps=30)
    q, k, v = W.prompt(wl, DEV)
    grp = P.O1Groups(wl.config)
    grp.prefill(q, k, v)
    singles = []
    for h in range(wl.hpk):
        s = P.O1Groups(wl.config.__class__(**{**wl.config.__dict__, "hpk": 1}))
        s.prefill(q[:, h:h + 1].contiguous(), k, v)
        singles.append(s)
    G = wl.groups
    out = torch.empty(G, wl.hpk, wl.dv, device=DEV)
    o1 = torch.empty(G, 1, wl.dv, device=DEV)
    for t in range(wl.steps):
        qq, kk, vv = W.decode_inputs(wl, t, DEV)
        grp.step(qq, kk, vv, out)
        for h, s in enumerate(singles):
            s.step(qq[:, h:h + 1].contiguous(), kk, vv, o1)
            assert torch.equal(o1[:, 0], out[:, h]), (t, h)


def test_entry_point_errors_on_device():
    wl = W.WORKLOADS["single_head"]
    grp = P.O1Groups(wl.config)
    G = wl.groups
    q = torch.zeros(G, 1, 64, device=DEV)
    k = torch.zeros(G, 64, device=DEV)
    v = torch.zeros(G, 64, device=DEV)
    out = torch.zeros(G, 1, 64, device=DEV)
    with pytest.raises(P.O1Error) as e:
        grp.step(q, k, v, out)
    assert e.value.status == P.O1_ESTATE
    T = wl.w + wl.sink + 8
    qp = torch.zeros(G, 1, T, 64, device=DEV)
    kp = torch.zeros(G, T, 64, device=DEV)
    with pytest.raises(P.O1Error) as e:
        grp.prefill(qp, kp, kp.clone())
    assert e.value.status == P.O1_EEXACT
    with pytest.raises(P.O1Error) as e:
        grp.write(P.FIELD_T_HAT, torch.zeros(4, device=DEV))
    assert e.value.status == P.O1_ESTATE
    # an empty prompt is refused through the C ABI itself (valid device buffers)
    L = P.lib()
    pv = P.o1_prompt_view()
    pv.q, pv.k, pv.v = qp.data_ptr(), kp.data_ptr(), kp.data_ptr()
    for T0 in (0, -3):
        assert L.o1_prefill(grp._h, qp.data_ptr(), kp.data_ptr(), kp.data_ptr(), T0, None, None) == P.O1_EINVAL
        assert L.o1_prefill_layer(grp._h, 0, ctypes.byref(pv), T0, None, None) == P.O1_EINVAL
        assert b"prompt length" in L.o1_last_error()
    info = grp.info()
    assert info.sealed == 0 and info.n_groups == G
