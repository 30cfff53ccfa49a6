"""GPU parity with keys wider than values, d = 192 and dv = 128, against the
oracle: the prefill freeze, the decode steps and the exact comparator.  The
oracle keeps the two widths apart everywhere (K~, Q~ and the near keys are d
wide; T^, the near values and the outputs dv wide; the score scale is
1/sqrt(d)), so a kernel that indexes a value row by the key width, or the
reverse, fails here where the d == dv shapes cannot show it.  A key row of 192
floats is 48 float4: the decode's row passes split it over 8 or 16 lanes (6 or
3 float4 each) and always run 512-thread work-groups; the landmark pass takes
the components in two chunks above m = 32.  The shapes cover every compiled
head count (1, 2, 4, 8, partial groups of 3 and 5, and 12 heads in two
blocks), m up to 64, windows below, at and above the fold period, a
1024-group grid and the Fm rectifier."""
import numpy as np
import pytest
import torch

import oracle as O
import streaming_nystr_attention_amd as P
from streaming_nystr_attention_amd import workloads as W

from parity_util import decode_parity, prefill_parity, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
D, DV = 192, 128


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    P.lib()
    yield


def _wl(name, n_seq, n_layer, n_kv, hpk, m, w, sink, T, steps, seed, std=1.0):
    return W.Workload(name, n_seq, n_layer, n_kv, hpk, D, DV, m, w, sink, T=T, steps=steps,
                      q_std=std, k_std=std, seed=seed)


SHAPES = [
    # two query heads per KV head, the page's default budget
    _wl("d192_h2_m32_w128", 2, 1, 8, 2, 32, 128, 4, T=256, steps=3 * P.FOLD_PERIOD, seed=191),
    # eight heads
    _wl("d192_h8_m32_w64", 2, 1, 2, 8, 32, 64, 4, T=300, steps=20, seed=192, std=2.0),
    # a window below the fold period: the far-insert logits are taken per step
    _wl("d192_h4_m16_w7", 2, 1, 3, 4, 16, 7, 2, T=120, steps=20, seed=193),
    # one head just above the fold period, no sinks
    _wl("d192_h1_m8_w9", 2, 1, 2, 1, 8, 9, 0, T=90, steps=3 * P.FOLD_PERIOD + 5, seed=194, std=2.0),
    # three heads (run as four), m not a multiple of 16
    _wl("d192_h3_m24_w100", 1, 2, 2, 3, 24, 100, 3, T=200, steps=16, seed=195),
    # m = 64: the landmark pass in two component chunks, the 64-landmark kernels
    _wl("d192_h2_m64_w128", 2, 1, 4, 2, 64, 128, 4, T=600, steps=3 * P.FOLD_PERIOD, seed=196, std=2.0),
    # m = 40, five heads (run as eight)
    _wl("d192_h5_m40_w64", 2, 1, 2, 5, 40, 64, 2, T=400, steps=20, seed=197),
    # twelve heads: blocks of eight and four
    _wl("d192_h12_m32_w32", 1, 1, 3, 12, 32, 32, 4, T=180, steps=20, seed=198),
]


@pytest.mark.parametrize("wl", SHAPES, ids=[w.name for w in SHAPES])
def test_prefill_d192(wl):
    prefill_parity(wl)


@pytest.mark.parametrize("wl", SHAPES, ids=[w.name for w in SHAPES])
def test_decode_d192(wl):
    decode_parity(wl)


def test_decode_d192_fm_rectifier():
    decode_parity(_wl("d192_h2_fm", 2, 1, 2, 2, 16, 32, 2, T=120, steps=20, seed=199, std=2.0),
                  rect=O.RECT_FM)


def test_d192_large_grid():
    # 1024 groups: 512-thread decode work-groups at this key width too
    wl = _wl("d192_grid", 128, 1, 8, 2, 32, 64, 4, T=160, steps=12, seed=200)
    assert wl.groups >= 1024
    prefill_parity(wl, sample=W.groups_of_sequences(wl, W.sample_sequences(wl)))
    decode_parity(wl, sample=W.sample_groups(wl))


@pytest.mark.parametrize("G,H,cap,n,first,std", [
    (3, 2, 1000, 1000, 0, 2.0),      # split key range + combine
    (2048, 2, 200, 200, 0, 3.0),     # many groups: one work-group per group
    (2, 8, 400, 300, 100, 1.0),      # eight heads, sliding-window start, ragged tail
    (5, 3, 300, 211, 7, 1.0),        # 3 heads (run as 4)
    (2, 12, 300, 257, 3, 1.0),       # 12 heads: blocks of 8 and 4
])
def test_exact_attend_d192(G, H, cap, n, first, std):
    say(f"[exact] G={G} hpk={H} d={D} dv={DV} cap={cap} n_keys={n} first={first}")
    g = torch.Generator(device=DEV).manual_seed(G * 11 + n)
    q = (std * torch.randn(G, H, D, device=DEV, generator=g)).contiguous()
    k = (std * torch.randn(G, cap, D, device=DEV, generator=g)).contiguous()
    v = torch.randn(G, cap, DV, device=DEV, generator=g).contiguous()
    out = torch.empty(G, H, DV, device=DEV)
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


def test_d192_other_value_widths_are_refused():
    for dv in (64, 192, 256):
        cfg = P.Config(n_seq=1, n_layer=1, n_kv=1, hpk=2, d=D, dv=dv, m=16, w=16, sink=2)
        with pytest.raises(P.O1Error) as e:
            P.O1Groups(cfg)
        assert e.value.status == P.O1_EUNSUPPORTED
