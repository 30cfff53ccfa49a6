"""GPU parity at head width d = dv = 256 against the oracle: the prefill freeze
and the decode steps, as the tests at d in {64, 96, 128} check them.  A row of
256 floats is 64 float4: the decode's row passes split a key row over 8, 16 or
32 lanes (8, 4 or 2 float4 each), its column passes give each value row a whole
wave (so it always runs 512-thread work-groups, eight row lanes for the held
rows), and above m = 32 the landmark pass takes the components in two chunks
(its f64 K~ and Q~ at full width would not fit in LDS), keeping the partial
exp-Gram dots in global memory between them.  The shapes cover every compiled
head count (1, 2, 4, 8 and the partial group of 3), m up to 64, windows below,
at and above the fold period, a 1024-group grid and the Fm rectifier."""
import pytest
import torch

import oracle as O
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


def _wl(name, n_seq, n_layer, n_kv, hpk, m, w, sink, T, steps, seed, std=1.0):
    return W.Workload(name, n_seq, n_layer, n_kv, hpk, 256, 256, m, w, sink, T=T, steps=steps,
                      q_std=std, k_std=std, seed=seed)


SHAPES = [
    # two query heads per KV head, the page's default budget
    _wl("d256_h2_m32_w128", 2, 1, 8, 2, 32, 128, 4, T=256, steps=3 * P.FOLD_PERIOD, seed=81),
    # eight heads
    _wl("d256_h8_m32_w64", 2, 1, 2, 8, 32, 64, 4, T=300, steps=20, seed=82, std=2.0),
    # a window below the fold period: the far-insert logits are taken per step
    _wl("d256_h4_m16_w7", 2, 1, 3, 4, 16, 7, 2, T=120, steps=20, seed=83),
    # one head just above the fold period, no sinks
    _wl("d256_h1_m8_w9", 2, 1, 2, 1, 8, 9, 0, T=90, steps=3 * P.FOLD_PERIOD + 5, seed=84, std=2.0),
    # three heads (run as four), m not a multiple of 16
    _wl("d256_h3_m24_w100", 1, 2, 2, 3, 24, 100, 3, T=200, steps=16, seed=85),
    # m = 64: the landmark pass in two component chunks, the 64-landmark kernels
    _wl("d256_h2_m64_w128", 2, 1, 4, 2, 64, 128, 4, T=600, steps=3 * P.FOLD_PERIOD, seed=87, std=2.0),
    # m = 40 (three 16-row tiles), eight heads
    _wl("d256_h8_m40_w64", 2, 1, 2, 8, 40, 64, 2, T=400, steps=20, seed=88),
    # m = 48, a window below the fold period, five heads (run as eight)
    _wl("d256_h5_m48_w5", 2, 1, 2, 5, 48, 5, 3, T=420, steps=20, seed=89),
]


@pytest.mark.parametrize("wl", SHAPES, ids=[w.name for w in SHAPES])
def test_prefill_d256(wl):
    prefill_parity(wl)


@pytest.mark.parametrize("wl", SHAPES, ids=[w.name for w in SHAPES])
def test_decode_d256(wl):
    decode_parity(wl)


def test_decode_d256_fm_rectifier():
    decode_parity(_wl("d256_h2_fm", 2, 1, 2, 2, 16, 32, 2, T=120, steps=20, seed=86, std=2.0),
                  rect=O.RECT_FM)


def test_d256_large_grid():
    # 1024 groups: still 512-thread decode work-groups at this width
    wl = _wl("d256_grid", 128, 1, 8, 2, 32, 64, 4, T=160, steps=12, seed=87)
    assert wl.groups >= 1024
    prefill_parity(wl, sample=W.groups_of_sequences(wl, W.sample_sequences(wl)))
    decode_parity(wl, sample=W.sample_groups(wl))


def test_d256_rejects_more_than_64_landmarks():
    cfg = P.Config(n_seq=1, n_layer=1, n_kv=1, hpk=2, d=256, dv=256, m=65, w=16, sink=2)
    with pytest.raises(P.O1Error) as e:
        P.O1Groups(cfg)
    assert e.value.status == P.O1_EUNSUPPORTED
