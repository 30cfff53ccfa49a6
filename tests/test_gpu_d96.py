"""GPU parity at head width d = dv = 96 against the oracle: the prefill freeze
and the decode steps, as the tests at d in {64, 128} check them.  A row of 96
floats is 24 float4, which does not tile a 64-lane wave: the row passes split
it over 8 lanes (3 float4 each), and the column passes give each value row 32
lanes, the last 8 of which repeat its last column and store nothing.  The
shapes cover every compiled head count (1, 2, 4, 8 and the partial groups 3
and 6), m up to 64, windows below, at and above the fold period, both launch
widths (512 threads below 1024 groups, 256 at and above), and the Fm rectifier."""
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
    return W.Workload(name, n_seq, n_layer, n_kv, hpk, 96, 96, m, w, sink, T=T, steps=steps,
                      q_std=std, k_std=std, seed=seed)


SHAPES = [
    # the stack's per-group shape at d = 96
    _wl("d96_h2_m32_w128", 2, 1, 8, 2, 32, 128, 4, T=256, steps=3 * P.FOLD_PERIOD, seed=61),
    # eight heads and the largest landmark count
    _wl("d96_h8_m64_w64", 2, 1, 2, 8, 64, 64, 4, T=300, steps=20, seed=62, std=2.0),
    # a window below the fold period: the far-insert logits are taken per step
    _wl("d96_h4_m16_w7", 2, 1, 3, 4, 16, 7, 2, T=120, steps=20, seed=63),
    # three heads (run as four) just above the fold period, no sinks
    _wl("d96_h3_m24_w9", 2, 1, 2, 3, 24, 9, 0, T=90, steps=3 * P.FOLD_PERIOD + 5, seed=64, std=2.0),
    # one head, a one-key window
    _wl("d96_h1_m8_w1", 2, 1, 1, 1, 8, 1, 1, T=40, steps=20, seed=65),
    # six heads (run as eight), m not a multiple of 16
    _wl("d96_h6_m40_w100", 1, 2, 2, 6, 40, 100, 3, T=200, steps=16, seed=66),
]


@pytest.mark.parametrize("wl", SHAPES, ids=[w.name for w in SHAPES])
def test_prefill_d96(wl):
    prefill_parity(wl)


@pytest.mark.parametrize("wl", SHAPES, ids=[w.name for w in SHAPES])
def test_decode_d96(wl):
    decode_parity(wl)


def test_decode_d96_fm_rectifier():
    decode_parity(_wl("d96_h2_fm", 2, 1, 2, 2, 16, 32, 2, T=120, steps=20, seed=67, std=2.0),
                  rect=O.RECT_FM)


def test_d96_large_grid():
    # 1024 groups: 256-thread decode work-groups
    wl = _wl("d96_grid", 128, 1, 8, 2, 32, 64, 4, T=160, steps=12, seed=68)
    assert wl.groups >= 1024
    prefill_parity(wl, sample=W.groups_of_sequences(wl, W.sample_sequences(wl)))
    decode_parity(wl, sample=W.sample_groups(wl))
