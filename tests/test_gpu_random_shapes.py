"""GPU parity at seeded random shapes: each case draws the query heads per group,
the head width, the landmark budget, window, sinks, prompt length, rectifier,
input scale and group counts within the compiled limits (d = dv in {64, 80, 96, 128, 256},
or d = 192 with dv = 128,
hpk <= 64, m <= 64, sink + w <= 1024 with hpk' * (sink + w) * 8 <= 32 KB for hpk'
min(hpk, 8) rounded up to a power of two),
then checks the prefill freeze and the decode steps against the oracle exactly
as the fixed-shape tests do."""
import numpy as np
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


def draw(case: int, widths=(64, 128), base=7000, max_m=64, min_hpk=1, max_hpk=8):
    r = np.random.default_rng(base + case)
    while True:
        # the first ten cases draw power-of-two head counts, the rest any count
        hpk = int(r.choice([1, 2, 4, 8])) if case < 10 else int(r.integers(min_hpk, max_hpk + 1))
        hc = 1 << (min(hpk, 8) - 1).bit_length()  # the compiled head count of its largest block
        d = int(r.choice(list(widths)))
        m = int(r.integers(4, max_m + 1))
        sink = int(r.integers(0, 17))
        w = int(r.integers(1, 300))
        if hc * (sink + w) * 8 > 32 * 1024 or sink + w > 1024:
            continue
        T = int(r.integers(w + sink + 9, w + sink + 400))  # skeleton mode: T > w + sink + 8
        n_seq, n_layer, n_kv = (int(x) for x in r.integers(1, 4, size=3))
        std = float(r.choice([1.0, 2.0, 3.0]))
        rect = int(r.integers(0, 2))
        steps = int(r.integers(5, 40))
        name = f"rand{case}" if base == 7000 else (f"rand{case}_h" if base == 7300 else
                                                   f"rand{case}_d{d}" + ("m" if base == 7400 else ""))
        dv = 128 if d == 192 else d  # keys of 192 floats come with values of 128
        wl = W.Workload(name, n_seq, n_layer, n_kv, hpk, d, dv, m, w, sink, T=T, steps=steps,
                        q_std=std, k_std=std, seed=900 + case)
        return wl, (O.RECT_AGGREGATE, O.RECT_FM)[rect]


CASES = [draw(i) for i in range(16)]
# d = 96 (value rows of 24 float4) drawn from their own seeds, so the cases
# above keep theirs
CASES += [draw(i, widths=(96,), base=7100) for i in range(6)]
# d = 256 (a value row per wave; m <= 32)
CASES += [draw(i, widths=(256,), base=7200, max_m=32) for i in range(4)]
# d = 256 with m up to 64 (the landmark pass in two component chunks above 32)
CASES += [draw(i, widths=(256,), base=7400) for i in range(3)]
# 9 to 16 heads per group (stepped in blocks of at most 8), d 64 to 128
CASES += [draw(10 + i, widths=(64, 96, 128), base=7300, min_hpk=9, max_hpk=16) for i in range(4)]
# keys of 192 floats with values of 128, 1 to 16 heads
CASES += [draw(10 + i, widths=(192,), base=7500, max_hpk=16) for i in range(4)]
# 17 to 64 heads per group (three to eight blocks)
CASES += [draw(10 + i, widths=(64, 128), base=7600, min_hpk=17, max_hpk=64) for i in range(2)]
# d = 80 (blocks of at most 4 heads), 1 to 12 heads
CASES += [draw(10 + i, widths=(80,), base=7700, max_hpk=12) for i in range(3)]


@pytest.mark.parametrize("wl,rect", CASES,
                         ids=[f"{w.name}-h{w.hpk}-d{w.d}-m{w.m}-w{w.w}-s{w.sink}-T{w.T}-r{r}"
                              for w, r in CASES])
def test_random_shape_prefill_and_decode(wl, rect):
    prefill_parity(wl)
    decode_parity(wl, rect=rect)
