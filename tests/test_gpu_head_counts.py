"""GPU parity at query-head counts that are not powers of two (3, 5, 6, 7, as
GQA models use them, e.g. 24 query heads over 8 KV heads).  Such a group runs
the kernels compiled for the next power of two with the extra heads as
placeholders: zero queries, no state, no outputs.  Each case checks the prefill
freeze and every decode step against the oracle exactly as the fixed-shape
tests do, on each launch path: 512-thread work-groups with the row pass as one
stream (hpk * d >= 512 after rounding) or not, 256-thread work-groups on grids
of at least 1024 groups, and a window shorter than the fold period (no per-slot
far-insert logits)."""
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


def _wl(name, n_seq, n_kv, hpk, d, m, w, sink, T, steps, std, seed):
    return W.Workload(name, n_seq, 1, n_kv, hpk, d, d, m, w, sink, T=T, steps=steps, q_std=std,
                      k_std=std, seed=seed)


CASES = [
    (_wl("h3_d128_stream_rows", 3, 4, 3, 128, 32, 128, 4, 256, 40, 2.0, 61), O.RECT_AGGREGATE),
    (_wl("h5_d64_fm", 2, 3, 5, 64, 32, 64, 0, 200, 30, 1.0, 62), O.RECT_FM),
    (_wl("h6_d128_m64", 2, 4, 6, 128, 64, 256, 4, 600, 24, 1.0, 63), O.RECT_AGGREGATE),
    (_wl("h7_d128", 2, 2, 7, 128, 32, 100, 3, 300, 40, 2.0, 64), O.RECT_AGGREGATE),
    (_wl("h3_d64_short_window", 2, 3, 3, 64, 8, 4, 2, 60, 20, 1.0, 65), O.RECT_AGGREGATE),
    (_wl("h6_d64_rows", 3, 2, 6, 64, 16, 40, 2, 120, 30, 3.0, 66), O.RECT_AGGREGATE),
]


@pytest.mark.parametrize("wl,rect", CASES, ids=[c[0].name for c in CASES])
def test_head_count_prefill_and_decode(wl, rect):
    prefill_parity(wl)
    decode_parity(wl, rect=rect)


def test_head_count_3_large_grid_sampled():
    """1120 groups of 3 heads: 256-thread work-groups (the compiled 4 heads x 16
    landmarks fit four per CU); a declared sample of sequences is compared."""
    wl = _wl("h3_grid1120", 70, 16, 3, 64, 16, 24, 2, 100, 20, 2.0, 67)
    sample = W.groups_of_sequences(wl, W.sample_sequences(wl))
    prefill_parity(wl, sample=sample)
    decode_parity(wl, sample=sample)


@pytest.mark.parametrize("hpk,seed", [(5, 68), (7, 69)], ids=["h5", "h7"])
def test_head_count_large_grid_eight_head_kernel(hpk, seed):
    """1024 groups of 5 or 7 heads at d = 128: 256-thread work-groups of the
    8-head kernel, whose per-head phase runs two heads per wave, one per
    half-wave.  With 7 heads the last wave's second half is a placeholder; with
    5 one wave holds a head and a placeholder and another only placeholders.  A
    declared sample of sequences is compared."""
    wl = _wl(f"h{hpk}_grid1024", 64, 16, hpk, 128, 32, 64, 4, 300, 20, 2.0, seed)
    sample = W.groups_of_sequences(wl, W.sample_sequences(wl))
    prefill_parity(wl, sample=sample)
    decode_parity(wl, sample=sample)
