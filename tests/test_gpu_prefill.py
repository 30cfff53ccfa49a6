"""GPU parity of the prefill freeze (o1_prefill computing everything itself)
against the CPU oracle on the same prompts.

  K~, Q~         equal to the oracle's f32 values (both sum the segment in row
                 order in f64 and round once); at most 1 ulp is allowed.
  M              judged by the residual ||A M A - A||_F / ||A||_F <= 1e-3 with the
                 oracle's f64 A, not elementwise (A is ill-conditioned).
  lambda, tries  lambda within 1e-12 relative, attempt number equal.
  far field      T^ e^{m_max} and Z^ e^{m_max} against the oracle's (which uses
                 the oracle's own landmarks): T^ within 1e-5 of each landmark
                 row's norm, Z^ within 1e-6 relative (f32 weights, as the page's
                 far_insert takes them).
  ring, sinks,   bit-exact; counters bit-exact for every group.
"""
import pytest
import torch

import streaming_nystr_attention_amd as P
from streaming_nystr_attention_amd import workloads as W

from parity_util import prefill_parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    P.lib()
    yield


def test_prefill_single_head():
    prefill_parity(W.WORKLOADS["single_head"])


def test_prefill_qwen3_layer():
    prefill_parity(W.WORKLOADS["qwen3_layer"])


def seq_sample(wl):
    """Every group of sequences {0, 1, B/2, B-1} and 4 seeded ones."""
    return W.groups_of_sequences(wl, W.sample_sequences(wl))


@pytest.mark.parametrize("name", ["stress_m8_s0", "stress_m8_s4", "stress_m16_s0", "stress_m16_s4", "stress_m32_s0", "stress_m32_s4"])
def test_prefill_stress(name):
    wl = W.WORKLOADS[name]
    prefill_parity(wl, sample=seq_sample(wl))


def test_prefill_wide_gqa():
    # every group
    prefill_parity(W.WORKLOADS["wide_gqa"])


def test_prefill_qwen3_stack_full_size():
    wl = W.WORKLOADS["qwen3_stack_b64"]
    prefill_parity(wl, sample=seq_sample(wl))


def test_prefill_ragged_segments():
    prefill_parity(W.Workload("ragged", 3, 1, 2, 2, 128, 128, 32, 16, 2, T=100, steps=0, seed=11))


def test_prefill_prompt_longer_than_budget():
    # T / 8 above the budget: m_eff clamps to m (the warn-once case of the page)
    prefill_parity(W.Workload("clamped", 2, 1, 2, 2, 64, 64, 16, 32, 4, T=300, steps=0, seed=21))


@pytest.mark.parametrize("wl", [
    W.Workload("max_window_hpk4", 2, 1, 2, 4, 128, 128, 64, 1000, 24, T=1100, steps=0, q_std=2.0,
               k_std=2.0, seed=16),
    W.Workload("max_heads_d64", 2, 1, 2, 8, 64, 64, 64, 500, 12, T=700, steps=0, seed=17),
], ids=["max_window_hpk4", "max_heads_d64"])
def test_prefill_maximum_sizes(wl):
    """The largest compiled near block (sink + w = 1024) and head count (hpk 8),
    both with m = 64."""
    prefill_parity(wl)
