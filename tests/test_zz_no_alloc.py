"""GPU test of o1_exact_attend_noalloc, the exact comparator without a work
space (its split partials live in the library's static per-device buffer):
through the C ABI, its outputs equal those of o1_exact_attend with a caller
work space bit for bit, on two calls in a row, the second with a smaller
input, and on a launch that needs no partials at all."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
import streaming_nystr_attention_amd as P

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    P.lib()
    yield


def _inputs(G, hpk, d, cap, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    q = torch.randn(G, hpk, d, generator=g, device=DEV) * 2.0
    k = torch.randn(G, cap, d, generator=g, device=DEV) * 2.0
    v = torch.randn(G, cap, d, generator=g, device=DEV)
    return q, k, v


def _both(G, hpk, d, cap, n_keys, first, seed):
    L = P.lib()
    q, k, v = _inputs(G, hpk, d, cap, seed)
    desc = P.o1_exact_desc(G, hpk, d, d, cap, first, n_keys, 0.0)
    need = ctypes.c_size_t()
    assert L.o1_exact_workspace_bytes(ctypes.byref(desc), ctypes.byref(need)) == 0
    ws = torch.empty(max(1, need.value), dtype=torch.uint8, device=DEV)
    ref = torch.full((G, hpk, d), float("nan"), device=DEV)
    got = torch.full((G, hpk, d), float("nan"), device=DEV)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = L.o1_exact_attend(ctypes.byref(desc), ptr(q), ptr(k), ptr(v), ptr(ref), ptr(ws),
                           need.value, stream)
    assert rc == 0, P.o1_last_error()
    rc = L.o1_exact_attend_noalloc(ctypes.byref(desc), ptr(q), ptr(k), ptr(v), ptr(got), stream)
    assert rc == 0, P.o1_last_error()
    torch.cuda.synchronize()
    return q, k, v, ref, got, need.value


def test_noalloc_equals_workspace_entry_point_on_two_calls():
    cases = [  # (G, hpk, d, cap, n_keys, first): splits > 1 in both, the second smaller
        (64, 8, 128, 3000, 3000, 0),
        (12, 2, 64, 900, 700, 5),
    ]
    used = []
    for i, (G, hpk, d, cap, n_keys, first) in enumerate(cases):
        print(f"[noalloc] call {i}: G={G} hpk={hpk} d={d} keys={first}..{n_keys - 1}", flush=True)
        q, k, v, ref, got, need = _both(G, hpk, d, cap, n_keys, first, seed=70 + i)
        assert need > 0, "the case must use the static buffer"
        used.append(need)
        assert torch.isfinite(ref).all()
        assert torch.equal(ref, got), (ref - got).abs().max().item()
        # and both are exact attention (oracle, brute force) on a few groups
        scale = O.f32_scale(d)
        qh, kh, vh, gh = (t.cpu().numpy() for t in (q, k, v, got))
        worst = 0.0
        for g in (0, G // 2, G - 1):
            for h in range(hpk):
                o = O.exact_attention(qh[g, h], kh[g, first:n_keys], vh[g, first:n_keys], scale)
                worst = max(worst, np.abs(gh[g, h] - o).max() / np.linalg.norm(o))
        print(f"[noalloc] call {i}: {need} bytes of partials, bit-equal; oracle row error {worst:.2e}",
              flush=True)
        assert worst <= 1e-5
    assert used[1] < used[0]


def test_noalloc_without_partials():
    # enough groups that the keys are not split: no work space at all
    q, k, v, ref, got, need = _both(1100, 2, 128, 300, 300, 0, seed=80)
    assert need == 0
    assert torch.equal(ref, got)
