"""GPU parity of the exact grouped-GQA comparator (o1_exact_attend) against the
oracle's brute-force exact attention (f64), which is pinned to scipy."""
import numpy as np
import pytest
import torch

import oracle as O
import streaming_nystr_attention_amd as P

from parity_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    P.lib()
    yield


@pytest.mark.parametrize("G,H,d,cap,n,first,std", [
    (3, 2, 128, 1000, 1000, 0, 2.0),      # few groups: split key range + combine
    (2, 8, 64, 400, 300, 100, 1.0),       # sliding-window start, ragged tail
    (2048, 2, 128, 200, 200, 0, 3.0),     # many groups: one work-group per group
    (5, 4, 128, 64, 1, 0, 1.0),           # a single key
    (7, 1, 64, 3000, 2999, 1234, 2.0),    # long range, odd counts
    (6, 3, 128, 900, 900, 0, 2.0),        # 3 heads (run as 4): split key range
    (1500, 6, 64, 150, 150, 10, 1.0),     # 6 heads (run as 8), many groups
    (2, 7, 128, 300, 257, 3, 1.0),        # 7 heads
    (4, 5, 64, 2000, 2000, 0, 2.0),       # 5 heads, split key range
    (3, 2, 96, 1000, 1000, 0, 2.0),       # d = 96: value rows of 24 float4, split key range
    (2048, 8, 96, 150, 150, 5, 1.0),      # d = 96, 8 heads, many groups
    (5, 3, 96, 300, 211, 7, 1.0),         # d = 96, 3 heads (run as 4), ragged tail
    (3, 2, 256, 700, 700, 0, 1.0),        # d = 256: a value row per wave, split key range
    (2048, 2, 256, 100, 100, 0, 1.0),     # d = 256, many groups
    (4, 8, 256, 300, 257, 3, 1.0),        # d = 256, 8 heads
    (3, 12, 128, 1000, 1000, 0, 2.0),     # 12 heads: blocks of 8 and 4, split key range
    (1500, 16, 64, 150, 150, 10, 1.0),    # 16 heads, many groups
    (2, 9, 96, 300, 257, 3, 1.0),         # 9 heads: blocks of 8 and 1
    (3, 32, 128, 700, 700, 0, 2.0),       # 32 heads: four blocks, split key range
    (1200, 64, 64, 150, 150, 10, 1.0),    # 64 heads: eight blocks, many groups
])
def test_exact_attend_matches_oracle(G, H, d, cap, n, first, std):
    say(f"[exact] G={G} hpk={H} d={d} cap={cap} n_keys={n} first={first}")
    g = torch.Generator(device=DEV).manual_seed(G * 7 + n)
    q = (std * torch.randn(G, H, d, device=DEV, generator=g)).contiguous()
    k = (std * torch.randn(G, cap, d, device=DEV, generator=g)).contiguous()
    v = torch.randn(G, cap, d, device=DEV, generator=g).contiguous()
    out = torch.empty(G, H, d, device=DEV)
    P.o1_exact_attend(q, k, v, out, n, first)
    torch.cuda.synchronize()
    qh, kh, vh, oh = q.cpu().numpy(), k.cpu().numpy(), v.cpu().numpy(), out.cpu().numpy()
    scale = O.f32_scale(d)
    check = range(G) if G <= 16 else [0, 1, G // 2, G - 1]
    worst = 0.0
    for gi in check:
        for h in range(H):
            ref = O.exact_attention(qh[gi, h], kh[gi, first:n], vh[gi, first:n], scale)
            worst = max(worst, np.abs(oh[gi, h] - ref).max() / np.linalg.norm(ref))
    say(f"  max row error {worst:.3e}")
    assert worst <= 1e-6
