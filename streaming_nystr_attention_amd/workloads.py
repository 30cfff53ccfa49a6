"""Seeded synthetic workloads for streaming Nystrom attention.

Shapes follow the model the nystrom.rs source page measures with (Qwen3-0.6B:
28 layers, 16 query heads over 8 KV heads, head width 128; m = 32, w = 128,
sink = 4, 256-token prefill).  No model weights or corpus are used: queries,
keys and values are i.i.d. Gaussian draws with the stated scales.  This module
draws random numbers and nothing else; it holds none of the method's
arithmetic, so the HIP path and the CPU oracle can both consume its output.

Each workload's inputs are drawn with torch generators seeded from
(workload seed, stream tag, step), so any step can be regenerated on its own.
Values are drawn on the requested device; callers that feed the oracle copy the
device values to the host rather than re-drawing them.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import torch

from . import Config


@dataclass(frozen=True)
class Workload:
    name: str
    n_seq: int
    n_layer: int
    n_kv: int
    hpk: int
    d: int
    dv: int
    m: int
    w: int
    sink: int
    T: int              # prompt (prefill) length
    steps: int          # decode steps after the prefill
    q_std: float = 1.0
    k_std: float = 1.0
    v_std: float = 1.0
    layer_scale: tuple | None = None  # (lo, hi): per-layer U[lo, hi] factor on q and k
    drift: float = 0.0  # key at absolute position p gets + drift * p on every component
    seed: int = 0

    @property
    def groups(self) -> int:
        return self.n_seq * self.n_layer * self.n_kv

    @property
    def config(self) -> Config:
        return Config(self.n_seq, self.n_layer, self.n_kv, self.hpk, self.d, self.dv, self.m,
                      self.w, self.sink)

    @property
    def m_eff(self) -> int:
        return max(4, min(self.T // 8, self.m))

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def _stress(m: int, sink: int) -> Workload:
    return Workload(f"stress_m{m}_s{sink}", n_seq=256, n_layer=1, n_kv=8, hpk=2, d=128, dv=128, m=m,
                    w=128, sink=sink, T=256, steps=8192, q_std=3.0, k_std=3.0, drift=0.01, seed=3)


WORKLOADS = {
    # one query head, d = 64: small enough for the oracle to finish in well under a second
    "single_head": Workload("single_head", 1, 1, 1, 1, 64, 64, 8, 16, 2, T=64, steps=64, seed=0),
    # one Qwen3-0.6B-shaped layer, batch 1
    "qwen3_layer": Workload("qwen3_layer", 1, 1, 8, 2, 128, 128, 32, 128, 4, T=256, steps=512,
                            q_std=2.0, k_std=2.0, seed=1),
    # the full 28-layer stack of that layer shape, 64 sequences
    "qwen3_stack_b64": Workload("qwen3_stack_b64", 64, 28, 8, 2, 128, 128, 32, 128, 4, T=256,
                                steps=1024, layer_scale=(1.0, 3.0), seed=2),
    # eviction / numerics stress: logits beyond the f32 exp range, drifting keys
    **{f"stress_m{m}_s{s}": _stress(m, s) for m in (8, 16, 32) for s in (0, 4)},
    # wide GQA: 64 query heads over 8 KV heads, long prompt
    "wide_gqa": Workload("wide_gqa", 32, 1, 8, 8, 128, 128, 64, 256, 4, T=4096, steps=2048,
                         seed=4),
    # eight query heads per KV head (64 query heads over 8 KV heads, the layer
    # shape of many large GQA models) at the stack's window and prompt: 16
    # sequences x 32 layers x 8 KV groups
    "gqa_h8_b16": Workload("gqa_h8_b16", 16, 32, 8, 8, 128, 128, 32, 128, 4, T=256, steps=256,
                           q_std=2.0, k_std=2.0, seed=5),
}

_TAG_PROMPT_Q, _TAG_PROMPT_K, _TAG_PROMPT_V, _TAG_STEP = 1, 2, 3, 4


def _gen(device, *key: int) -> torch.Generator:
    seed = 0x9E3779B1
    for k in key:
        seed = (seed * 1000003 + int(k) + 0x632BE5AB) % (1 << 62)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def layer_scales(wl: Workload) -> torch.Tensor:
    """Per-layer factor on q and k (CPU, f32), 1.0 when the workload has none."""
    if wl.layer_scale is None:
        return torch.ones(wl.n_layer, dtype=torch.float32)
    lo, hi = wl.layer_scale
    u = torch.rand(wl.n_layer, generator=_gen("cpu", wl.seed, 99), dtype=torch.float64)
    return (lo + (hi - lo) * u).to(torch.float32)


def _group_scale(wl: Workload, device) -> torch.Tensor:
    """[G] factor of each group's q and k (group g sits in layer (g // n_kv) % n_layer)."""
    s = layer_scales(wl).to(device)
    layer_of_group = (torch.arange(wl.groups, device=device) // wl.n_kv) % wl.n_layer
    return s[layer_of_group]


def prompt(wl: Workload, device, groups: slice | None = None):
    """Prompt tensors q [G][hpk][T][d], k [G][T][d], v [G][T][dv] (f32, on `device`).

    Drawn for all groups; `groups` returns a slice of them (same values)."""
    G, H, T = wl.groups, wl.hpk, wl.T
    f32 = torch.float32
    q = torch.randn(G, H, T, wl.d, generator=_gen(device, wl.seed, _TAG_PROMPT_Q), device=device,
                    dtype=f32)
    k = torch.randn(G, T, wl.d, generator=_gen(device, wl.seed, _TAG_PROMPT_K), device=device,
                    dtype=f32)
    v = torch.randn(G, T, wl.dv, generator=_gen(device, wl.seed, _TAG_PROMPT_V), device=device,
                    dtype=f32)
    gs = _group_scale(wl, device)
    q.mul_((wl.q_std * gs).view(G, 1, 1, 1))
    k.mul_((wl.k_std * gs).view(G, 1, 1))
    if wl.v_std != 1.0:
        v.mul_(wl.v_std)
    if wl.drift:
        k.add_((wl.drift * torch.arange(T, device=device, dtype=f32)).view(1, T, 1))
    if groups is not None:
        q, k, v = q[groups], k[groups], v[groups]
    return q.contiguous(), k.contiguous(), v.contiguous()


def decode_inputs(wl: Workload, step: int, device, out=None):
    """Inputs of decode step `step` (absolute position T + step):
    q [G][hpk][d], k [G][d], v [G][dv].  With `out=(q, k, v)` fills those."""
    G, H = wl.groups, wl.hpk
    gen = _gen(device, wl.seed, _TAG_STEP, step)
    f32 = torch.float32
    if out is None:
        q = torch.empty(G, H, wl.d, device=device, dtype=f32)
        k = torch.empty(G, wl.d, device=device, dtype=f32)
        v = torch.empty(G, wl.dv, device=device, dtype=f32)
    else:
        q, k, v = out
    q.normal_(generator=gen)
    k.normal_(generator=gen)
    v.normal_(generator=gen)
    gs = _group_scale(wl, device)
    q.mul_((wl.q_std * gs).view(G, 1, 1))
    k.mul_((wl.k_std * gs).view(G, 1))
    if wl.v_std != 1.0:
        v.mul_(wl.v_std)
    if wl.drift:
        k.add_(wl.drift * (wl.T + step))
    return q, k, v


def sample_groups(wl: Workload, extra: int = 4) -> list[int]:
    """Groups whose outputs the oracle recomputes at full size: sequences
    {0, 1, B/2, B-1} x layers {0, L/2, L-1} x KV heads {0, K-1}, plus `extra`
    seeded groups."""
    B, L, K = wl.n_seq, wl.n_layer, wl.n_kv
    seqs = sorted({0, min(1, B - 1), B // 2, B - 1})
    picks = []
    for s in seqs:
        for layer in sorted({0, L // 2, L - 1}):
            for kv in sorted({0, K - 1}):
                picks.append((s * L + layer) * K + kv)
    g = torch.Generator().manual_seed(wl.seed * 7919 + 17)
    picks += torch.randint(0, wl.groups, (extra,), generator=g).tolist()
    return sorted(set(picks))


def sample_sequences(wl: Workload, extra: int = 4) -> list[int]:
    """Sequences {0, 1, B/2, B-1} plus `extra` further seeded sequences (fewer when
    the batch has no more)."""
    B = wl.n_seq
    seqs = {0, min(1, B - 1), B // 2, B - 1}
    want = min(B, len(seqs) + extra)
    g = torch.Generator().manual_seed(wl.seed * 7919 + 29)
    for s in torch.randperm(B, generator=g).tolist():
        if len(seqs) >= want:
            break
        seqs.add(s)
    return sorted(seqs)


def groups_of_sequences(wl: Workload, seqs) -> list[int]:
    """Every group (all layers and KV heads) of the given sequences, in group order."""
    per = wl.n_layer * wl.n_kv
    return [s * per + i for s in sorted(seqs) for i in range(per)]
