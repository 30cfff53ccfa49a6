#!/usr/bin/env python3
"""Throughput of batched streaming Nystrom attention on one MI355X.

One bench step is one whole job over the workload: the prefill freeze of every
group (o1_prefill) followed by the workload's decode steps (one o1_step launch
each, every group of every sequence and layer per launch).  All inputs are
generated into HBM before the timed region; each job re-prefills, so every
timed job does identical work.

value       decode group-steps per second over the whole timed job (prefill
            time included); tokens_per_s = sequences x decode steps / time.
roofline    the decode kernel against the MI355X HBM peak of 8 TB/s, from its
            average launch time (HIP events on the launch stream):
              achieved / frac       algorithmic bytes of the per-eviction step
                                    (every state value read once, its modified
                                    part written once, q/k/v in, outputs out)
              kernel_*              the bytes this kernel's algorithm must move
                                    (T^ written and q~ read once per fold period),
                                    averaged over the period
              traffic / dram_*      HBM bytes the counters measured per launch
prefill     the prefill freeze: prompt read once and state written once against
            the HBM peak, and the far field's f64 matrix-core flops over the
            whole prefill time against the f64 MFMA peak (a lower bound of that
            kernel's rate).
workloads   decode launches of other workloads (eviction stress, wide GQA) with
            the same roofline figures.
cpu_baseline  the CPU oracle (tests' reference implementation, untuned) on a
            bounded sample of the same workload, on every CPU this process may
            use.
exact_comparator  exact grouped-GQA attention (o1_exact_attend) over the job's
            final context at the same shape: the O(context) decode replaced.
exact_only_mode  o1_step in the exact-only mode (prompt of w + sink + 8 tokens,
            every key kept exactly) at the same group count and shape.
per_layer_mode  the same state sealed layer by layer from model-layout buffers
            and stepped with one o1_step_layer launch per layer and token,
            eager and from a captured HIP graph.

Default workload: qwen3_stack_b64 (64 sequences x 28 layers x 8 KV heads, 2 query
heads per KV head, d = dv = 128, m = 32, w = 128, sink = 4, 256-token prefill,
1024 decode steps).
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Nyström decode group-steps/sec & tokens/s at 1 GPU; achieved HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0
F64_MFMA_PEAK_TFLOPS = 78.6
DECODE_SRC = [os.path.join(ROOT, "streaming_nystr_attention_amd", "csrc", f)
              for f in ("o1_decode.hip", "o1_internal.h")] + [os.path.join(ROOT, "include", "o1.h")]
# HBM bytes per decode launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE (scaled by
# a 1 GiB copy in the same process), keyed by (workload, sha256 prefix of the decode
# kernel's sources).
# A changed kernel (comments aside) has no entry, and the roofline's traffic is then null.
MEASURED_TRAFFIC = {
    ("qwen3_stack_b64", "4980a7cb59cd0132"): 3051928802,
    ("stress_m32_s4", "4980a7cb59cd0132"): 436433102,
    ("stress_m8_s0", "4980a7cb59cd0132"): 318891388,
    ("wide_gqa", "4980a7cb59cd0132"): 208450051,
    ("gqa_h8_b16", "4980a7cb59cd0132"): 1567424054,
}


def decode_source_sha() -> str:
    """Hash of the decode kernel's sources with comments and whitespace removed,
    so the key changes with the code, not with its comments."""
    import hashlib
    import re

    h = hashlib.sha256()
    for path in DECODE_SRC:
        with open(path, encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def step_bytes_per_group_step(wl) -> int:
    """Algorithmic bytes of one group-step of the per-eviction step
    (NystromState::step_group of the nystrom.rs source page), f32 throughout:
    read the near rows, K~, and per head Q~, M, T^, Z^ and the running max, plus
    the inputs q, k, v; write the new ring row, per head T^, Z^ and the running
    max, and the outputs."""
    S, w, d, dv, m, H = wl.sink, wl.w, wl.d, wl.dv, wl.m_eff, wl.hpk
    read = (S + w) * (d + dv) + m * d + H * (m * d + m * m + m * dv + 2 * m) + H * d + d + dv
    write = (d + dv) + H * (m * dv + 2 * m) + H * dv
    return 4 * (read + write)


def prefill_bytes_and_flops(wl) -> tuple[int, int]:
    """Algorithmic work of the prefill freeze per launch over every group: the
    prompt (each head's queries, keys, values) read once and the frozen state
    written once (near rows, K~, per head Q~, M, T^, Z^, running max), f32; and
    the far field's matrix products, 2 m T_far (d + dv) flops per head
    (logits Q~ K_far^T, then weights times V) over the T - sink - w far keys."""
    S, w, d, dv, m, H, T = wl.sink, wl.w, wl.d, wl.dv, wl.m_eff, wl.hpk, wl.T
    read = H * T * d + T * d + T * dv
    write = (S + w) * (d + dv) + m * d + H * (m * d + m * m + m * dv + 2 * m)
    flops = H * 2 * m * (T - S - w) * (d + dv)
    return 4 * (read + write) * wl.groups, flops * wl.groups


def host_cpu_share() -> tuple[int, str]:
    """CPUs this process may run on: its affinity set, capped by a cgroup CPU
    quota when one is set; with how that was found."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    how = f"affinity {n} of {os.cpu_count()} host CPUs"
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            quota, period = f.read().split()[:2]
        if quota != "max":
            q = max(1, int(float(quota) / float(period)))
            if q < n:
                n = q
                how += f", cgroup quota {quota}/{period}"
    except (OSError, ValueError):
        pass
    return n, how


def decode_bytes_per_group_step(wl) -> tuple[float, float]:
    """Algorithmic HBM bytes of one group-step, averaged over a fold period:
    each stored value read once, each modified value written once (f32 state,
    Z^ and held logits f64, far_len i64).

    T^ is read every step and written on the fold step only (once per
    FOLD_PERIOD = K steps).  A step with P evictions held (P = 0 .. K-1, each
    equally often) reads their value rows and logits; a step that does not fold
    writes its own eviction's row and logits into the held set.  With w >= K
    the far-insert logits are kept per ring slot: the query landmarks are read
    on the fold step only, when the logits of the K keys that arrived since the
    previous fold are written, and every step reads its evicted key's logits."""
    from streaming_nystr_attention_amd import FOLD_PERIOD as K

    S, w, d, dv, m, H = wl.sink, wl.w, wl.d, wl.dv, wl.m_eff, wl.hpk
    held = dv * 4 + H * m * 8                # one held eviction: value row, logits per head
    ring = w >= K                            # far-insert logits kept per ring slot
    q_tilde = H * m * d * 4                  # every head's query landmarks
    read = ((S + w) * (d + dv) * 4           # sinks + ring rows
            + m * d * 4                      # key landmarks
            + (q_tilde / K + H * m * 8 if ring else q_tilde)
            + H * (m * m * 4                 # per head: M
                   + m * dv * 4 + m * 8      # T^, Z^ (f64)
                   + m * 4 + m * 4)          # running max, its value at the last fold
            + (K - 1) / 2 * held             # the held evictions
            + (H * d + d + dv) * 4           # inputs q, k, v
            + 4 + H * 8)                     # win_head, far_len
    write = ((d + dv) * 4                    # the new ring row
             + H * (m * 8 + m * 4)           # Z^, running max
             + H * (m * dv * 4 + m * 4) / K  # T^ and its max, on the fold step
             + (K - 1) / K * held            # this eviction joins the held set
             + (H * m * 8 if ring else 0)    # logits of the arrivals, on the fold step
             + H * dv * 4                    # outputs
             + 4 + H * 8)
    return read, write


def cpu_baseline(wl, q, k, v, Q, K, V, n_dec, threads, n, share):
    """Time the oracle on a bounded sample of n groups (whole jobs)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import torch

    import oracle as O

    g = torch.Generator().manual_seed(1234)
    idx = torch.randperm(wl.groups, generator=g)[:n].sort().values
    di = idx.to(q.device)
    qh, kh, vh = (t.index_select(0, di).cpu().numpy() for t in (q, k, v))
    Qh = Q.index_select(1, di).cpu().numpy()
    Kh = K.index_select(1, di).cpu().numpy()
    Vh = V.index_select(1, di).cpu().numpy()

    def one(i):
        grp = O.Group(wl.m, wl.w, wl.sink, wl.hpk)
        grp.prefill(qh[i], kh[i], vh[i])
        grp.step_many(np.ascontiguousarray(Qh[:, i]), np.ascontiguousarray(Kh[:, i]),
                      np.ascontiguousarray(Vh[:, i]))
        return 0

    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(one, range(n)))
    dt = time.perf_counter() - t0
    return {
        "value": n * n_dec / dt,
        "unit": "group-steps/s",
        "cores": threads,
        "host_cpus": os.cpu_count(),
        "cpu_share": share,
        "kind": "oracle",
        "sample": (f"{n} of the {wl.groups} groups of {wl.name} (seeded pick), each a whole job: "
                   f"prefill of {wl.T} tokens + {n_dec} decode steps; f64 C oracle, "
                   f"{threads} threads (one per CPU this process may use), {dt:.1f} s wall"),
    }


def decode_roofline(wl, us_per_launch, traffic=None) -> dict:
    """Roofline figures of one decode launch over every group of `wl`."""
    G = wl.groups
    alg = step_bytes_per_group_step(wl) * G
    rd, wr = decode_bytes_per_group_step(wl)
    kern = (rd + wr) * G
    t = us_per_launch * 1e-6
    res = {"bound": "hbm", "achieved": alg / t / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": alg / t / 1e9 / HBM_PEAK_GBS, "traffic": traffic,
           "traffic_unit": "bytes per launch", "bytes_per_launch": alg,
           "bytes_per_group_step": alg / G,
           "kernel_bytes_per_group_step": kern / G,
           "kernel_GBps": kern / t / 1e9, "kernel_frac": kern / t / 1e9 / HBM_PEAK_GBS,
           "basis": "achieved/frac: the per-eviction step's algorithmic bytes (every state value read once, "
                    "its modified part written once, each step); this kernel moves fewer (T^ written and "
                    "q~ read once per fold period), so frac can pass 1 where those dominate; kernel_*: this "
                    "kernel's own algorithmic bytes; dram_*: HBM bytes from the rocprofv3 counters"}
    if traffic:
        res["dram_GBps"] = traffic / t / 1e9
        res["dram_frac"] = traffic / t / 1e9 / HBM_PEAK_GBS
    return res


def other_workload(name, n_steps, dev):
    """Prefill, then n_steps decode launches of workload `name`, timed with HIP
    events on the launch stream (inputs generated beforehand)."""
    import torch

    import streaming_nystr_attention_amd as P
    from streaming_nystr_attention_amd import workloads as W

    wl = W.WORKLOADS[name]
    G, H = wl.groups, wl.hpk
    try:
        q, k, v = W.prompt(wl, dev)
        Q = torch.empty(n_steps, G, H, wl.d, device=dev)
        K = torch.empty(n_steps, G, wl.d, device=dev)
        V = torch.empty(n_steps, G, wl.dv, device=dev)
        for t in range(n_steps):
            W.decode_inputs(wl, t, dev, out=(Q[t], K[t], V[t]))
        out = torch.empty(G, H, wl.dv, device=dev)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        with P.O1Groups(wl.config) as grp:
            for timed in (False, True):  # the first pass warms up, the second is timed
                e[0].record()
                grp.prefill(q, k, v)
                e[1].record()
                for t in range(n_steps):
                    grp.step(Q[t], K[t], V[t], out)
                e[2].record()
            torch.cuda.synchronize()
        us = e[1].elapsed_time(e[2]) * 1e3 / n_steps
        pf_bytes, pf_flops = prefill_bytes_and_flops(wl)
        pf_ms = e[0].elapsed_time(e[1])
        del q, k, v, Q, K, V
        torch.cuda.empty_cache()
        return {"groups": G, "hpk": H, "m": wl.m_eff, "w": wl.w, "sink": wl.sink,
                "prompt_len": wl.T, "decode_steps_timed": n_steps, "us_per_launch": us,
                "group_steps_per_s": G / (us * 1e-6),
                "roofline": decode_roofline(wl, us, MEASURED_TRAFFIC.get((name, decode_source_sha()))),
                "prefill_ms": pf_ms, "prefill_frac_hbm": pf_bytes / (pf_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "prefill_far_tflops": pf_flops / (pf_ms * 1e-3) / 1e12}
    except Exception as exc:  # context, never the headline
        return {"error": str(exc)[:200]}


def exact_comparator(wl, ctx, nystrom_us, dev):
    """Exact grouped-GQA attention over `ctx` stored keys per group at the same
    shape (o1_exact_attend): the O(context) decode the O(1) operator replaces."""
    import torch

    import streaming_nystr_attention_amd as P

    G, H = wl.groups, wl.hpk
    try:
        g = torch.Generator(device=dev).manual_seed(77)
        kc = torch.randn(G, ctx, wl.d, device=dev, generator=g)
        vc = torch.randn(G, ctx, wl.dv, device=dev, generator=g)
        q = torch.randn(G, H, wl.d, device=dev, generator=g)
        out = torch.empty(G, H, wl.dv, device=dev)
        desc = P._exact_desc(q, kc, vc, ctx, 0, None)
        need = P.o1_exact_workspace_bytes(desc)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        for _ in range(2):
            P.o1_exact_attend(q, kc, vc, out, ctx, 0, workspace=ws)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record()
        for _ in range(reps):
            P.o1_exact_attend(q, kc, vc, out, ctx, 0, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        nbytes = G * ctx * (wl.d + wl.dv) * 4 + G * H * (wl.d + wl.dv) * 4
        del kc, vc
        torch.cuda.empty_cache()
        return {"context": ctx, "us_per_launch": us, "bytes_per_launch": nbytes,
                "achieved_GBps": nbytes / (us * 1e-6) / 1e9,
                "frac_of_peak": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                "nystrom_decode_us": nystrom_us, "exact_over_nystrom": us / nystrom_us}
    except Exception as exc:  # the comparator is context, never the headline
        return {"context": ctx, "error": str(exc)[:200]}


def exact_only_mode(wl, n_steps, dev):
    """Decode steps in the exact-only mode at the workload's group count and
    shape: an exact-only prefill of the longest such prompt (w + sink + 8
    tokens, q not read), then n_steps o1_step launches, each appending one key
    and attending exactly over all of them."""
    import dataclasses

    import torch

    import streaming_nystr_attention_amd as P
    from streaming_nystr_attention_amd import workloads as W

    T = wl.w + wl.sink + 8
    G, H = wl.groups, wl.hpk
    try:
        cfg = dataclasses.replace(wl.config, exact_cap=T + n_steps)
        _, k, v = W.prompt(wl.with_(T=T), dev)
        Q = torch.empty(n_steps, G, H, wl.d, device=dev)
        K = torch.empty(n_steps, G, wl.d, device=dev)
        V = torch.empty(n_steps, G, wl.dv, device=dev)
        for t in range(n_steps):
            W.decode_inputs(wl, t, dev, out=(Q[t], K[t], V[t]))
        out = torch.empty(G, H, wl.dv, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with P.O1Groups(cfg) as grp:
            for timed in (False, True):  # the first pass warms up, the second is timed
                grp.prefill(None, k, v)
                if timed:
                    e0.record()
                for t in range(n_steps):
                    grp.step(Q[t], K[t], V[t], out)
                if timed:
                    e1.record()
            torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / n_steps
        # step t reads T + t stored rows and the new one, stores the new row,
        # reads the queries and writes the outputs
        row = (wl.d + wl.dv) * 4
        rows_read = n_steps * (T + 1) + n_steps * (n_steps - 1) // 2
        nbytes = G * (rows_read * row + n_steps * row + n_steps * H * row) / n_steps
        del Q, K, V, k, v
        torch.cuda.empty_cache()
        return {"prompt_len": T, "decode_steps": n_steps, "exact_cap": T + n_steps,
                "us_per_launch": us, "bytes_per_launch": nbytes,
                "achieved_GBps": nbytes / (us * 1e-6) / 1e9,
                "frac_of_peak": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}
    except Exception as exc:  # context, never the headline
        return {"prompt_len": T, "error": str(exc)[:200]}


def per_layer_mode(wl, n_tokens, dev):
    """The workload driven one layer at a time, as a model runs it: every layer
    sealed from a position-major query trace and per-KV-head caches
    (o1_prefill_layer), then per token one o1_step_layer launch per layer
    (n_seq * n_kv groups each), eager and replayed from a captured HIP graph."""
    import torch

    import streaming_nystr_attention_amd as P
    from streaming_nystr_attention_amd import workloads as W

    B, L, K, H = wl.n_seq, wl.n_layer, wl.n_kv, wl.hpk
    T = wl.T
    try:
        grp = P.O1Groups(wl.config)
        q, k, v = W.prompt(wl, dev)
        layer_idx = [torch.tensor([(s * L + l) * K + kv for s in range(B) for kv in range(K)],
                                  device=dev) for l in range(L)]
        # model-side buffers of each layer, built outside the timed region
        bufs = []
        for l in range(L):
            ql = q.index_select(0, layer_idx[l]).view(B, K, H, T, wl.d)
            trace = ql.permute(0, 3, 1, 2, 4).reshape(B, T, K * H, wl.d).contiguous()
            kc = k.index_select(0, layer_idx[l]).view(B, K, T, wl.d).contiguous()
            vc = v.index_select(0, layer_idx[l]).view(B, K, T, wl.dv).contiguous()
            bufs.append((trace, kc, vc))
        del q, k, v
        Q = torch.empty(n_tokens, L, B, K * H, wl.d, device=dev)
        Kn = torch.empty(n_tokens, L, B, K, wl.d, device=dev)
        Vn = torch.empty(n_tokens, L, B, K, wl.dv, device=dev)
        for t in range(n_tokens):
            qa, ka, va = W.decode_inputs(wl, t, dev)
            for l in range(L):
                Q[t, l] = qa.index_select(0, layer_idx[l]).view(B, K * H, wl.d)
                Kn[t, l] = ka.index_select(0, layer_idx[l]).view(B, K, wl.d)
                Vn[t, l] = va.index_select(0, layer_idx[l]).view(B, K, wl.dv)
        out = torch.empty(L, B, K * H, wl.dv, device=dev)

        def seal():
            for l in range(L):
                trace, kc, vc = bufs[l]
                grp.prefill_layer(l, trace.permute(0, 2, 1, 3), kc, vc)

        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        seal()
        torch.cuda.synchronize()
        ev[0].record()
        seal()
        ev[1].record()
        for t in range(n_tokens):
            for l in range(L):
                grp.step_layer(l, Q[t, l], Kn[t, l], Vn[t, l], out[l])
        ev[2].record()
        torch.cuda.synchronize()
        seal_ms = ev[0].elapsed_time(ev[1])
        eager_us = ev[1].elapsed_time(ev[2]) * 1e3 / n_tokens

        # one token's L launches captured once and replayed (static inputs)
        sq, sk, sv = Q[0].clone(), Kn[0].clone(), Vn[0].clone()
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for l in range(L):  # warm launch on the capture stream
                grp.step_layer(l, sq[l], sk[l], sv[l], out[l])
        torch.cuda.current_stream().wait_stream(side)
        gc.collect()  # finalise leftovers before the capture (freeing device memory during it aborts)
        with torch.cuda.graph(graph):
            for l in range(L):
                grp.step_layer(l, sq[l], sk[l], sv[l], out[l])
        graph.replay()
        torch.cuda.synchronize()
        ev[2].record()
        for _ in range(n_tokens):
            graph.replay()
        ev[3].record()
        torch.cuda.synchronize()
        graph_us = ev[2].elapsed_time(ev[3]) * 1e3 / n_tokens
        rd, wr = decode_bytes_per_group_step(wl)
        nbytes = (rd + wr) * wl.groups  # one token over every layer
        del graph  # destroyed before the handle's buffers are freed, outside any capture
        grp.close()
        del bufs, Q, Kn, Vn
        torch.cuda.empty_cache()
        return {"launches_per_token": L, "groups_per_launch": B * K, "tokens": n_tokens,
                "seal_ms": seal_ms, "eager_us_per_token": eager_us,
                "graph_us_per_token": graph_us, "graph_us_per_launch": graph_us / L,
                "achieved_GBps_graph": nbytes / (graph_us * 1e-6) / 1e9,
                "frac_of_peak_graph": nbytes / (graph_us * 1e-6) / 1e9 / HBM_PEAK_GBS}
    except Exception as exc:  # context, never the headline
        return {"error": str(exc)[:200]}


# Decode at common model shapes (--model-shapes): (name, n_seq, n_layer, n_kv, hpk, d, dv, m); the
# stack's window, sinks and 256-token prompts, batches that put 2 816 - 16 384 groups in one launch.
MODEL_SHAPES = [
    ("hpk2_d128", 64, 28, 8, 2, 128, 128, 32),
    ("hpk4_d128", 32, 32, 8, 4, 128, 128, 32),
    ("hpk5_d128", 32, 28, 8, 5, 128, 128, 32),
    ("hpk7_d128", 64, 28, 4, 7, 128, 128, 32),
    ("hpk8_d128", 16, 32, 8, 8, 128, 128, 32),
    ("hpk3_d128", 64, 28, 8, 3, 128, 128, 32),
    ("hpk12_d128", 16, 24, 8, 12, 128, 128, 32),
    ("hpk16_d128", 16, 16, 8, 16, 128, 128, 32),
    ("hpk2_d64", 64, 16, 16, 2, 64, 64, 32),
    ("hpk4_d64", 64, 16, 8, 4, 64, 64, 32),
    ("hpk7_d64", 64, 24, 2, 7, 64, 64, 32),
    ("hpk8_d64", 32, 22, 4, 8, 64, 64, 32),
    ("hpk1_d80", 16, 32, 32, 1, 80, 80, 32),
    ("hpk4_d80", 32, 32, 8, 4, 80, 80, 32),
    ("hpk1_d96", 16, 32, 32, 1, 96, 96, 32),
    ("hpk1_d192_v128", 16, 27, 16, 1, 192, 128, 32),
    ("hpk2_d192_v128", 64, 28, 8, 2, 192, 128, 32),
    ("hpk8_d192_v128", 16, 32, 8, 8, 192, 128, 32),
    ("hpk2_d256", 32, 42, 8, 2, 256, 256, 32),
]


def model_shapes(dev, n_steps, only=None):
    """One JSON line per model shape: prefill, then n_steps decode launches twice
    (the first pass warms up), the second timed with HIP events."""
    import torch

    import streaming_nystr_attention_amd as P
    from streaming_nystr_attention_amd import workloads as W

    base = W.WORKLOADS["qwen3_stack_b64"]
    for name, ns, nl, nkv, hpk, d, dv, m in MODEL_SHAPES:
        if only and not any(o in name for o in only):
            continue
        wl = base.with_(name=name, n_seq=ns, n_layer=nl, n_kv=nkv, hpk=hpk, d=d, dv=dv, m=m,
                        layer_scale=None, T=256)
        G = wl.groups
        q, k, v = W.prompt(wl, dev)
        Q = torch.empty(n_steps, G, hpk, d, device=dev)
        K = torch.empty(n_steps, G, d, device=dev)
        V = torch.empty(n_steps, G, dv, device=dev)
        for t in range(n_steps):
            W.decode_inputs(wl, t, dev, out=(Q[t], K[t], V[t]))
        out = torch.empty(G, hpk, dv, device=dev)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        with P.O1Groups(wl.config) as grp:
            for timed in (False, True):
                grp.prefill(q, k, v)
                e[0].record()
                for t in range(n_steps):
                    grp.step(Q[t], K[t], V[t], out)
                e[1].record()
            torch.cuda.synchronize()
        us = e[0].elapsed_time(e[1]) * 1e3 / n_steps
        r = decode_roofline(wl, us)
        print(json.dumps({"shape": name, "groups": G, "hpk": hpk, "d": d, "dv": dv, "m": m,
                          "us_per_launch": us, "frac": r["frac"], "kernel_frac": r["kernel_frac"]}),
              flush=True)
        del q, k, v, Q, K, V, out
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3, help="timed jobs")
    ap.add_argument("--warmup", type=int, default=1, help="untimed jobs first")
    ap.add_argument("--workload", default="qwen3_stack_b64")
    ap.add_argument("--decode-steps", type=int, default=None,
                    help="decode steps per job (default: the workload's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-groups", type=int, default=512,
                    help="groups (whole jobs) in the oracle's timed sample")
    ap.add_argument("--other-workloads", default="stress_m32_s4,stress_m8_s0,wide_gqa,gqa_h8_b16",
                    help="comma-separated workloads whose decode launches are also timed ('' skips)")
    ap.add_argument("--other-steps", type=int, default=256,
                    help="decode launches timed per other workload")
    ap.add_argument("--exact-context", type=int, default=-1,
                    help="also time the exact grouped-GQA comparator over this many keys per "
                         "group (-1: the job's final context, 0: skip)")
    ap.add_argument("--exact-only-steps", type=int, default=64,
                    help="also time this many decode steps in the exact-only mode (0: skip)")
    ap.add_argument("--per-layer-tokens", type=int, default=32,
                    help="also time this many tokens stepped one layer at a time (0: skip)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one device copy of this size (for HBM counter scaling)")
    ap.add_argument("--model-shapes", default=None, metavar="SUBSTRINGS",
                    help="instead of the bench line: decode timing at common model shapes "
                         "('all', or comma-separated name substrings)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: runs on one GPU only; every group is independent, so more "
              "GPUs would each run the same kernel on their own share of the groups. "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import streaming_nystr_attention_amd as P
    from streaming_nystr_attention_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    P.lib()  # fails loudly when the HIP library is missing
    dev = "cuda"
    if args.model_shapes:
        only = None if args.model_shapes == "all" else args.model_shapes.split(",")
        model_shapes(dev, args.decode_steps or 32, only)
        return
    wl = W.WORKLOADS[args.workload]
    n_dec = args.decode_steps or wl.steps
    G, H = wl.groups, wl.hpk

    # ---- inputs resident in HBM before any timing -------------------------
    q, k, v = W.prompt(wl, dev)
    Q = torch.empty(n_dec, G, H, wl.d, device=dev)
    K = torch.empty(n_dec, G, wl.d, device=dev)
    V = torch.empty(n_dec, G, wl.dv, device=dev)
    for t in range(n_dec):
        W.decode_inputs(wl, t, dev, out=(Q[t], K[t], V[t]))
    out = torch.empty(G, H, wl.dv, device=dev)
    grp = P.O1Groups(wl.config)
    torch.cuda.synchronize()

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        a = torch.empty(n, device=dev)
        b = torch.empty(n, device=dev)
        a.fill_(1.0)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    def job():
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        grp.prefill(q, k, v)
        e[1].record()
        for t in range(n_dec):
            grp.step(Q[t], K[t], V[t], out)
        e[2].record()
        return e

    for _ in range(args.warmup):
        job()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    events = [job() for _ in range(args.steps)]
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    prefill_ms = sum(e[0].elapsed_time(e[1]) for e in events) / len(events)
    decode_ms = sum(e[1].elapsed_time(e[2]) for e in events) / len(events)
    launch_us = decode_ms * 1e3 / n_dec
    group_steps = args.steps * n_dec * G
    pf_bytes, pf_flops = prefill_bytes_and_flops(wl)
    roofline = decode_roofline(wl, launch_us, MEASURED_TRAFFIC.get((wl.name, decode_source_sha())))
    roofline["kernel"] = ("decode_kernel<128,128,2>" if (wl.d == 128 and H == 2) else "decode_kernel")

    res = {
        "metric": METRIC,
        "value": group_steps / elapsed,
        "unit": "group-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "n_seq": wl.n_seq, "n_layer": wl.n_layer, "n_kv": wl.n_kv,
            "hpk": H, "d": wl.d, "dv": wl.dv, "m": wl.m, "m_eff": wl.m_eff, "w": wl.w,
            "sink": wl.sink, "prompt_len": wl.T, "decode_steps": n_dec, "groups_per_launch": G,
            "step": "prefill of every group + decode_steps o1_step launches",
            "state": "f32 rows/landmarks/M/T^/running max, f64 Z^; f64 arithmetic",
        },
        "tokens_per_s": args.steps * n_dec * wl.n_seq / elapsed,
        "decode_group_steps_per_s": n_dec * G / (decode_ms * 1e-3),
        "decode_us_per_launch": launch_us,
        "prefill_ms": prefill_ms,
        "roofline": roofline,
        "prefill": {
            "bound": "hbm", "bytes_per_launch": pf_bytes, "ms": prefill_ms,
            "achieved": pf_bytes / (prefill_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": pf_bytes / (prefill_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "far_field_gflop": pf_flops / 1e9,
            "far_field_tflops_over_whole_prefill": pf_flops / (prefill_ms * 1e-3) / 1e12,
            "f64_mfma_peak_tflops": F64_MFMA_PEAK_TFLOPS,
            "far_field_frac_f64_mfma": pf_flops / (prefill_ms * 1e-3) / 1e12 / F64_MFMA_PEAK_TFLOPS,
        },
    }
    ctx = wl.T + n_dec if args.exact_context < 0 else args.exact_context
    if ctx > 0:
        del Q, K, V  # make room for the comparator's KV cache
        torch.cuda.empty_cache()
        res["exact_comparator"] = exact_comparator(wl, ctx, launch_us, dev)
        Q = K = V = None
    if args.exact_only_steps > 0:
        res["exact_only_mode"] = exact_only_mode(wl, args.exact_only_steps, dev)
    if args.per_layer_tokens > 0 and wl.n_layer > 1:
        res["per_layer_mode"] = per_layer_mode(wl, args.per_layer_tokens, dev)
    others = [n for n in args.other_workloads.split(",") if n and n != wl.name]
    if others and args.other_steps > 0:
        del Q, K, V
        torch.cuda.empty_cache()
        Q = None
        res["workloads"] = {n: other_workload(n, args.other_steps, dev) for n in others}
    if not args.no_cpu_baseline:
        if Q is None:
            Q = torch.empty(n_dec, G, H, wl.d, device=dev)
            K = torch.empty(n_dec, G, wl.d, device=dev)
            V = torch.empty(n_dec, G, wl.dv, device=dev)
            for t in range(n_dec):
                W.decode_inputs(wl, t, dev, out=(Q[t], K[t], V[t]))
        threads, share = host_cpu_share()
        res["cpu_baseline"] = cpu_baseline(wl, q, k, v, Q, K, V, n_dec, threads,
                                           min(args.cpu_groups, G), share)
    else:
        res["cpu_baseline"] = None
    grp.close()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
