"""Benchmark of the sparse-page decode step on one MI355X.

One step = the decode-time path of one layer for one batch: refresh the summary of each
sequence's tail page, score every page and select the top-k per (sequence, KV head), and run
the sparse paged decode attention (split-K + merge) over the selected pages -- one
kvsel_select_attend call (scores, then the attention launch with the top-k fused in, then the
merge); the same step as two calls (kvsel_score_topk + kvsel_sparse_decode_attn) is reported
beside it. Inputs are resident in HBM before the timed region.

The step is timed over R copies of the cache at distinct HBM addresses (default 96), used in
turn like the layers of a model: the selected K/V of all copies (96 x 8 MiB at 32K) is three
times the 256 MB Infinity Cache, so a copy's pages and its small per-call data (ids, query,
partials) have been evicted by the time it is visited again (the situation of a real decode,
where every layer, weights included, runs between two visits of one layer's cache). With 48
copies the K/V tiles were already cold but the rest was not: the 32K attention call read 12 %
faster than with 96 or 192 copies, which agree within 1.5 %.
Exactly --warmup untimed steps run first; exactly --steps timed steps (step i on copy i mod R)
are captured in one HIP graph and replayed once between two HIP events.

Prints ONE JSON line: µs/step of the whole path (the headline value), the roofline of the
dominant kernel (the attention call: its time per call from a graph of back-to-back calls between
two HIP events on the replay stream), a plain gather of the same K/V tiles for context, the
128K-context secondary numbers, and the CPU oracle timed on a bounded sample of the same workload
as a baseline.

Usage: python bench.py [--gpus 1] [--steps 400] [--warmup 40] [--workload llama8b_32k]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402
from query_aware_sparse_page_amd import kvsel as K  # noqa: E402
from query_aware_sparse_page_amd.accounting import selected_kv_bytes, summary_bytes  # noqa: E402

HBM_PEAK_GBPS = 8000.0
METRIC = "sparse decode-attn µs/step and achieved HBM GB/s (% of peak) at 32K/128K ctx"


class Layer:
    """One copy of the cache (its own HBM addresses) with preallocated outputs/workspaces."""

    def __init__(self, w, dev, k_pool, v_pool, page_table, seq_lens, fp8=False, rope=None,
                 page_fill=None):
        self.kv = K.PagedKV(k_pool, v_pool, page_table, seq_lens, w.Hq, page_fill=page_fill)
        if fp8:  # E4M3 pages with per-tile scales, quantized on the device
            self.kv = K.quantize_pages(self.kv)
        self.rope = rope  # rotary re-positioning fused into the key gathers, or None
        self.q = w.q.to(dev)
        self.k = w.k
        self.summ = K.build_summaries(self.kv, rope=rope)
        self.sel = torch.empty((w.B, w.Hkv, w.k), dtype=torch.int32, device=dev)
        self.cnt = torch.empty((w.B, w.Hkv), dtype=torch.int32, device=dev)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=dev)
        self.ws_score = K.new_workspace(self.kv, w.k, K.KVSEL_OP_SCORE_TOPK)
        self.ws_attn = K.new_workspace(self.kv, w.k, K.KVSEL_OP_ATTENTION)
        self.ws_fused = K.new_workspace(self.kv, w.k, K.KVSEL_OP_SELECT_ATTEND)

    def select(self):
        K.score_topk(self.kv, self.summ, self.q, self.k, refresh_tail=True, rope=self.rope,
                     sel_idx=self.sel, sel_cnt=self.cnt, workspace=self.ws_score)

    pps = 0  # pages per split: 0 = the library's choice

    def attend(self):
        K.sparse_decode_attn(self.kv, self.q, self.sel, self.cnt, self.k, rope=self.rope,
                             out=self.out, lse=self.lse, pages_per_split=self.pps,
                             workspace=self.ws_attn)

    def probe(self):
        """Plain gather of the K/V tiles the selection names (measurement context)."""
        K.gather_probe(self.probe_addr, self.probe_chunk, self.probe_sink)

    def step(self):
        """The decode step as one kvsel_select_attend call (top-k fused into the attention)."""
        K.select_attend(self.kv, self.summ, self.q, self.k, refresh_tail=True, rope=self.rope,
                        sel_idx=self.sel, sel_cnt=self.cnt, out=self.out, lse=self.lse,
                        workspace=self.ws_fused)

    def step_two_calls(self):
        """The same step as kvsel_score_topk + kvsel_sparse_decode_attn."""
        self.select()
        self.attend()

    def step_current(self):
        """The step over summaries that are already current (as kvsel_append_kv keeps them): no
        tail refresh, so scores + top-k + attention + merge only."""
        K.select_attend(self.kv, self.summ, self.q, self.k, refresh_tail=False, rope=self.rope,
                        sel_idx=self.sel, sel_cnt=self.cnt, out=self.out, lse=self.lse,
                        workspace=self.ws_fused)


def make_layers(w, dev, n, fp8=False):
    """n copies of the cache at distinct HBM addresses, used in turn like a model's layers: each
    has its own K / V pools, summaries, query and outputs; the page table and sequence lengths
    are shared by all, as a serving engine's block table is shared by every layer."""
    k0 = w.k_pool.to(dev)
    v0 = K.device_v_layout(w.v_pool.to(dev))
    table, lens = w.page_table.to(dev), w.seq_lens.to(dev)
    layers = [Layer(w, dev, k0, v0, table, lens, fp8)]
    for _ in range(n - 1):
        layers.append(Layer(w, dev, k0.clone(), v0.clone(), table, lens, fp8))
    torch.cuda.synchronize()
    return layers


def batched_layers(name, dev, n):
    """n independently drawn batches of the same shape (seeds 1006, 1007, ...), each with its own
    pools and page table, drawn on the device, used in turn like layers."""
    layers, first = [], None
    for c in range(n):
        w = W.batched_device(name, dev, seed=1006 + c)
        v = K.device_v_layout(w.v_pool)
        w.v_pool = None  # only the channel-major copy is kept
        lay = Layer(w, dev, w.k_pool, v, w.page_table, w.seq_lens)
        lay.table_cpu = w.page_table.cpu()
        layers.append(lay)
        first = first or w
    torch.cuda.synchronize()
    return first, layers


def time_graph(layers, steps, warmup, step=Layer.step):
    """µs per step of the whole path: exactly ``warmup`` untimed steps (eager), then exactly
    ``steps`` timed steps captured in one HIP graph and replayed once between two HIP events. Step
    i runs on cache copy i mod R, so a timed step reads a copy that R - 1 other copies were used
    after it (cold for R = 96 at 32K: 96 x 8 MiB of selected K/V is three Infinity Caches)."""
    R = len(layers)
    for i in range(warmup):
        step(layers[i % R])
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(warmup, warmup + steps):
            step(layers[i % R])
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1000.0 / steps, steps


def time_calls(layers, fn, launches):
    """Average GPU time (µs) of one ``fn(layer)`` call: ``launches`` calls, rotating over the
    layers, are captured in a HIP graph and replayed back to back between two HIP events on the
    replay stream; the time per call includes the call's own launch gaps, so it equals the sum
    of its kernels' durations in a rocprofv3 kernel trace of the same run."""
    for lay in layers:
        lay.select()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(len(layers)):  # eager warm-up before capture
            fn(layers[i])
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(launches):
            fn(layers[i % len(layers)])
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    reps = 3
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1000.0 / (reps * launches)


def attention_bytes(w, lay):
    """K+V bytes of the selected pages' valid tokens; fp8 pages add their two 4-byte scales."""
    sel = lay.sel.cpu().numpy()
    cnt = lay.cnt.cpu().numpy()
    if lay.kv.is_fp8:
        return selected_kv_bytes(w.seq_lens.tolist(), sel, cnt, w.Hkv, w.P, w.D, 1) + \
            8 * int(cnt.sum())
    esize = 4 if w.dtype == "f32" else 2
    if lay.kv.page_fill is not None:  # a composed context: pages that end early hold fewer tokens
        fill = lay.kv.page_fill.cpu().numpy()
        toks = 0
        for b, L in enumerate(w.seq_lens.tolist()):
            for j in range(w.Hkv):
                for n in sel[b, j, :cnt[b, j]]:
                    p = int(w.page_table[b, int(n)])
                    toks += min(w.P, int(L) - int(n) * w.P, int(fill[p]))
        return 2 * toks * w.D * esize
    return selected_kv_bytes(w.seq_lens.tolist(), sel, cnt, w.Hkv, w.P, w.D, esize)


def progress(msg):
    """One line per finished phase, on stderr (stdout carries only the result line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def measure(name, dev, steps, warmup, n_layers, fp8=False):
    if name in W.BATCHED:
        w, layers = batched_layers(name, dev, n_layers)
    else:
        w = W.make(name)
        layers = make_layers(w, dev, n_layers, fp8)
    us_step, n = time_graph(layers, steps, warmup)
    us_two, _ = time_graph(layers, steps, warmup, Layer.step_two_calls)
    us_current, _ = time_graph(layers, steps, warmup, Layer.step_current)
    n_calls = max(len(layers), min(steps, 512) // len(layers) * len(layers))
    attn_mean = time_calls(layers, Layer.attend, n_calls)
    sel_mean = time_calls(layers, Layer.select, n_calls)
    esize = 1 if fp8 else 4 if w.dtype == "f32" else 2
    for lay in layers:  # the tiles each layer's selection names, at that layer's addresses
        lay.probe_addr = K.tile_addresses(lay.kv, lay.sel, lay.cnt,
                                          getattr(lay, "table_cpu", w.page_table))
        lay.probe_chunk = w.P * w.D * esize
        lay.probe_sink = torch.zeros(1, dtype=torch.int32, device=dev)
    probe_us = time_calls(layers, Layer.probe, n_calls)
    probe_bytes = int(layers[0].probe_addr.numel()) * w.P * w.D * esize
    abytes = attention_bytes(w, layers[0])
    sbytes = summary_bytes(w.seq_lens.tolist(), w.Hkv, w.P, w.D, 2 if fp8 else esize)
    return dict(w=w, layers=layers, us_step=us_step, us_two_calls=us_two, us_current=us_current,
                steps=n, attn_us=attn_mean,
                select_us=sel_mean, attn_bytes=abytes, summary_bytes=sbytes, probe_us=probe_us,
                probe_bytes=probe_bytes, calls_timed=n_calls)


# The sources the attention call's kernels are compiled from: a change to any of them makes the
# committed counter summary stale.
ATTENTION_SOURCES = ("attention.hip", "kvsel_attn.h", "kvsel_device.h", "kvsel_topk.h")


def attention_source_hash():
    import hashlib
    h = hashlib.sha256()
    for name in ATTENTION_SOURCES:
        with open(os.path.join(ROOT, "query_aware_sparse_page_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """Attention HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current attention sources (else None)."""
    path = os.path.join(ROOT, "profiles", "attention_llama8b_32k_counters.md")
    try:
        text = open(path).read()
        sha = attention_source_hash()
    except OSError:
        return None
    vals = dict(line.split("=", 1) for line in text.splitlines() if "=" in line and " " not in line)
    if vals.get("attention_source_sha256_16") != sha:
        return None
    return int(float(vals["attention_traffic_bytes_per_launch"]))


def sweep_pps(name, dev, n_layers, launches=256):
    """Attention call time for each split size (pages per split)."""
    w = W.make(name)
    layers = make_layers(w, dev, n_layers)
    out = {}
    for pps in (1, 2, 4, 8):
        for lay in layers:
            lay.pps = pps
            lay.ws_attn = K.new_workspace(lay.kv, w.k, K.KVSEL_OP_ATTENTION, pps)
        out[pps] = round(time_calls(layers, Layer.attend, launches), 3)
    print(json.dumps({"sweep_pps": name, "attn_us_by_pages_per_split": out}), flush=True)


def speculative(dev, reps=3, tau=None):
    """The speculative workload: a 32K cache built from eight rotary-encoded 4096-token blocks,
    re-positioned on the fly (fused rotary gather), then 64 decode steps with AR(1) queries where
    step t attends over step t-1's pages unless the group-mean query similarity is below tau.
    The 64 steps are one HIP graph, as speculative steps and as serial calls; reports
    µs per step of both (warm: the same cache every step) and the quality statistics."""
    w = W.speculative_rope()
    bt = w.extra["block_tokens"]
    blocks = bt // w.P
    npg = w.num_phys_pages
    cos, sin = K.rope_table(w.extra["theta"], w.D, 0, 8 * bt, dev)
    kv_raw = K.PagedKV(w.k_pool.to(dev), K.device_v_layout(w.v_pool.to(dev)),
                       w.page_table.to(dev), w.seq_lens.to(dev), w.Hq)
    enc_row = torch.from_numpy(((np.arange(npg) % blocks) * w.P).astype(np.int32)).to(dev)
    shift_row = torch.from_numpy(((np.arange(npg) // blocks) * bt).astype(np.int32)).to(dev)
    tau = w.extra["tau"] if tau is None else tau
    enc = K.rope_shift(kv_raw, K.Rope(cos, sin, enc_row, 1))  # the precomputed blocks
    kv = K.PagedKV(enc, kv_raw.v_pool, kv_raw.page_table, kv_raw.seq_lens, w.Hq)
    shift = K.Rope(cos, sin, shift_row, 0)
    summ = K.build_summaries(kv, rope=shift)
    qs = w.extra["q_steps"].to(dev)
    T = qs.shape[0]
    B, Hkv, k = w.B, w.Hkv, w.k
    sel = torch.zeros((T, B, Hkv, k), dtype=torch.int32, device=dev)
    cnt = torch.zeros((T, B, Hkv), dtype=torch.int32, device=dev)
    out = torch.empty((T,) + tuple(w.q.shape), dtype=qs.dtype, device=dev)
    lse = torch.empty((T, B, w.Hq), dtype=torch.float32, device=dev)
    ws_s = K.new_workspace(kv, k, K.KVSEL_OP_SCORE_TOPK)
    spps = K.step_pages_per_split(kv, k)  # the speculative step's split: equal outputs
    ws_a = K.new_workspace(kv, k, K.KVSEL_OP_ATTENTION, spps)
    res = []

    def loop_serial():
        res.clear()
        for t in range(T):
            r = K.score_topk(kv, summ, qs[t], k, sel_idx=sel[t], sel_cnt=cnt[t], workspace=ws_s,
                             reuse=K.Reuse(qs[t - 1] if t else qs[t], sel[t - 1] if t else sel[t],
                                           cnt[t - 1] if t else cnt[t], tau, first_step=(t == 0)))
            res.append(r)
            K.sparse_decode_attn(kv, qs[t], r[2], r[3], k, rope=shift, out=out[t], lse=lse[t],
                                 pages_per_split=spps, workspace=ws_a)

    def loop_overlapped():
        res.clear()
        for t in range(T):
            r = K.speculative_step(kv, summ, qs[t], k,
                                   K.Reuse(qs[t - 1] if t else qs[t], sel[t - 1] if t else sel[t],
                                           cnt[t - 1] if t else cnt[t], tau, first_step=(t == 0)),
                                   rope=shift, sel_idx=sel[t], sel_cnt=cnt[t], out=out[t],
                                   lse=lse[t], workspace=ws_f)
            res.append(r)

    def timed(loop):
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            loop()
        torch.cuda.current_stream().wait_stream(st)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            loop()
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1000.0 / (reps * T)

    ws_f = K.new_workspace(kv, k, K.KVSEL_OP_SPECULATIVE_STEP)
    us_serial = timed(loop_serial)
    out_serial = out.clone()
    us = timed(loop_overlapped)
    torch.cuda.synchronize()
    same = bool(torch.equal(out, out_serial))
    corrected = torch.stack([r[4] for r in res]).cpu().numpy()   # [T][B][Hkv]
    used = torch.stack([r[2] for r in res]).cpu().numpy()
    ucnt = torch.stack([r[3] for r in res]).cpu().numpy()
    fresh, fcnt = sel.cpu().numpy(), cnt.cpu().numpy()
    overlap = []
    for t in range(1, T):
        for b in range(B):
            for j in range(Hkv):
                u = set(used[t, b, j, :ucnt[t, b, j]].tolist())
                f = set(fresh[t, b, j, :fcnt[t, b, j]].tolist())
                overlap.append(len(u & f) / k)
    return {"us_per_step": round(us, 3), "serial_us_per_step": round(us_serial, 3),
            "overlapped_equals_serial": same, "steps": T, "tau": tau, "rho": w.extra["rho"],
            "correction_rate": round(float(corrected[1:].mean()), 4),
            "corrections": int(corrected[1:].sum()), "decisions": int(corrected[1:].size),
            "mean_overlap_used_fresh": round(float(np.mean(overlap)), 4),
            "step": "kvsel_speculative_step: attention over the previous step's pages in the "
                    "same launch as the page scoring and the reuse decision, then the fused "
                    "selection (corrected lists attended again over their fresh pages) and the "
                    "merge; rotary re-positioning fused into the key gather (warm: one cache). "
                    "serial_us_per_step: kvsel_score_topk with reuse, then "
                    "kvsel_sparse_decode_attn over the used pages at the step's split"}


def speculative_growing(dev, reps=3):
    """The speculative workload as a growing-context decode loop: each of the 64 steps appends the
    new token's key and value (kvsel_append_kv, which keeps the tail page's summary current, so no
    refresh is needed), then runs the speculative step over the grown cache (32768 -> 32832
    tokens; the pool has two more pages for them, which the appends take from a device-side
    free-page list into the table; the new keys are stored as given, without a rotary shift). The
    graph of 64 steps starts by resetting the length and the free count, so every replay grows the
    same cache. Reports µs per step (append + speculative step) against the serial
    calls (append + kvsel_score_topk with reuse + kvsel_sparse_decode_attn)."""
    w = W.speculative_rope()
    bt = w.extra["block_tokens"]
    blocks = bt // w.P
    npg = w.num_phys_pages
    qs = w.extra["q_steps"].to(dev)
    T, tau = qs.shape[0], w.extra["tau"]
    extra = -(-T // w.P)
    cos, sin = K.rope_table(w.extra["theta"], w.D, 0, 8 * bt, dev)
    kv_raw = K.PagedKV(w.k_pool.to(dev), K.device_v_layout(w.v_pool.to(dev)),
                       w.page_table.to(dev), w.seq_lens.to(dev), w.Hq)
    enc_row = torch.from_numpy(((np.arange(npg) % blocks) * w.P).astype(np.int32)).to(dev)
    enc = K.rope_shift(kv_raw, K.Rope(cos, sin, enc_row, 1))  # the precomputed blocks
    k_pool = torch.cat([enc, torch.zeros((extra,) + tuple(enc.shape[1:]), dtype=enc.dtype,
                                         device=dev)])
    v_pool = torch.cat([kv_raw.v_pool, torch.zeros((extra,) + tuple(kv_raw.v_pool.shape[1:]),
                                                   dtype=enc.dtype, device=dev)])
    table = torch.zeros((w.B, w.max_pages + extra), dtype=torch.int32)
    table[:, : w.max_pages] = w.page_table
    table[0, w.max_pages:] = -1  # set by the appends from the free list
    free_ids = torch.arange(npg + extra - 1, npg - 1, -1, dtype=torch.int32, device=dev)
    free_n0 = torch.tensor([extra], dtype=torch.int32, device=dev)
    free = K.FreePages(free_ids, free_n0.clone())
    lens0 = w.seq_lens.to(dev)
    lens = lens0.clone()
    kv = K.PagedKV(k_pool, v_pool, table.to(dev), lens, w.Hq,
                   max_seq_len=int(w.seq_lens.max()) + T)  # the longest length the loop reaches
    shift_row = torch.full((npg + extra,), -1, dtype=torch.int32)
    shift_row[:npg] = torch.from_numpy(((np.arange(npg) // blocks) * bt).astype(np.int32))
    shift = K.Rope(cos, sin, shift_row.to(dev), 0)
    summ = K.build_summaries(kv, rope=shift)
    ks, vs = W.appended_tokens(w, T, seed=2005)
    ks, vs = ks.to(dev), vs.to(dev)
    B, Hkv, k = w.B, w.Hkv, w.k
    sel = torch.zeros((T, B, Hkv, k), dtype=torch.int32, device=dev)
    cnt = torch.zeros((T, B, Hkv), dtype=torch.int32, device=dev)
    out = torch.empty((T,) + tuple(w.q.shape), dtype=qs.dtype, device=dev)
    lse = torch.empty((T, B, w.Hq), dtype=torch.float32, device=dev)
    ws_s = K.new_workspace(kv, k, K.KVSEL_OP_SCORE_TOPK)
    spps = K.step_pages_per_split(kv, k)  # the speculative step's split: equal outputs
    ws_a = K.new_workspace(kv, k, K.KVSEL_OP_ATTENTION, spps)
    ws_f = K.new_workspace(kv, k, K.KVSEL_OP_SPECULATIVE_STEP)

    def reuse(t):
        return K.Reuse(qs[t - 1] if t else qs[t], sel[t - 1] if t else sel[t],
                       cnt[t - 1] if t else cnt[t], tau, first_step=(t == 0))

    def loop_serial():
        lens.copy_(lens0)
        free.count.copy_(free_n0)
        for t in range(T):
            K.append_kv(kv, ks[t], vs[t], summ=summ, free_pages=free)
            r = K.score_topk(kv, summ, qs[t], k, sel_idx=sel[t], sel_cnt=cnt[t], workspace=ws_s,
                             reuse=reuse(t))
            K.sparse_decode_attn(kv, qs[t], r[2], r[3], k, rope=shift, out=out[t], lse=lse[t],
                                 pages_per_split=spps, workspace=ws_a)

    def loop_speculative():
        lens.copy_(lens0)
        free.count.copy_(free_n0)
        for t in range(T):
            K.append_kv(kv, ks[t], vs[t], summ=summ, free_pages=free)
            K.speculative_step(kv, summ, qs[t], k, reuse(t), rope=shift, sel_idx=sel[t],
                               sel_cnt=cnt[t], out=out[t], lse=lse[t], workspace=ws_f)

    def timed(loop):
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            loop()
        torch.cuda.current_stream().wait_stream(st)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            loop()
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1000.0 / (reps * T)

    us_serial = timed(loop_serial)
    out_serial = out.clone()
    us = timed(loop_speculative)
    torch.cuda.synchronize()
    return {"us_per_step": round(us, 3), "serial_us_per_step": round(us_serial, 3),
            "speculative_equals_serial": bool(torch.equal(out, out_serial)),
            "final_len": int(lens.item()), "free_pages_left": int(free.count.item()), "steps": T,
            "step": "kvsel_append_kv (pages from a device-side free list), then "
                    "kvsel_speculative_step over the grown cache (warm); "
                    "serial: kvsel_append_kv, kvsel_score_topk with reuse, "
                    "kvsel_sparse_decode_attn at the step's split"}


COMPOSED_DOCS = (4000, 3100, 517, 2900, 6000, 1, 3333, 2048, 4500, 1234, 777, 3600)


def composed_context(dev, steps, warmup, n_layers=96):
    """A 32K-token context composed of 12 independently cached documents of ragged lengths
    (the positional half of RAG reuse): each document's keys encoded at its own positions
    [0, len), its pages chained in the context with the last page of each document ending early
    (page_fill), and every page moved to its composed position by a rotary shift fused into the
    key gathers. Same step and timing as the headline (one kvsel_select_attend call per layer
    copy, 96 copies rotated)."""
    w = W.composed(1007, doc_lens=COMPOSED_DOCS, B=1, k=64)
    page_in_doc = w.extra["page_in_doc"].numpy()
    doc_of_page = w.extra["doc_of_page"].numpy()
    start = w.extra["doc_start"].numpy()[0]
    cos, sin = K.rope_table(w.extra["theta"], w.D, 0, int(start.max()) + max(COMPOSED_DOCS) + w.P,
                            dev)
    table, lens = w.page_table.to(dev), w.seq_lens.to(dev)
    fill = w.extra["page_fill"].to(dev)
    v0 = K.device_v_layout(w.v_pool.to(dev))
    raw = K.PagedKV(w.k_pool.to(dev), v0, table, lens, w.Hq, page_fill=fill)
    enc_row = torch.from_numpy((page_in_doc * w.P).astype(np.int32)).to(dev)
    k0 = K.rope_shift(raw, K.Rope(cos, sin, enc_row, 1))  # the documents as cached
    shift = K.Rope(cos, sin, torch.from_numpy(start[doc_of_page].astype(np.int32)).to(dev), 0)
    layers = [Layer(w, dev, k0 if i == 0 else k0.clone(), v0 if i == 0 else v0.clone(), table,
                    lens, rope=shift, page_fill=fill) for i in range(n_layers)]
    torch.cuda.synchronize()
    us_step, _ = time_graph(layers, steps, warmup)
    n_calls = max(len(layers), min(steps, 512) // len(layers) * len(layers))
    attn_us = time_calls(layers, Layer.attend, n_calls)
    abytes = attention_bytes(w, layers[0])
    return {"us_per_step": round(us_step, 3), "attn_us": round(attn_us, 3),
            "attn_GBps": round(abytes / (attn_us * 1e-6) / 1e9, 1), "attn_bytes": abytes,
            "context_slots": int(w.seq_lens[0]), "documents": len(COMPOSED_DOCS),
            "tokens": int(sum(COMPOSED_DOCS)), "layers_rotated": n_layers,
            "step": "kvsel_select_attend over the composed context: tail refresh, scores, top-k "
                    "and attention, every key gather rotating its page by its document's offset"}


def cpu_baseline(w, lay, budget_s=12.0):
    """The oracle's decode step (tail summary + scores + top-k + attention) on the host, for a
    bounded number of repetitions of the same workload; also checks the GPU's step output."""
    import oracle as O
    from threadpoolctl import threadpool_limits

    scale = K.default_scale(w.D)
    summ = O.page_summaries(w.k_pool, w.page_table, w.seq_lens, w.P)  # prefill, untimed
    times = []
    with threadpool_limits(limits=1):
        t_end = time.perf_counter() + budget_s
        while True:
            t0 = time.perf_counter()
            for b in range(w.B):  # decode-time refresh of each tail page's summary
                L = int(w.seq_lens[b])
                n = (L - 1) // w.P
                p = int(w.page_table[b, n])
                toks = O.as_f64(w.k_pool[p, :, :L - n * w.P])
                summ[p, :, 0] = toks.min(axis=1)
                summ[p, :, 1] = toks.max(axis=1)
            sel, cnt, out, lse = O.decode_step(w.q, summ, w.k_pool, w.v_pool, w.page_table,
                                               w.seq_lens, w.P, w.k, scale)
            times.append(time.perf_counter() - t0)
            if time.perf_counter() > t_end or len(times) >= 50:
                break
    ok_sel = bool(np.array_equal(lay.sel.cpu().numpy(), sel) and
                  np.array_equal(lay.cnt.cpu().numpy(), cnt))
    err = float(np.abs(lay.out.float().cpu().numpy() - out).max())
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    host = dict(affinity=len(os.sched_getaffinity(0)), cpu_count=os.cpu_count(), model=model)
    return dict(value=float(np.median(times)) * 1e6, unit="us/step", cores=1, kind="oracle",
                host=host,
                sample=f"{len(times)} full decode steps of the same workload (B={w.B}, "
                       f"ctx={int(w.seq_lens.max())}), fp64 NumPy, 1 thread",
                parity=dict(selection_bit_exact=ok_sel, attention_max_abs_err=err))


def counter_pass(name, dev, n_layers, split_sizes=()):
    """Eager steps over the rotated layers (and attention calls at the given split sizes), then a
    plain device copy of exactly 64 MiB: its FETCH_SIZE / WRITE_SIZE per dispatch calibrate the
    counters against known bytes."""
    if name in W.BATCHED:
        w, layers = batched_layers(name, dev, n_layers)
    else:
        w = W.make(name)
        layers = make_layers(w, dev, n_layers)
    for _ in range(2):
        for lay in layers:
            lay.step()  # kvsel_select_attend
        for lay in layers:
            lay.step_two_calls()  # kvsel_score_topk + kvsel_sparse_decode_attn
    torch.cuda.synchronize()
    if split_sizes:  # the attention call at other split sizes (dispatches differ in grid size)
        for pps in split_sizes:
            for lay in layers:
                lay.pps = pps
                lay.ws_attn = K.new_workspace(lay.kv, w.k, K.KVSEL_OP_ATTENTION, pps)
            for _ in range(2):
                for lay in layers:
                    lay.attend()
            torch.cuda.synchronize()
    src = torch.empty(64 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"counter_pass": name, "layers": n_layers, "steps_per_form": 2 * n_layers,
                      "calibration_copy_bytes": 64 << 20,
                      "attention_source_sha256_16": attention_source_hash()}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="llama8b_32k")
    ap.add_argument("--layers", type=int, default=96,
                    help="cache copies rotated like layers (96 x 8 MiB of selected K/V is three "
                         "times the 256 MB Infinity Cache, so every call reads HBM)")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--sweep-pps", action="store_true",
                    help="time the attention call for each split size and exit")
    ap.add_argument("--counter-pass", action="store_true",
                    help="only run a few eager steps plus a 64 MiB calibration copy (for rocprofv3 "
                         "--pmc FETCH_SIZE / WRITE_SIZE runs) and exit")
    ap.add_argument("--counter-splits", default="",
                    help="with --counter-pass: comma-separated split sizes (pages per split) at "
                         "which the attention call also runs")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    K.lib()
    if args.counter_pass:
        counter_pass(args.workload, dev, args.layers,
                     [int(x) for x in args.counter_splits.split(",") if x])
        return
    if args.sweep_pps:
        for name in (args.workload, "qwen4b_128k", "ragged_batch"):
            sweep_pps(name, dev, args.layers // 2)
            torch.cuda.empty_cache()
        return

    m = measure(args.workload, dev, args.steps, args.warmup, args.layers)
    w = m["w"]
    achieved = m["attn_bytes"] / (m["attn_us"] * 1e-6) / 1e9
    result = {
        "metric": METRIC,
        "value": round(m["us_step"], 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": m["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(m["us_step"] / 1000.0, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
            "head_dim": w.D, "context": int(w.seq_lens.max()), "page_size": w.P,
            "topk_pages": w.k, "layers_rotated": args.layers,
            "step": "tail-page summary refresh + page scores + top-k + sparse attention "
                    "(one kvsel_select_attend call)",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "kvsel_sparse_decode_attn: attn_bf16_kernel (split-K) + attn_merge_kernel",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": recorded_traffic() if w.name == "llama8b_32k" else None,
            "algorithmic_bytes": m["attn_bytes"],
            "avg_us": round(m["attn_us"], 3),
            "calls_timed": m["calls_timed"],
            # the same K/V tiles moved by a plain gather (no index chain, math or merge)
            "gather_probe": {"bytes": m["probe_bytes"], "avg_us": round(m["probe_us"], 3),
                             "GBps": round(m["probe_bytes"] / (m["probe_us"] * 1e-6) / 1e9, 1)},
        },
        "select_us": round(m["select_us"], 3),
        "two_call_us_per_step": round(m["us_two_calls"], 3),
        # the same step over summaries already current (no tail refresh): scores + top-k +
        # attention + merge, the decode step after kvsel_append_kv has updated the tail summary
        "step_current_summaries_us": round(m["us_current"], 3),
    }
    keep = m["layers"][0]  # its last step's outputs are checked against the CPU oracle
    del m["layers"]
    torch.cuda.empty_cache()
    progress(f"{w.name}: step {result['value']} us, attention call {m['attn_us']:.3f} us")
    # the 128K case of the metric, and the batched case whose 64 MiB per step is where bandwidth
    # rather than latency sets the time
    # and both again with fp8 (E4M3) pages: half the bytes of the selected K/V
    # and batches of the 32K and 128K shapes (256 MiB of selected K/V per step, two independently
    # drawn batches rotated), where the attention call is bandwidth-bound
    # (each rotation moves about 768 MiB of selected K/V at the default --layers 96)
    for name, n_layers, fp8 in (("qwen4b_128k", max(2, args.layers // 2), False),
                                ("ragged_batch", max(2, args.layers // 8), False),
                                (args.workload, 2 * args.layers, True),
                                ("ragged_batch", max(2, args.layers // 4), True),
                                ("llama8b_32k_batch32", 3, False),
                                ("qwen4b_128k_batch16", 3, False)):
        if args.no_secondary or (name == args.workload and not fp8):
            continue
        s = measure(name, dev, args.steps, args.warmup, n_layers, fp8)
        sach = s["attn_bytes"] / (s["attn_us"] * 1e-6) / 1e9
        key = name + ("_fp8" if fp8 else "")
        result.setdefault("secondary", {})[key] = {
            "us_per_step": round(s["us_step"], 3),
            "two_call_us_per_step": round(s["us_two_calls"], 3),
            "step_current_summaries_us": round(s["us_current"], 3), "attn_us": round(s["attn_us"], 3),
            "attn_GBps": round(sach, 1), "attn_frac": round(sach / HBM_PEAK_GBPS, 4),
            "select_us": round(s["select_us"], 3), "attn_bytes": s["attn_bytes"],
            "layers_rotated": n_layers,
            "gather_probe": {"avg_us": round(s["probe_us"], 3),
                             "GBps": round(s["probe_bytes"] / (s["probe_us"] * 1e-6) / 1e9, 1)}}
        if fp8:
            result["secondary"][key]["pages"] = "fp8 E4M3 K/V, per-tile fp32 scales, bf16 summaries"
        if name in W.BATCHED:
            result["secondary"][key].update(
                batch=s["w"].B, context=int(s["w"].seq_lens.max()), topk_pages=s["w"].k,
                data="drawn on the device (workloads.batched_device)")
        progress(f"{key}: step {s['us_step']:.3f} us, attention call {s['attn_us']:.3f} us")
        del s
        torch.cuda.empty_cache()
    if not args.no_secondary:
        result.setdefault("secondary", {})["speculative_rope_64_steps"] = speculative(dev)
        progress("speculative workload done")
        torch.cuda.empty_cache()
        # the same loop at tau 0.85, where about half the decisions correct (re-select and
        # re-attend inside the speculative step)
        result["secondary"]["speculative_rope_64_steps_tau0.85"] = speculative(dev, tau=0.85)
        progress("speculative workload (tau 0.85) done")
        torch.cuda.empty_cache()
        result["secondary"]["speculative_growing_64_steps"] = speculative_growing(dev)
        progress("growing speculative workload done")
        torch.cuda.empty_cache()
        result["secondary"]["composed_32k_12_documents"] = composed_context(dev, args.steps,
                                                                           args.warmup,
                                                                           args.layers)
        progress("composed-context workload done")
        torch.cuda.empty_cache()
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(w, keep)
        progress("cpu baseline done")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
