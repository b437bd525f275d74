"""Seeded synthetic inputs for the sparse-page decode workloads.

This module is shared by the CPU oracle's tests, the GPU parity tests and the benchmark. It holds
random draws, shapes and the layout of the paged KV pool only: none of the arithmetic of the
method itself (no page summary, no score, no selection, no attention, no rotary rotation).

The shapes follow the pages' workloads:
  * a paged KV cache with fixed-size token pages and grouped-query heads ("Key-Value (KV) Cache"
    wiki page, the PagedAttention and GQA entries);
  * Llama-3.1-8B / Qwen-3-4B shaped long-context decode (the KV Packet review, section 3, names
    both models);
  * strongly correlated queries of adjacent decode steps (FreeKV summary, section 2.1: cosine of
    about 0.84 or more between neighbouring steps' queries).

Every tensor is a CPU torch tensor; callers move it to the device (except ``batched_device``,
whose batches of long contexts are drawn on the device: several GiB per pool). bf16 values are produced by
round-to-nearest-even of fp32/fp64 draws (torch's conversion).

Seeds: workload ``i`` (1-based) draws from ``numpy.random.Generator(PCG64(1000 + i))`` unless a
seed is given, in a fixed order: q, K, V, structure (plants / needles / outliers), page table.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np
import torch

__all__ = [
    "Workload",
    "WORKLOADS",
    "make",
    "tiny_fp32",
    "llama8b_32k",
    "ragged_batch",
    "qwen4b_128k",
    "speculative_rope",
    "composed",
    "custom",
    "BATCHED",
    "batched_device",
]


@dataclass
class Workload:
    """One decode problem over a paged GQA KV cache.

    Pool layout: ``k_pool``/``v_pool`` are ``[num_phys_pages][Hkv][P][D]``; ``page_table[b][n]``
    is the physical page holding logical page ``n`` of sequence ``b``; ``seq_lens[b]`` is the
    number of valid tokens. Entries of ``page_table`` at or beyond ``ceil(L_b / P)`` are 0 and
    never read.
    """

    name: str
    dtype: str  # "f32" or "bf16"
    B: int
    Hq: int
    Hkv: int
    D: int
    P: int
    k: int  # pages selected per (sequence, KV head)
    seq_lens: torch.Tensor  # int32 [B]
    page_table: torch.Tensor  # int32 [B][max_pages]
    k_pool: torch.Tensor  # [Npp][Hkv][P][D]
    v_pool: torch.Tensor  # [Npp][Hkv][P][D]
    q: torch.Tensor  # [B][Hq][D] (first decode step)
    extra: Dict[str, object] = field(default_factory=dict)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def num_phys_pages(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    def n_pages(self, b: int) -> int:
        return -(-int(self.seq_lens[b]) // self.P)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _to(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"element type {dtype!r}: expected 'f32' or 'bf16'")
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t if dtype == "f32" else t.to(torch.bfloat16)


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float64)


def _identity_table(B: int, n_pages: int) -> torch.Tensor:
    return torch.arange(B * n_pages, dtype=torch.int32).reshape(B, n_pages)


def _outlier_channels(rng: np.random.Generator, Hkv: int, D: int, n: int = 4) -> np.ndarray:
    return np.stack([rng.choice(D, size=n, replace=False) for _ in range(Hkv)])


def _apply_outliers(keys: np.ndarray, chans: np.ndarray, scale: float = 8.0) -> None:
    # keys: [Npp][Hkv][P][D]; channels chans[j] of KV head j are scaled in place
    for j in range(chans.shape[0]):
        keys[:, j, :, chans[j]] *= scale


def tiny_fp32(seed: int = 1001) -> Workload:
    """1 sequence, 8 query / 2 KV heads, D 64, 1024 tokens, P 16 (64 pages), k 16, fp32.

    q, K, V ~ N(0,1); four planted tokens in four distinct pages. At planted token g (g = 0..3)
    the key of KV head j is 3*sqrt(D) * q[j*G + g] / |q[j*G + g]|, so every query head of a group
    has one strongly matching token and selection is not trivial.
    """
    B, Hq, Hkv, D, L, P, k = 1, 8, 2, 64, 1024, 16, 16
    G = Hq // Hkv
    rng = _rng(seed)
    q = _normal(rng, (B, Hq, D)).astype(np.float32).astype(np.float64)
    npg = L // P
    K = _normal(rng, (npg, Hkv, P, D))
    V = _normal(rng, (npg, Hkv, P, D))
    pages = rng.choice(npg, size=G, replace=False)
    slots = rng.integers(0, P, size=G)
    for g in range(G):
        for j in range(Hkv):
            qh = q[0, j * G + g]
            K[pages[g], j, slots[g]] = 3.0 * np.sqrt(D) * qh / np.linalg.norm(qh)
    return Workload(
        "tiny_fp32", "f32", B, Hq, Hkv, D, P, k,
        seq_lens=torch.tensor([L], dtype=torch.int32),
        page_table=_identity_table(B, npg),
        k_pool=_to(K, "f32"), v_pool=_to(V, "f32"), q=_to(q, "f32"),
        extra={"planted_pages": pages.tolist(), "planted_slots": slots.tolist()},
    )


def llama8b_32k(seed: int = 1002, context: int = 32768, budget_tokens: int = 2048) -> Workload:
    """Llama-3.1-8B-shaped decode step: B 1, 32 / 8 heads, D 128, bf16, P 32, top-k = budget / P.

    q, V ~ N(0,1); K ~ N(0,1) with 4 outlier channels per KV head scaled by 8.
    """
    B, Hq, Hkv, D, P = 1, 32, 8, 128, 32
    rng = _rng(seed)
    q = _normal(rng, (B, Hq, D))
    npg = -(-context // P)
    K = _normal(rng, (npg, Hkv, P, D))
    V = _normal(rng, (npg, Hkv, P, D))
    chans = _outlier_channels(rng, Hkv, D)
    _apply_outliers(K, chans)
    return Workload(
        "llama8b_32k", "bf16", B, Hq, Hkv, D, P, budget_tokens // P,
        seq_lens=torch.tensor([context], dtype=torch.int32),
        page_table=_identity_table(B, npg),
        k_pool=_to(K, "bf16"), v_pool=_to(V, "bf16"), q=_to(q, "bf16"),
        extra={"outlier_channels": chans.tolist()},
    )


def ragged_batch(seed: int = 1003, B: int = 16, lo: int = 4096, hi: int = 16384,
                 budget_tokens: int = 1024) -> Workload:
    """Batch of 16 sequences with lengths uniform in [4096, 16384], shared paged pool.

    32 / 8 heads, D 128, bf16, P 32, k = 1024 / 32 = 32. q, V ~ N(0,1); K as in the 32K case
    (4 outlier channels per KV head, x8). One random permutation of the pool's pages is laid out
    over all (sequence, logical page) pairs in order, so every sequence's table is permuted.
    """
    Hq, Hkv, D, P = 32, 8, 128, 32
    rng = _rng(seed)
    q = _normal(rng, (B, Hq, D))
    lens = rng.integers(lo, hi + 1, size=B)
    npgs = [-(-int(L) // P) for L in lens]
    Npp = int(sum(npgs))
    K = _normal(rng, (Npp, Hkv, P, D))
    V = _normal(rng, (Npp, Hkv, P, D))
    chans = _outlier_channels(rng, Hkv, D)
    _apply_outliers(K, chans)
    perm = rng.permutation(Npp)
    maxp = max(npgs)
    table = np.zeros((B, maxp), dtype=np.int32)
    off = 0
    for b, n in enumerate(npgs):
        table[b, :n] = perm[off:off + n]
        off += n
    return Workload(
        "ragged_batch", "bf16", B, Hq, Hkv, D, P, budget_tokens // P,
        seq_lens=torch.tensor(lens, dtype=torch.int32),
        page_table=torch.from_numpy(table),
        k_pool=_to(K, "bf16"), v_pool=_to(V, "bf16"), q=_to(q, "bf16"),
        extra={"outlier_channels": chans.tolist()},
    )


def qwen4b_128k(seed: int = 1004, context: int = 131072, budget_tokens: int = 4096,
                n_needles: int = 16, cosine: float = 0.9) -> Workload:
    """Qwen-3-4B-shaped long context: B 1, 32 / 8 heads, D 128, bf16, P 32, k = 4096 / 32 = 128.

    q, K, V ~ N(0,1), plus 16 needle pages (distinct logical pages, shared by all KV heads). In a
    needle page of KV head j the 32 keys are (noise - its token mean) + m_j with
    m_j = sqrt(D) * (c * u + sqrt(1 - c^2) * w): u is the unit vector along the sum of the group's
    (bf16) queries, w a random unit vector orthogonal to u, c = 0.9. The needle page's mean key
    therefore has cosine c with the group's query direction (before bf16 rounding).
    """
    B, Hq, Hkv, D, P = 1, 32, 8, 128, 32
    G = Hq // Hkv
    rng = _rng(seed)
    q = torch.from_numpy(_normal(rng, (B, Hq, D)).astype(np.float32)).to(torch.bfloat16)
    qd = q.to(torch.float64).numpy()
    npg = -(-context // P)
    K = _normal(rng, (npg, Hkv, P, D))
    V = _normal(rng, (npg, Hkv, P, D))
    needles = np.sort(rng.choice(npg, size=n_needles, replace=False))
    for j in range(Hkv):
        u = qd[0, j * G:(j + 1) * G].sum(axis=0)
        u /= np.linalg.norm(u)
        for p in needles:
            w = _normal(rng, (D,))
            w -= (w @ u) * u
            w /= np.linalg.norm(w)
            m = np.sqrt(D) * (cosine * u + np.sqrt(1.0 - cosine * cosine) * w)
            noise = K[p, j]
            K[p, j] = noise - noise.mean(axis=0, keepdims=True) + m
    return Workload(
        "qwen4b_128k", "bf16", B, Hq, Hkv, D, P, budget_tokens // P,
        seq_lens=torch.tensor([context], dtype=torch.int32),
        page_table=_identity_table(B, npg),
        k_pool=_to(K, "bf16"), v_pool=_to(V, "bf16"), q=q,
        extra={"needle_pages": needles.tolist()},
    )


def speculative_rope(seed: int = 1005, steps: int = 64, rho: float = 0.85, tau: float = 0.8,
                     context: int = 32768, block_tokens: int = 4096,
                     theta: float = 500000.0) -> Workload:
    """32K Llama-shaped cache built from precomputed blocks, plus a run of correlated queries.

    Shapes as the 32K case (B 1, 32 / 8 heads, D 128, bf16, P 32, k 64). Queries follow
    q_t = rho * q_{t-1} + sqrt(1 - rho^2) * eps_t per head (fp32, on unrounded values; the bf16
    copy of each step is the input). ``k_pool`` holds the RAW (un-rotated) keys, N(0,1) with 4
    outlier channels per KV head (x8); the rotary encoding of each 4096-token block at positions
    0..4095 and its re-positioning to offset 4096 * block are steps of the method, done by each
    side. ``extra['q_steps']`` is bf16 [steps][B][Hq][D].
    """
    B, Hq, Hkv, D, P = 1, 32, 8, 128, 32
    rng = _rng(seed)
    q0 = _normal(rng, (B, Hq, D)).astype(np.float32)
    npg = -(-context // P)
    K = _normal(rng, (npg, Hkv, P, D))
    V = _normal(rng, (npg, Hkv, P, D))
    chans = _outlier_channels(rng, Hkv, D)
    _apply_outliers(K, chans)
    qs = [q0]
    a = np.float32(rho)
    c = np.float32(np.sqrt(1.0 - rho * rho))
    for _ in range(1, steps):
        eps = _normal(rng, (B, Hq, D)).astype(np.float32)
        qs.append((a * qs[-1] + c * eps).astype(np.float32))
    q_steps = torch.from_numpy(np.stack(qs)).to(torch.bfloat16)
    return Workload(
        "speculative_rope", "bf16", B, Hq, Hkv, D, P, 2048 // P,
        seq_lens=torch.tensor([context], dtype=torch.int32),
        page_table=_identity_table(B, npg),
        k_pool=_to(K, "bf16"), v_pool=_to(V, "bf16"), q=q_steps[0].clone(),
        extra={"q_steps": q_steps, "rho": rho, "tau": tau, "theta": theta,
               "block_tokens": block_tokens, "outlier_channels": chans.tolist()},
    )


def appended_tokens(w: Workload, steps: int, seed: int):
    """Keys and values of `steps` decode tokens per sequence, appended one per step to `w`'s cache
    (a growing-context decode loop): drawn like the cache's own (N(0,1); keys scaled x8 on the
    workload's outlier channels when it has them). Returns (k_steps, v_steps), each
    [steps][B][Hkv][D] in the workload's element type."""
    rng = _rng(seed)
    K = _normal(rng, (steps, w.B, w.Hkv, w.D))
    V = _normal(rng, (steps, w.B, w.Hkv, w.D))
    chans = w.extra.get("outlier_channels")
    if chans is not None:
        for j, cs in enumerate(chans):
            K[:, :, j, cs] *= 8.0
    return _to(K, w.dtype), _to(V, w.dtype)


def custom(seed: int, B: int, Hq: int, Hkv: int, D: int, P: int, k: int, lens, dtype: str = "bf16",
           permute: bool = True, spare_pages: int = 0) -> Workload:
    """Small seeded case with arbitrary shapes (for edge-case tests): q, K, V ~ N(0,1).

    ``lens`` gives each sequence's token count (0 allowed). With ``permute`` the pool's pages are
    shuffled over the (sequence, logical page) pairs; ``spare_pages`` adds unreferenced pages.
    """
    rng = _rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    q = _normal(rng, (B, Hq, D))
    npgs = [-(-int(L) // P) for L in lens]
    Npp = int(sum(npgs)) + spare_pages
    Npp = max(Npp, 1)
    K = _normal(rng, (Npp, Hkv, P, D))
    V = _normal(rng, (Npp, Hkv, P, D))
    perm = rng.permutation(Npp) if permute else np.arange(Npp)
    maxp = max(max(npgs), 1)
    table = np.zeros((B, maxp), dtype=np.int32)
    off = 0
    for b, n in enumerate(npgs):
        table[b, :n] = perm[off:off + n]
        off += n
    return Workload(
        f"custom_{seed}", dtype, B, Hq, Hkv, D, P, k,
        seq_lens=torch.tensor(lens, dtype=torch.int32),
        page_table=torch.from_numpy(table),
        k_pool=_to(K, dtype), v_pool=_to(V, dtype), q=_to(q, dtype),
    )


def composed(seed: int = 1006, doc_lens=(3000, 517, 4099, 1, 2222, 700, 5120, 31), order=None,
             B: int = 1, Hq: int = 32, Hkv: int = 8, D: int = 128, P: int = 32, k: int = 48,
             dtype: str = "bf16", lead: int = 0, theta: float = 500000.0) -> Workload:
    """Contexts composed of independently cached documents (the positional half of RAG reuse).

    Document i holds doc_lens[i] tokens in pages of its own; its last page holds
    doc_lens[i] % P valid slots when that is not 0 (``page_fill`` gives every physical page's
    valid slots). Sequence b chains the documents' pages in ``order[b]`` (default: document order
    for b = 0, rotated by b for later sequences, so sequences share documents in different
    orders); its length counts slots, holes included. In sequence b the document at chain
    position c starts at position lead + the tokens of the documents before it. Keys, values and
    the query are N(0,1) with the usual outlier key channels; physical pages are shuffled.

    extra: page_fill int32 [Npp]; page_in_doc int32 [Npp] (index of the page within its
    document); doc_of_page int32 [Npp]; doc_start int32 [B][n_docs] (position of each document in
    sequence b); theta (the rotary base of the positional tests).
    """
    rng = _rng(seed)
    n_docs = len(doc_lens)
    if order is None:
        order = [[(c + b) % n_docs for c in range(n_docs)] for b in range(B)]
    pages_of = [-(-int(L) // P) for L in doc_lens]
    Npp = int(sum(pages_of))
    perm = rng.permutation(Npp)
    doc_pages, off = [], 0
    page_fill = np.full(Npp, P, dtype=np.int32)
    page_in_doc = np.zeros(Npp, dtype=np.int32)
    doc_of_page = np.zeros(Npp, dtype=np.int32)
    for i, L in enumerate(doc_lens):
        pg = perm[off:off + pages_of[i]]
        off += pages_of[i]
        doc_pages.append(pg)
        page_in_doc[pg] = np.arange(len(pg), dtype=np.int32)
        doc_of_page[pg] = i
        if L % P:
            page_fill[pg[-1]] = L % P
    width = max(sum(pages_of[i] for i in o) for o in order)
    table = np.zeros((B, width), dtype=np.int32)
    lens = np.zeros(B, dtype=np.int64)
    doc_start = np.zeros((B, n_docs), dtype=np.int32)
    for b, o in enumerate(order):
        chain = np.concatenate([doc_pages[i] for i in o])
        table[b, :len(chain)] = chain
        lens[b] = (len(chain) - 1) * P + int(page_fill[chain[-1]])
        pos = lead
        for i in o:
            doc_start[b, i] = pos
            pos += int(doc_lens[i])
    chans = _outlier_channels(rng, Hkv, D)
    K = _normal(rng, (Npp, Hkv, P, D))
    _apply_outliers(K, chans)
    V = _normal(rng, (Npp, Hkv, P, D))
    q = _normal(rng, (B, Hq, D))
    return Workload(
        "composed", dtype, B, Hq, Hkv, D, P, k,
        seq_lens=torch.tensor(lens, dtype=torch.int32), page_table=torch.from_numpy(table),
        k_pool=_to(K, dtype), v_pool=_to(V, dtype), q=_to(q, dtype),
        extra={"page_fill": torch.from_numpy(page_fill), "page_in_doc": torch.from_numpy(page_in_doc),
               "doc_of_page": torch.from_numpy(doc_of_page), "doc_start": torch.from_numpy(doc_start),
               "doc_lens": list(doc_lens), "order": order, "theta": theta},
    )



# Batches of the 32K and 128K decode shapes, for the bandwidth-bound regime of the attention:
# name -> (batch, context tokens, token budget).
BATCHED = {
    "llama8b_32k_batch32": (32, 32768, 2048),
    "qwen4b_128k_batch16": (16, 131072, 4096),
}


def batched_device(name: str, device, seed: int = 1006) -> Workload:
    """B sequences of the 32K or 128K decode shape (``BATCHED``), every one at the full context:
    32 / 8 heads, D 128, bf16, P 32, k = budget / P. q, V ~ N(0,1); K ~ N(0,1) with 4 outlier
    channels per KV head scaled by 8 (the 32K recipe; no needles). One random permutation of the
    pool's pages is laid out over all (sequence, logical page) pairs in order.

    Drawn on ``device`` from ``torch.Generator(device)`` seeded with ``seed``, in the order q, page
    permutation, outlier channels, then K and V in chunks of 2048 pages (fp32 draws rounded to
    bf16); the tensors stay on the device.
    """
    B, context, budget = BATCHED[name]
    Hq, Hkv, D, P = 32, 8, 128, 32
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    q = torch.randn((B, Hq, D), generator=g, device=dev).to(torch.bfloat16)
    npg = context // P
    Npp = B * npg
    perm = torch.randperm(Npp, generator=g, device=dev).to(torch.int32)
    chans = torch.stack([torch.randperm(D, generator=g, device=dev)[:4] for _ in range(Hkv)])
    k_pool = torch.empty((Npp, Hkv, P, D), dtype=torch.bfloat16, device=dev)
    v_pool = torch.empty((Npp, Hkv, P, D), dtype=torch.bfloat16, device=dev)
    step = 2048
    for p0 in range(0, Npp, step):
        n = min(step, Npp - p0)
        kc = torch.randn((n, Hkv, P, D), generator=g, device=dev)
        for j in range(Hkv):
            kc[:, j, :, chans[j]] *= 8.0
        k_pool[p0:p0 + n] = kc.to(torch.bfloat16)
        v_pool[p0:p0 + n] = torch.randn((n, Hkv, P, D), generator=g, device=dev).to(torch.bfloat16)
        del kc
    return Workload(
        name, "bf16", B, Hq, Hkv, D, P, budget // P,
        seq_lens=torch.full((B,), context, dtype=torch.int32, device=dev),
        page_table=perm.reshape(B, npg).contiguous(),
        k_pool=k_pool, v_pool=v_pool, q=q,
        extra={"outlier_channels": chans.cpu().tolist(), "device": True},
    )

WORKLOADS = {
    "tiny_fp32": tiny_fp32,
    "llama8b_32k": llama8b_32k,
    "ragged_batch": ragged_batch,
    "qwen4b_128k": qwen4b_128k,
    "speculative_rope": speculative_rope,
    "composed": composed,
}


def make(name: str, seed: Optional[int] = None) -> Workload:
    fn = WORKLOADS[name]
    return fn() if seed is None else fn(seed=seed)
