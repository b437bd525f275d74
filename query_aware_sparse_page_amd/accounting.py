"""Byte accounting of the decode path (what each step must move through HBM).

The KV-cache size formula follows the KVzap blog post's introduction (Llama 65B at 128,000 tokens
needs about 335 GB of KV cache): 2 (K and V) x layers x KV width x bytes x tokens. The decode
step is memory-bandwidth bound ("Key-Value (KV) Cache" wiki page, bottleneck entry), so the
roofline of every kernel here is HBM bytes.
"""
from __future__ import annotations

from typing import Sequence


def kv_cache_bytes(num_layers: int, kv_width: int, tokens: int, bytes_per_elem: int) -> int:
    """Dense K+V bytes of a cache: 2 * layers * (KV heads * head dim) * tokens * element bytes."""
    return 2 * num_layers * kv_width * tokens * bytes_per_elem


def _tokens_of_pages(seq_len: int, page_size: int, pages: Sequence[int]) -> int:
    t = 0
    for n in pages:
        if n < 0:
            continue
        t += max(0, min(page_size, seq_len - n * page_size))
    return t


def selected_kv_bytes(seq_lens, sel_idx, sel_cnt, num_kv_heads: int, page_size: int,
                      head_dim: int, bytes_per_elem: int) -> int:
    """K+V bytes the sparse attention must read: valid tokens of every selected page.

    ``sel_idx[b][j][:sel_cnt[b][j]]`` lists the logical pages of sequence b, KV head j.
    """
    total = 0
    for b, L in enumerate(seq_lens):
        for j in range(num_kv_heads):
            c = int(sel_cnt[b][j])
            total += _tokens_of_pages(int(L), page_size, [int(x) for x in sel_idx[b][j][:c]])
    return 2 * total * head_dim * bytes_per_elem


def summary_bytes(seq_lens, num_kv_heads: int, page_size: int, head_dim: int,
                  bytes_per_elem: int) -> int:
    """Bytes of page summaries (lo and hi rows) the scoring reads for one decode step."""
    pages = sum(-(-int(L) // page_size) for L in seq_lens)
    return pages * num_kv_heads * 2 * head_dim * bytes_per_elem
