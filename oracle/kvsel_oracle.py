"""CPU oracle of the query-aware sparse-page decode path — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline`` leg may import
or call this module. It shares no code with the HIP library: it imports neither the library nor
its binding, and reads nothing but the input arrays handed to it.

Plain, slow, obviously-correct NumPy in float64, one function per step of the path, in the order
the pages describe it. Sources (cited by page title and section):

* [FreeKV] "FreeKV: Boosting KV Cache Retrieval for Efficient LLM Inference" (Korean summary),
  technical summary: section 1 (Problem: keep the whole cache, use only the needed part each
  step), section 2.1 (Algorithm: query-aware choice of KV pages per KV head, speculative reuse of
  the previous step's pages, correction when the group-mean query similarity C_i is below tau).
* [KV-Cache wiki] "Key-Value (KV) Cache" wiki page: "Synthesized Content" (prefill stores K/V,
  decode appends one token and reads the rest; decode speed is set by memory bandwidth),
  "Contradictions & Updates" (PagedAttention pages), "Graph" (grouped-query attention).
* [KV Packet] "[Paper review] KV Packet: Recomputation-Free Context-Independent KV Caching for
  LLMs", section 1 (RoPE re-aligns precomputed KV states to new positions).

Readings taken where the pages are silent (each restated at its function):

* R1  The page score is the channel-wise min/max upper bound sum_d max(q_d*lo_d, q_d*hi_d) of
      q.k over the page's keys; the pages only say pages are chosen with the current query.
* R2  A KV head's score sums that bound over the G query heads of its group.
* R3  Scores: exact products, exactly rounded sum (math.fsum), one round-to-nearest-even to fp32.
* R4  Top-k: larger score first, ties to the lower logical page index; output in ascending page
      order, padded with -1; all pages when a sequence has no more than k.
* R5  Only the valid slots of a partly filled last page enter its summary and the attention.
* R6  Query head h reads KV head h // G.
* R7  Softmax scale is the fp32 value handed in (1/sqrt(D) rounded to fp32 by the caller).
* R8  Correction: C = mean over the group's heads of cos(q_t, q_{t-1}) in fp64; the fresh
      selection is used when this is the first step or C < tau (strict), else the previous one.
* R9  Rotary convention: rotate-half pairs (i, i + D/2), inverse frequency theta^(-2i/D); the
      cos/sin table is fp64 libm values rounded to fp32; the rotation itself is fp32 with every
      product and sum rounded on its own (no fused multiply-add), then rounded to the cache dtype.
* R12 A quantized cache stores OCP FP8 E4M3 codes, rounded to nearest (ties to even mantissa),
      saturating at 448.
* R13 One fp32 scale per (physical page, KV head) tile of K and of V: amax / 448; a code stands
      for decode(code) * scale, and attention runs over those values.
* R14 Summaries of an fp8 page are bf16, rounded outward (lo down, hi up) from the extremes of
      the dequantized keys, so the page score stays an upper bound.
* R15 Composition ([KV Packet] sections 1 and 3: independently cached documents reused at new
      positions without recomputation): a sequence may chain the pages of several documents in
      any order; a page may hold fewer valid slots than P (a document's last page), given per
      physical page as page_fill; positions come from the rotary page rows.
"""
from __future__ import annotations

import math
from typing import Tuple

import numpy as np
import torch

__all__ = [
    "as_f64",
    "n_pages",
    "valid_slots",
    "page_summaries",
    "append_tokens",
    "page_scores",
    "top_pages",
    "selection_margin_ulps",
    "query_similarity",
    "speculative_choice",
    "sparse_decode_attention",
    "dense_decode_attention",
    "gather_tokens",
    "rope_table",
    "rope_rotate",
    "round_to_dtype",
    "decode_step",
    "FP8_E4M3_MAX",
    "fp8_e4m3_decode",
    "fp8_e4m3_encode",
    "quantize_pages",
    "dequantize_pages",
    "bf16_round_down",
    "bf16_round_up",
    "page_summaries_fp8",
]


# ----------------------------------------------------------------------------------------------
# helpers (input widening only)
# ----------------------------------------------------------------------------------------------

def as_f64(x) -> np.ndarray:
    """Exact widening of a CPU torch tensor (fp32 / bf16) or array to float64 NumPy."""
    if isinstance(x, torch.Tensor):
        return x.detach().cpu().to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _ints(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        return x.detach().cpu().numpy().astype(np.int64)
    return np.asarray(x, dtype=np.int64)


def n_pages(seq_len: int, page_size: int) -> int:
    """Number of logical pages holding ``seq_len`` tokens (paged cache, [KV-Cache wiki])."""
    return -(-int(seq_len) // int(page_size))


def valid_slots(seq_len: int, n: int, page_size: int, phys_page: int, page_fill=None) -> int:
    """Valid slots of logical page n (physical page ``phys_page``) of a sequence of ``seq_len``
    slots: reading R5 (a partial last page) and, with ``page_fill``, reading R15 (a page of a
    composed sequence may end early: slot s is valid only below page_fill[phys_page])."""
    v = min(int(page_size), int(seq_len) - int(n) * int(page_size))
    if page_fill is not None:
        v = min(v, int(_ints(page_fill)[phys_page]))
    return v


def round_to_dtype(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 values to the cache dtype ("f32" or "bf16", round-to-nearest-even) and return
    them widened back to fp32 NumPy. Uses torch's conversion as a library primitive."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "f32":
        return x32.copy()
    return torch.from_numpy(x32).to(torch.bfloat16).to(torch.float32).numpy()


# ----------------------------------------------------------------------------------------------
# a1: per-page key summaries
# ----------------------------------------------------------------------------------------------

def page_summaries(k_pool, page_table, seq_lens, page_size: int, page_fill=None) -> np.ndarray:
    """Channel-wise min and max of the keys of every referenced page, per KV head.

    [FreeKV] section 2.1 chooses whole KV pages with the query; the pages do not say what a page
    keeps about its keys. Reading R1/R5: keep lo = min and hi = max over the page's valid tokens,
    for each KV head and channel (valid slots per valid_slots, with ``page_fill`` if given).

    Returns ``summ[Npp][Hkv][2][D]`` (index 0 = lo, 1 = hi) in float64; pages no sequence
    references stay NaN.
    """
    K = as_f64(k_pool)
    table = _ints(page_table)
    lens = _ints(seq_lens)
    Npp, Hkv, P, D = K.shape
    assert P == page_size
    summ = np.full((Npp, Hkv, 2, D), np.nan)
    for b in range(len(lens)):
        L = int(lens[b])
        for n in range(n_pages(L, P)):
            p = int(table[b, n])
            valid = valid_slots(L, n, P, p, page_fill)
            assert valid >= 1, "a page holds at least one valid slot"
            toks = K[p, :, :valid, :]  # [Hkv][valid][D]
            summ[p, :, 0, :] = toks.min(axis=1)
            summ[p, :, 1, :] = toks.max(axis=1)
    return summ


def append_tokens(k_pool, v_pool, page_table, seq_lens, k_new, v_new, page_size: int):
    """One decode step's append of a token's key and value to every sequence.

    [KV-Cache wiki] "Synthesized Content": a decode step stores the new token's key and value and
    keeps every earlier one. In the paged layout ("Contradictions & Updates", PagedAttention) the
    token at position L = seq_lens[b] lives in slot L % P of logical page L // P, i.e. physical
    page page_table[b][L // P] (reading: the caller's page allocator has set that table entry
    when the token opens a new page). A sequence whose table has no room (L == width * P) is left
    unchanged and reported.

    k_new, v_new: ``[B][Hkv][D]``. Pools in the oracle layout ``[Npp][Hkv][P][D]`` (both K and V).
    Returns (k_pool, v_pool, seq_lens, rejected) as new arrays; ``rejected[b]`` is True where
    nothing was written.
    """
    K = np.array(k_pool, copy=True)
    V = np.array(v_pool, copy=True)
    table = _ints(page_table)
    lens = _ints(seq_lens).copy()
    kn, vn = np.asarray(k_new), np.asarray(v_new)
    width = table.shape[1]
    rejected = np.zeros(len(lens), dtype=bool)
    for b in range(len(lens)):
        L = int(lens[b])
        if L < 0 or L >= width * page_size:
            rejected[b] = True
            continue
        p = int(table[b, L // page_size])
        K[p, :, L % page_size, :] = kn[b]
        V[p, :, L % page_size, :] = vn[b]
        lens[b] = L + 1
    return K, V, lens, rejected


# ----------------------------------------------------------------------------------------------
# a2: query-aware page scores
# ----------------------------------------------------------------------------------------------

def page_scores(q, summ, page_table, seq_lens, page_size: int) -> np.ndarray:
    """Score of every logical page of every (sequence, KV head) for the current query.

    [FreeKV] section 2.1: the pages to use are chosen per KV head from the current query.
    Readings R1-R3: for each query head g of KV head j's group and channel d, take the larger of
    q_d*lo_d and q_d*hi_d (the largest q_d*k_d any key of the page can give), and sum over d and
    over the G heads. Every product of two bf16 (or two fp32) values is exact in fp64; the sum is
    rounded once (math.fsum) and then to fp32.

    Returns float32 ``scores[B][Hkv][max_pages]``; slots past a sequence's last page are NaN.
    """
    Q = as_f64(q)
    S = np.asarray(summ, dtype=np.float64)
    table = _ints(page_table)
    lens = _ints(seq_lens)
    B, Hq, D = Q.shape
    Hkv = S.shape[1]
    G = Hq // Hkv
    scores = np.full((B, Hkv, table.shape[1]), np.nan, dtype=np.float32)
    for b in range(B):
        N = n_pages(lens[b], page_size)
        pages = table[b, :N]
        for j in range(Hkv):
            qg = Q[b, j * G:(j + 1) * G, :]  # [G][D]
            lo = S[pages, j, 0, :]  # [N][D]
            hi = S[pages, j, 1, :]
            best = np.maximum(qg[None, :, :] * lo[:, None, :], qg[None, :, :] * hi[:, None, :])
            for n in range(N):
                scores[b, j, n] = np.float32(math.fsum(best[n].ravel()))
    return scores


# ----------------------------------------------------------------------------------------------
# a3: top-k page selection
# ----------------------------------------------------------------------------------------------

def top_pages(scores, seq_lens, page_size: int, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """The k best logical pages of every (sequence, KV head).

    [FreeKV] section 2.1 selects a subset of KV pages per KV head. Reading R4: order by score
    (larger first), ties to the lower page index (np.lexsort), keep the first min(k, N), and list
    them in ascending page order padded with -1.

    Returns ``sel_idx[B][Hkv][k]`` int32 and ``sel_cnt[B][Hkv]`` int32.
    """
    sc = np.asarray(scores)
    lens = _ints(seq_lens)
    B, Hkv, _ = sc.shape
    sel = np.full((B, Hkv, k), -1, dtype=np.int32)
    cnt = np.zeros((B, Hkv), dtype=np.int32)
    for b in range(B):
        N = n_pages(lens[b], page_size)
        idx = np.arange(N)
        for j in range(Hkv):
            s = sc[b, j, :N].astype(np.float64)
            order = np.lexsort((idx, -s))
            take = np.sort(order[:min(k, N)])
            sel[b, j, :take.size] = take
            cnt[b, j] = take.size
    return sel, cnt


def _orderable(x: np.ndarray) -> np.ndarray:
    """fp32 -> int64 whose integer order is the float order (+0 and -0 map to the same value)."""
    x = np.where(np.asarray(x, dtype=np.float32) == 0, np.float32(0), x).astype(np.float32)
    u = x.view(np.int32).astype(np.int64)
    return np.where(u < 0, -(u & 0x7FFFFFFF), u)


def selection_margin_ulps(scores, seq_lens, page_size: int, k: int) -> np.ndarray:
    """Distance in fp32 ulps between the k-th and (k+1)-th best score of every (b, j).

    A diagnostic for the parity tests: a margin of 0 is an exact tie (decided by page index,
    identical on both sides when the scores are bit-identical); a margin of 1 would be the only
    place where a 1-ulp difference in accumulation order could change the selected set. Lists
    with no more than k pages get a large sentinel.
    """
    sc = np.asarray(scores)
    lens = _ints(seq_lens)
    B, Hkv, _ = sc.shape
    out = np.full((B, Hkv), 1 << 40, dtype=np.int64)
    for b in range(B):
        N = n_pages(lens[b], page_size)
        if N <= k:
            continue
        for j in range(Hkv):
            o = np.sort(_orderable(sc[b, j, :N]))[::-1]
            out[b, j] = o[k - 1] - o[k]
    return out


# ----------------------------------------------------------------------------------------------
# a4: speculative reuse and correction
# ----------------------------------------------------------------------------------------------

def query_similarity(q_t, q_prev, num_kv_heads: int) -> np.ndarray:
    """C[b][j]: mean over the query heads of KV head j's group of cos(q_t, q_{t-1}).

    [FreeKV] section 2.1: adjacent steps' queries are highly similar; the correction decision
    uses the similarity averaged over the heads of a GQA group so the group stays consistent.
    Reading R8: fp64 cosines of the (bf16) query values.
    """
    A = as_f64(q_t)
    Bq = as_f64(q_prev)
    B, Hq, _ = A.shape
    G = Hq // num_kv_heads
    C = np.zeros((B, num_kv_heads))
    for b in range(B):
        for j in range(num_kv_heads):
            cos = []
            for h in range(j * G, (j + 1) * G):
                dot = math.fsum(A[b, h] * Bq[b, h])
                na = math.sqrt(math.fsum(A[b, h] * A[b, h]))
                nb = math.sqrt(math.fsum(Bq[b, h] * Bq[b, h]))
                cos.append(dot / (na * nb))
            C[b, j] = math.fsum(cos) / G
    return C


def speculative_choice(fresh_idx, fresh_cnt, prev_idx, prev_cnt, C, tau: float,
                       first_step: bool):
    """Which page list each (sequence, KV head) attends over at this step.

    [FreeKV] section 2.1: attention at step i reuses the pages selected at step i-1; when the
    group similarity C_i falls below tau, that KV head is corrected with a fresh selection for
    the current query. Reading R8: step 0 always uses the fresh selection; otherwise fresh iff
    C < tau (strict).

    Returns (used_idx, used_cnt, corrected[B][Hkv] as uint8).
    """
    C = np.asarray(C, dtype=np.float64)
    corrected = np.ones(C.shape, dtype=bool) if first_step else (C < tau)
    used_idx = np.where(corrected[:, :, None], fresh_idx, prev_idx).astype(np.int32)
    used_cnt = np.where(corrected, fresh_cnt, prev_cnt).astype(np.int32)
    return used_idx, used_cnt, corrected.astype(np.uint8)


# ----------------------------------------------------------------------------------------------
# a5 + a6: attention over the selected pages
# ----------------------------------------------------------------------------------------------

def gather_tokens(pool, page_table, seq_len: int, b: int, j: int, pages, page_size: int,
                  page_fill=None):
    """Rows [T][D] (float64) of KV head j for the valid tokens of logical pages ``pages`` of
    sequence b, in the order given (reading R5: a partial last page contributes its valid
    slots only; R15: so does a page that ``page_fill`` ends early)."""
    X = pool if isinstance(pool, np.ndarray) and pool.dtype == np.float64 else as_f64(pool)
    table = _ints(page_table)
    rows = []
    for n in pages:
        n = int(n)
        p = int(table[b, n])
        valid = valid_slots(seq_len, n, page_size, p, page_fill)
        rows.append(X[p, j, :valid, :])
    if not rows:
        return np.zeros((0, X.shape[-1]))
    return np.concatenate(rows, axis=0)


def _softmax_attend(qv: np.ndarray, Kr: np.ndarray, Vr: np.ndarray, scale: float):
    z = scale * (Kr @ qv)
    m = z.max()
    w = np.exp(z - m)
    l = w.sum()
    return (w @ Vr) / l, m + math.log(l)


def sparse_decode_attention(q, k_pool, v_pool, page_table, seq_lens, sel_idx, sel_cnt,
                            page_size: int, scale: float, page_fill=None):
    """Decode attention of every query head over the tokens of its KV head's chosen pages.

    [FreeKV] section 2.1: attention runs over the retrieved pages only; [KV-Cache wiki]: one
    decode query attends over cached keys/values; GQA maps query head h to KV head h // G
    (reading R6). In fp64: z = scale * q.k, weights softmax(z), o = sum of weights * v,
    lse = max z + ln(sum exp(z - max z)). A (sequence, head) with no selected token returns
    o = 0 and lse = -inf.

    Returns (out[B][Hq][D], lse[B][Hq]) in float64.
    """
    Q = as_f64(q)
    K = as_f64(k_pool)
    V = as_f64(v_pool)
    lens = _ints(seq_lens)
    sel = _ints(sel_idx)
    cnt = _ints(sel_cnt)
    B, Hq, D = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        for j in range(Hkv):
            pages = sel[b, j, :cnt[b, j]]
            Kr = gather_tokens(K, page_table, lens[b], b, j, pages, page_size, page_fill)
            Vr = gather_tokens(V, page_table, lens[b], b, j, pages, page_size, page_fill)
            if Kr.shape[0] == 0:
                continue
            for h in range(j * G, (j + 1) * G):
                out[b, h], lse[b, h] = _softmax_attend(Q[b, h], Kr, Vr, scale)
    return out, lse


def dense_decode_attention(q, keys, values, scale: float):
    """Plain decode attention over all tokens: q[B][Hq][D], keys/values[B][Hkv][T][D] (fp64)."""
    Q = as_f64(q)
    K = as_f64(keys)
    V = as_f64(values)
    B, Hq, D = Q.shape
    G = Hq // K.shape[1]
    out = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    for b in range(B):
        for h in range(Hq):
            out[b, h], lse[b, h] = _softmax_attend(Q[b, h], K[b, h // G], V[b, h // G], scale)
    return out, lse


# ----------------------------------------------------------------------------------------------
# a7: rotary re-positioning of precomputed blocks
# ----------------------------------------------------------------------------------------------

def rope_table(theta: float, head_dim: int, first_position: int, n_rows: int):
    """cos/sin of position * theta^(-2i/D) for positions first_position .. + n_rows - 1.

    [KV Packet] section 1: RoPE encodes position by rotation, and is the tool that re-aligns
    precomputed KV states to new positions. Reading R9: fp64 libm values (Python's math module),
    rounded to fp32. Returns (cos, sin) float32 [n_rows][D/2].
    """
    half = head_dim // 2
    inv = np.array([math.pow(theta, -(2.0 * i) / head_dim) for i in range(half)])
    pos = np.arange(first_position, first_position + n_rows, dtype=np.float64)
    ang = (pos[:, None] * inv[None, :]).ravel()
    c = np.fromiter(map(math.cos, ang), dtype=np.float64, count=ang.size)
    s = np.fromiter(map(math.sin, ang), dtype=np.float64, count=ang.size)
    return (c.astype(np.float32).reshape(n_rows, half), s.astype(np.float32).reshape(n_rows, half))


def rope_rotate(k_pool, cos, sin, page_row, row_step: int, dtype: str) -> np.ndarray:
    """Rotate the keys of every page whose ``page_row`` entry is >= 0.

    [KV Packet] section 1 (RoPE re-positioning of precomputed KV). Token slot s of physical page
    p uses table row ``page_row[p] + row_step * s`` (row_step 1 encodes per-token positions,
    row_step 0 shifts a whole page by one offset). Reading R9: with c, s from the table, pair
    (x_i, x_{i+D/2}) becomes (x_i*c - x_{i+D/2}*s, x_{i+D/2}*c + x_i*s), each product and each
    sum rounded to fp32 on its own, then the result rounded to the cache dtype. Pages with
    ``page_row`` < 0 are copied unchanged.

    Returns the rotated pool as float32 NumPy (values exactly representable in ``dtype``).
    """
    X = as_f64(k_pool).astype(np.float32)
    cos = np.asarray(cos, dtype=np.float32)
    sin = np.asarray(sin, dtype=np.float32)
    rows_of = _ints(page_row)
    Npp, Hkv, P, D = X.shape
    half = D // 2
    out = X.copy()
    for p in range(Npp):
        r0 = int(rows_of[p])
        if r0 < 0:
            continue
        rows = r0 + row_step * np.arange(P)
        c = cos[rows][None, :, :]  # [1][P][half]
        s = sin[rows][None, :, :]
        x1 = X[p, :, :, :half]
        x2 = X[p, :, :, half:]
        y1 = np.subtract(np.multiply(x1, c, dtype=np.float32), np.multiply(x2, s, dtype=np.float32),
                         dtype=np.float32)
        y2 = np.add(np.multiply(x2, c, dtype=np.float32), np.multiply(x1, s, dtype=np.float32),
                    dtype=np.float32)
        out[p] = round_to_dtype(np.concatenate([y1, y2], axis=-1), dtype)
    return out


# ----------------------------------------------------------------------------------------------
# fp8 pages: a quantized cache ([KV-Cache wiki] "Contradictions & Updates": a quantized cache
# holds longer contexts at a small accuracy cost; [KV Packet] section 3: compatible with KV
# compression). The pages fix no format; readings R12-R14 below.
# ----------------------------------------------------------------------------------------------

FP8_E4M3_MAX = 448.0


def fp8_e4m3_decode(codes) -> np.ndarray:
    """Values of 8-bit codes in the E4M3 format of the Open Compute Project 8-bit floating point
    specification (OFP8): a sign bit, 4 exponent bits with bias 7 and 3 mantissa bits; exponent
    field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; there are no infinities, and the largest
    finite magnitude is 1.75 * 2^8 = 448. Returns float64 (every value is exact)."""
    c = _ints(codes) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (c & 0x7 == 7), np.nan, mag)
    return sign * mag


def fp8_e4m3_encode(x) -> np.ndarray:
    """Reading R12: round each value to the nearest E4M3 value, ties to the code with an even
    mantissa (last bit 0), magnitudes beyond 448 saturate to 448; the sign bit is kept (so -0.0
    is 0x80). Plainly: the nearest of the 127 non-negative finite values, by search. Returns
    uint8 codes."""
    x = np.asarray(x, dtype=np.float64)
    assert not np.isnan(x).any()
    table = fp8_e4m3_decode(np.arange(127))  # codes 0x00..0x7E, increasing values
    a = np.minimum(np.abs(x), FP8_E4M3_MAX)
    hi = np.searchsorted(table, a, side="left")  # first value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - table[lo]
    d_hi = table[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(table[hi] == a, hi, np.where(pick_hi, hi, lo))
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def quantize_pages(pool) -> Tuple[np.ndarray, np.ndarray]:
    """Reading R13: one fp32 scale per (physical page, KV head) tile, amax / 448 (fp32 division;
    1 for an all-zero tile), and every element coded as encode(fp32(x / scale)) with x the cache
    value (bf16 and fp32 values are exact in fp32; the division is fp32, correctly rounded).
    The layout of a tile's elements does not matter (amax and the coding are per element).

    Returns (codes uint8, same shape as pool; scales float32 [Npp][Hkv])."""
    X = as_f64(pool).astype(np.float32)  # exact: the cache values are fp32 or bf16
    amax = np.abs(X).reshape(X.shape[0], X.shape[1], -1).max(axis=2)
    scale = np.where(amax > 0, amax / np.float32(FP8_E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = (X / scale[:, :, None, None]).astype(np.float32)
    return fp8_e4m3_encode(y), scale


def dequantize_pages(codes, scales) -> np.ndarray:
    """The value each code stands for: decode(code) * its tile's scale, exact in float64."""
    return fp8_e4m3_decode(codes) * np.asarray(scales, dtype=np.float64)[:, :, None, None]


def bf16_round_down(x) -> np.ndarray:
    """Largest bf16 value <= x (8 significant bits), for x zero or of magnitude >= 2^-126."""
    return _bf16_directed(x, np.floor)


def bf16_round_up(x) -> np.ndarray:
    """Smallest bf16 value >= x (8 significant bits), for x zero or of magnitude >= 2^-126."""
    return _bf16_directed(x, np.ceil)


def _bf16_directed(x, step) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    nz = x[x != 0]
    assert (np.abs(nz) >= 2.0 ** -126).all(), "bf16 subnormal range"
    m, e = np.frexp(x)  # x = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(step(m * 256.0), e - 8)  # m * 2^8 has 8 integer bits; scaling is exact


def page_summaries_fp8(k_codes, k_scale, page_table, seq_lens, page_size: int,
                       page_fill=None) -> np.ndarray:
    """Reading R14: the summary of an fp8 page is bf16, the outward rounding of the extremes of
    its dequantized keys: lo = the largest bf16 <= min, hi = the smallest bf16 >= max (products of
    a code's value and the fp32 scale are exact in float64). The outward rounding keeps every
    page score an upper bound of q.k over the page's keys. Valid slots only, as page_summaries.

    Returns summ[Npp][Hkv][2][D] float64 (bf16 values); unreferenced pages stay NaN."""
    summ = page_summaries(dequantize_pages(k_codes, k_scale), page_table, seq_lens, page_size,
                          page_fill)
    out = np.full_like(summ, np.nan)
    done = ~np.isnan(summ[:, 0, 0, 0])
    out[done, :, 0, :] = bf16_round_down(summ[done, :, 0, :])
    out[done, :, 1, :] = bf16_round_up(summ[done, :, 1, :])
    return out


# ----------------------------------------------------------------------------------------------
# one whole decode step (used by the benchmark's CPU baseline)
# ----------------------------------------------------------------------------------------------

def decode_step(q, summ, k_pool, v_pool, page_table, seq_lens, page_size: int, k: int,
                scale: float):
    """Score, select and attend for one decode step (a2 + a3 + a5/a6), given the summaries."""
    sc = page_scores(q, summ, page_table, seq_lens, page_size)
    sel, cnt = top_pages(sc, seq_lens, page_size, k)
    out, lse = sparse_decode_attention(q, k_pool, v_pool, page_table, seq_lens, sel, cnt,
                                       page_size, scale)
    return sel, cnt, out, lse
