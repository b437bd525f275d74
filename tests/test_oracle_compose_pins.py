"""Pins of the oracle's composed-context reading (R15: pages of independently cached documents
chained into one sequence, a page possibly ending early, given by page_fill) against a dense
reference built by hand: the documents' valid tokens concatenated in chain order, attended with
torch's own scaled_dot_product_attention in fp64, and the page summaries by brute-force loops.
Planted mistakes (the fill ignored, or indexed by the logical page) must fail."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W


def small_composed(seed=41):
    return W.composed(seed, doc_lens=(37, 5, 64, 1, 20, 16), P=16, B=2, Hq=4, Hkv=2, D=16, k=3)


def dense_sequence(w, b):
    """Keys and values [Hkv][T][D] of sequence b: each document's tokens, in chain order, read
    straight from the documents' pages (not through valid_slots)."""
    K = w.k_pool.double().numpy()
    V = w.v_pool.double().numpy()
    doc_lens = w.extra["doc_lens"]
    page_in_doc = w.extra["page_in_doc"].numpy()
    doc_of_page = w.extra["doc_of_page"].numpy()
    ks, vs = [], []
    for i in w.extra["order"][b]:
        pages = sorted(np.nonzero(doc_of_page == i)[0], key=lambda p: page_in_doc[p])
        left = doc_lens[i]
        for p in pages:
            take = min(w.P, left)
            ks.append(K[p, :, :take])
            vs.append(V[p, :, :take])
            left -= take
    return np.concatenate(ks, axis=1), np.concatenate(vs, axis=1)


def composition_ok(attend, summaries, w):
    fill = w.extra["page_fill"]
    scale = float(np.float32(1.0 / math.sqrt(w.D)))
    # every page of every sequence selected
    N = max(w.n_pages(b) for b in range(w.B))
    sel = np.full((w.B, w.Hkv, N), -1, dtype=np.int64)
    cnt = np.zeros((w.B, w.Hkv), dtype=np.int64)
    for b in range(w.B):
        sel[b, :, :w.n_pages(b)] = np.arange(w.n_pages(b))
        cnt[b, :] = w.n_pages(b)
    out, lse = attend(w.q, w.k_pool, w.v_pool, w.page_table, w.seq_lens, sel, cnt, w.P, scale, fill)
    for b in range(w.B):
        Kd, Vd = dense_sequence(w, b)
        q = w.q[b].double()[None, :, None, :]
        k = torch.from_numpy(Kd).repeat_interleave(w.G, dim=0)[None]
        v = torch.from_numpy(Vd).repeat_interleave(w.G, dim=0)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)[0, :, 0]
        if not np.allclose(out[b], ref.numpy(), rtol=0, atol=1e-12):
            return False
        z = scale * torch.einsum("hd,htd->ht", w.q[b].double(), k[0])
        if not np.allclose(lse[b], torch.logsumexp(z, dim=-1).numpy(), rtol=0, atol=1e-12):
            return False
    # summaries: brute-force min / max over each page's document tokens
    summ = summaries(w.k_pool, w.page_table, w.seq_lens, w.P, fill)
    K = w.k_pool.double().numpy()
    for p in range(w.num_phys_pages):
        f = int(fill[p])
        for j in range(w.Hkv):
            for d in range(w.D):
                col = [K[p, j, s, d] for s in range(f)]
                if summ[p, j, 0, d] != min(col) or summ[p, j, 1, d] != max(col):
                    return False
    return True


def test_composed_context_equals_dense_documents():
    w = small_composed()
    assert (w.extra["page_fill"] < w.P).any()  # there are holes
    assert composition_ok(O.sparse_decode_attention, O.page_summaries, w)


@pytest.mark.parametrize("mistake", ["fill_ignored", "fill_by_logical_page"])
def test_planted_composition_mistakes_are_caught(mistake):
    w = small_composed()

    def fill_for(table, fill):
        if mistake == "fill_ignored":
            return None
        # fill looked up with the logical page index of sequence 0 instead of the physical page
        f = np.full_like(fill.numpy(), w.P)
        t = table.numpy()[0]
        for n in range(w.n_pages(0)):
            f[n] = int(fill[t[n]])
        return torch.from_numpy(f)

    def attend(q, kp, vp, table, lens, sel, cnt, P, sc, fill):
        return O.sparse_decode_attention(q, kp, vp, table, lens, sel, cnt, P, sc,
                                         fill_for(table, fill))

    def summaries(kp, table, lens, P, fill):
        return O.page_summaries(kp, table, lens, P, fill_for(table, fill))

    assert not composition_ok(attend, summaries, w)


def test_fp8_summaries_respect_the_fill():
    w = small_composed(43)
    kc, ks = O.quantize_pages(w.k_pool)
    fill = w.extra["page_fill"]
    summ = O.page_summaries_fp8(kc, ks, w.page_table, w.seq_lens, w.P, fill)
    deq = O.dequantize_pages(kc, ks)
    for p in range(w.num_phys_pages):
        f = int(fill[p])
        keys = deq[p, :, :f, :]
        assert (summ[p, :, 0, :] <= keys.min(axis=1)).all()
        assert (summ[p, :, 1, :] >= keys.max(axis=1)).all()
        np.testing.assert_array_equal(summ[p, :, 1, :], O.bf16_round_up(keys.max(axis=1)))
