"""The live page bound (the descriptor's max_seq_len) on page tables allocated far wider than the
live lengths: launches follow the bound, and every entry point still gives the oracle's results
(the table entries past each sequence's pages hold junk, which must never be followed). A length
past the bound is selected over as its first max_seq_len tokens, its last live page counted
whole, and kvsel_check_inputs reports it."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as W
from gpu_common import (assert_attention_close, assert_selection_equal, assert_summaries_equal,
                        kv_of, oracle_path, say, scale_of)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from query_aware_sparse_page_amd import kvsel as K
    K.lib()  # raises if libkvsel.so is missing: no fallback
    return K


def widened(w, width, seed):
    """The same cache with table rows `width` pages wide; every entry past a sequence's pages is
    junk (far outside the pool, either sign)."""
    rng = np.random.default_rng(seed)
    table = rng.integers(-(1 << 30), 1 << 30, size=(w.B, width)).astype(np.int32)
    for b in range(w.B):
        n = w.n_pages(b)
        table[b, :n] = w.page_table[b, :n].numpy()
    return dataclasses.replace(w, page_table=torch.from_numpy(table))


CASES = [
    # 1500 live pages in a 4096-page table: the 1025..2048-page forms of every launch
    dict(seed=801, B=3, Hq=32, Hkv=8, D=128, P=32, k=64, lens=[1500 * 32 - 7, 300 * 32 + 1, 5],
         dtype="bf16", width=4096, bound="max"),
    # a bound beyond the table is capped at the table width
    dict(seed=802, B=2, Hq=8, Hkv=4, D=64, P=16, k=12, lens=[100 * 16 + 3, 37], dtype="f32",
         width=1500, bound=10 ** 9),
    # G = 8, P = 16: 700 live pages of an 8192-page table
    dict(seed=803, B=2, Hq=16, Hkv=2, D=128, P=16, k=40, lens=[700 * 16 + 9, 16 * 10],
         dtype="bf16", width=8192, bound="max"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c['seed']}")
def test_live_bound_matches_oracle(K, case):
    c = dict(case)
    width, bound = c.pop("width"), c.pop("bound")
    w = widened(W.custom(**c), width, c["seed"] + 1)
    msl = max(c["lens"]) if bound == "max" else bound
    say(f"live bound {case['seed']}: lens {c['lens']}, table {width}, max_seq_len {msl}")
    kv = kv_of(K, w)
    kv.max_seq_len = msl
    q = w.q.cuda()
    ref = oracle_path(w, scale_of(w.D))
    summ = K.build_summaries(kv)
    torch.cuda.synchronize()
    assert_summaries_equal(summ, ref["summ"], w)
    sel, cnt = K.score_topk(kv, summ, q, w.k, refresh_tail=True)
    out, lse = K.sparse_decode_attn(kv, q, sel, cnt, w.k)
    torch.cuda.synchronize()
    assert_selection_equal(sel, cnt, ref["sel"], ref["cnt"], ref["fp32"])
    assert_attention_close(out, lse, ref["out"], ref["lse"], w.dtype)
    fs, fc, fo, fl = K.select_attend(kv, summ, q, w.k, refresh_tail=True)
    torch.cuda.synchronize()
    assert_selection_equal(fs, fc, ref["sel"], ref["cnt"], ref["fp32"])
    assert_attention_close(fo, fl, ref["out"], ref["lse"], w.dtype)
    # speculative step: the first step takes the fresh selection; the second reuses it where the
    # queries agree and must equal the serial calls bit for bit
    zi = torch.zeros((w.B, w.Hkv, w.k), dtype=torch.int32, device="cuda")
    zc = torch.zeros((w.B, w.Hkv), dtype=torch.int32, device="cuda")
    s1 = K.speculative_step(kv, summ, q, w.k, K.Reuse(q, zi, zc, 0.8, first_step=True))
    torch.cuda.synchronize()
    assert_selection_equal(s1[0], s1[1], ref["sel"], ref["cnt"], ref["fp32"])
    assert_attention_close(s1[6], s1[7], ref["out"], ref["lse"], w.dtype)
    gen = torch.Generator().manual_seed(c["seed"] + 2)
    q2 = (w.q.float() + 0.3 * torch.randn(w.q.shape, generator=gen)).to(w.q.dtype).cuda()
    reuse = K.Reuse(q, s1[0].clone(), s1[1].clone(), 0.95)
    s2 = K.speculative_step(kv, summ, q2, w.k, reuse)
    r2 = K.score_topk(kv, summ, q2, w.k, reuse=reuse)
    o2, l2 = K.sparse_decode_attn(kv, q2, r2[2], r2[3], w.k,
                                  pages_per_split=K.step_pages_per_split(kv, w.k))
    torch.cuda.synchronize()
    for x, y, name in zip(s2, tuple(r2) + (o2, l2),
                          ("sel", "cnt", "used", "ucnt", "corrected", "similarity", "out", "lse")):
        assert torch.equal(x, y), f"second step: {name} differs"
    flags = K.check_inputs(kv, sel, cnt)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0


def test_length_past_the_bound(K):
    """A sequence longer than max_seq_len: selection over its first 30 pages (the 30th counted
    whole), attention over the selected pages; the check reports the length."""
    P, live = 32, 30
    lens = [40 * P + 3, 10 * P, 30 * P]
    c = dict(seed=811, B=3, Hq=8, Hkv=2, D=128, P=P, k=8, lens=lens, dtype="bf16")
    w = widened(W.custom(**c), 64, 812)
    say(f"length past the bound: lens {lens}, max_seq_len {live * P}")
    kv = kv_of(K, w)
    kv.max_seq_len = live * P
    cut = dataclasses.replace(w, seq_lens=torch.tensor([min(L, live * P) for L in lens],
                                                       dtype=torch.int32))
    ref = oracle_path(cut, scale_of(w.D))
    q = w.q.cuda()
    summ = K.build_summaries(kv)
    sel, cnt, out, lse = K.select_attend(kv, summ, q, w.k, refresh_tail=True)
    torch.cuda.synchronize()
    assert_summaries_equal(summ, ref["summ"], cut)
    assert_selection_equal(sel, cnt, ref["sel"], ref["cnt"], ref["fp32"])
    assert_attention_close(out, lse, ref["out"], ref["lse"], w.dtype)
    flags = K.check_inputs(kv)
    torch.cuda.synchronize()
    assert int(flags.item()) == 1  # KVSEL_CHECK_SEQ_LEN only


def test_live_bound_fp8(K):
    """fp8 pages with 1500 live pages in a 4096-page table: the fused selection with 8 keys per
    thread and the fp8 co-launch, against the oracle over the dequantized cache."""
    import oracle as O
    c = dict(seed=821, B=2, Hq=32, Hkv=8, D=128, P=32, k=64, lens=[1500 * 32 - 3, 700 * 32 + 9],
             dtype="bf16")
    w = widened(W.custom(**c), 4096, 822)
    say(f"live bound, fp8: lens {c['lens']}, table 4096")
    scale = scale_of(w.D)
    kc, ks = O.quantize_pages(w.k_pool)
    vc, vs = O.quantize_pages(w.v_pool)
    summ_ref = O.page_summaries_fp8(kc, ks, w.page_table, w.seq_lens, w.P)
    sc = O.page_scores(w.q, summ_ref, w.page_table, w.seq_lens, w.P)
    sel_ref, cnt_ref = O.top_pages(sc, w.seq_lens, w.P, w.k)
    out_ref, lse_ref = O.sparse_decode_attention(w.q, O.dequantize_pages(kc, ks),
                                                 O.dequantize_pages(vc, vs), w.page_table,
                                                 w.seq_lens, sel_ref, cnt_ref, w.P, scale)
    kv = kv_of(K, w)
    kv.max_seq_len = max(c["lens"])
    kv8 = K.quantize_pages(kv)
    q = w.q.cuda()
    summ = K.build_summaries(kv8)
    sel, cnt, out, lse = K.select_attend(kv8, summ, q, w.k, refresh_tail=True, scale=scale)
    zi = torch.zeros((w.B, w.Hkv, w.k), dtype=torch.int32, device="cuda")
    zc = torch.zeros((w.B, w.Hkv), dtype=torch.int32, device="cuda")
    spec = K.speculative_step(kv8, summ, q, w.k, K.Reuse(q, zi, zc, 0.8, first_step=True),
                              scale=scale)
    torch.cuda.synchronize()
    assert_summaries_equal(summ, summ_ref, w)
    assert_selection_equal(sel, cnt, sel_ref, cnt_ref)
    assert_attention_close(out, lse, out_ref, lse_ref, "bf16")
    for a, b_, name in ((spec[0], sel, "sel"), (spec[6], out, "out"), (spec[7], lse, "lse")):
        assert torch.equal(a, b_), f"speculative step: {name} differs from kvsel_select_attend"
