"""Composed contexts (pages of independently cached documents chained in any order, a page
possibly ending early: page_fill) through the C ABI against the oracle: summaries bit for bit,
selection exactly, attention within tolerance; the one-call forms against the separate calls;
the contract check of the fill; and, with the documents pre-encoded at their own positions and
moved to the composed ones by per-page rotary shifts, the fused gather against materialized keys
bit for bit."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_common import (assert_attention_close, assert_selection_equal, assert_summaries_equal,
                        fp32_boundary,
                        kv_of, say, scale_of)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from query_aware_sparse_page_amd import kvsel as K
    K.lib()  # raises if libkvsel.so is missing: no fallback
    return K


def composed_kv(K, w):
    kv = kv_of(K, w)
    kv.page_fill = w.extra["page_fill"].cuda()
    return kv


def oracle_composed(w, scale, fp8=False):
    fill = w.extra["page_fill"]
    if fp8:
        kc, ks = O.quantize_pages(w.k_pool)
        vc, vs = O.quantize_pages(w.v_pool)
        keys, values = O.dequantize_pages(kc, ks), O.dequantize_pages(vc, vs)
        q = w.q.to(torch.bfloat16)
        summ = O.page_summaries_fp8(kc, ks, w.page_table, w.seq_lens, w.P, fill)
    else:
        keys, values, q = w.k_pool, w.v_pool, w.q
        summ = O.page_summaries(w.k_pool, w.page_table, w.seq_lens, w.P, fill)
    sc = O.page_scores(q, summ, w.page_table, w.seq_lens, w.P)
    sel, cnt = O.top_pages(sc, w.seq_lens, w.P, w.k)
    fp32 = None if fp8 else fp32_boundary(w.dtype, sc, w.seq_lens, w.P, w.k)
    out, lse = O.sparse_decode_attention(q, keys, values, w.page_table, w.seq_lens, sel, cnt, w.P,
                                         scale, fill)
    return dict(q=q, summ=summ, sel=sel, cnt=cnt, fp32=fp32, out=out, lse=lse)


CASES = [
    dict(name="bf16-P32-G4-B2", kw=dict(seed=1201, B=2), fp8=False),
    dict(name="f32-P16-D64-G2", kw=dict(seed=1202, doc_lens=(700, 33, 16, 250, 1, 90), P=16, B=2,
                                        Hq=8, Hkv=4, D=64, k=20, dtype="f32"), fp8=False),
    dict(name="bf16-P16-G8-B1", kw=dict(seed=1203, doc_lens=(1000, 17, 333, 5, 64), P=16, B=1,
                                        Hq=16, Hkv=2, D=128, k=24), fp8=False),
    dict(name="fp8-P32-B2", kw=dict(seed=1204, B=2), fp8=True),
    # wider tables: the fused selection's fill variants at 4 keys per thread for fp32 and for bf16
    # with P 16 (356 and 174 pages)
    dict(name="f32-P16-D64-wide", kw=dict(seed=1205, doc_lens=(3000, 517, 1400, 33, 700), P=16,
                                          B=1, Hq=8, Hkv=4, D=64, k=24, dtype="f32"), fp8=False),
    dict(name="bf16-P16-G8-wide", kw=dict(seed=1206, doc_lens=(1500, 17, 900, 333), P=16, B=2,
                                          Hq=16, Hkv=2, D=128, k=24), fp8=False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c["name"])
def test_composed_matches_oracle(K, case):
    w = W.composed(**case["kw"])
    say(f"composed {case['name']}: lens {w.seq_lens.tolist()}, "
        f"{int((w.extra['page_fill'] < w.P).sum())} pages that end early")
    scale = scale_of(w.D)
    ref = oracle_composed(w, scale, case["fp8"])
    kv = composed_kv(K, w)
    if case["fp8"]:
        kv = K.quantize_pages(kv)
    q = ref["q"].cuda()
    summ = K.build_summaries(kv)
    stale = summ.clone()
    for b in range(w.B):  # the tail refresh rebuilds each sequence's last page
        stale[b, :, w.n_pages(b) - 1] = 0
    sel, cnt, out, lse = K.select_attend(kv, stale, q, w.k, refresh_tail=True, scale=scale)
    torch.cuda.synchronize()
    dtype = "bf16" if case["fp8"] else w.dtype
    assert_summaries_equal(summ, ref["summ"], w)
    assert_summaries_equal(stale, ref["summ"], w)
    assert_selection_equal(sel, cnt, ref["sel"], ref["cnt"], ref["fp32"])
    assert_attention_close(out, lse, ref["out"], ref["lse"], dtype)
    s2, c2 = K.score_topk(kv, summ, q, w.k)
    o2, l2 = K.sparse_decode_attn(kv, q, s2, c2, w.k, scale=scale,
                                  pages_per_split=K.step_pages_per_split(kv, w.k))
    zi = torch.zeros((w.B, w.Hkv, w.k), dtype=torch.int32, device="cuda")
    zc = torch.zeros((w.B, w.Hkv), dtype=torch.int32, device="cuda")
    spec = K.speculative_step(kv, summ, q, w.k, K.Reuse(q, zi, zc, 0.8, first_step=True), scale=scale)
    torch.cuda.synchronize()
    for a, b_, name in ((s2, sel, "sel"), (c2, cnt, "cnt"), (o2, out, "out"), (l2, lse, "lse"),
                        (spec[0], sel, "spec sel"), (spec[6], out, "spec out")):
        assert torch.equal(a, b_), f"{name}: separate calls differ from kvsel_select_attend"
    flags = K.check_inputs(kv, sel, cnt)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0


def test_bad_fill_is_reported(K):
    w = W.composed(1211, doc_lens=(40, 7, 33), P=16, Hq=4, Hkv=2, D=64, k=4)
    kv = composed_kv(K, w)
    say("composed: bad fill")
    for bad in (0, w.P + 1):
        kv.page_fill = w.extra["page_fill"].clone().cuda()
        kv.page_fill[int(w.page_table[0, 1])] = bad
        flags = K.check_inputs(kv)
        torch.cuda.synchronize()
        assert int(flags.item()) == K.KVSEL_CHECK_PAGE_FILL


def test_composed_rotary_gather_equals_materialized(K):
    """Documents encoded at their own positions (page rows = the page's index in its document,
    row_step 1) and moved to their composed positions by one shift per page (row_step 0): the
    fused gather gives the summaries, selection and attention of the materialized keys."""
    w = W.composed(1221, B=1)
    say(f"composed rotary gather: {len(w.extra['doc_lens'])} documents, length {int(w.seq_lens[0])}")
    page_in_doc = w.extra["page_in_doc"].numpy()
    doc_of_page = w.extra["doc_of_page"].numpy()
    start = w.extra["doc_start"].numpy()[0]
    n_rows = int(start.max()) + max(w.extra["doc_lens"]) + w.P
    cos, sin = K.rope_table(w.extra["theta"], w.D, 0, n_rows, torch.device("cuda"))
    kv_raw = composed_kv(K, w)
    enc_row = torch.from_numpy((page_in_doc * w.P).astype(np.int32)).cuda()
    enc = K.rope_shift(kv_raw, K.Rope(cos, sin, enc_row, 1))
    kv_enc = K.PagedKV(enc, kv_raw.v_pool, kv_raw.page_table, kv_raw.seq_lens, w.Hq,
                       page_fill=kv_raw.page_fill)
    shift = K.Rope(cos, sin, torch.from_numpy(start[doc_of_page].astype(np.int32)).cuda(), 0)
    kv_abs = K.PagedKV(K.rope_shift(kv_enc, shift), kv_raw.v_pool, kv_raw.page_table,
                       kv_raw.seq_lens, w.Hq, page_fill=kv_raw.page_fill)
    q = w.q.cuda()
    s_f = K.build_summaries(kv_enc, rope=shift)
    s_m = K.build_summaries(kv_abs)
    fused = K.select_attend(kv_enc, s_f, q, w.k, rope=shift)
    mat = K.select_attend(kv_abs, s_m, q, w.k)
    torch.cuda.synchronize()
    assert torch.equal(s_f, s_m)
    for a, b_, name in zip(fused, mat, ("sel", "cnt", "out", "lse")):
        assert torch.equal(a, b_), f"{name}: fused rotary gather differs from materialized keys"


def test_shared_documents_at_different_offsets(K):
    """Two sequences chain the same documents in different orders, so a shared page sits at a
    different position in each; rows by (sequence, logical page) place it per sequence. Each
    sequence's summaries and step outputs equal those of that sequence alone with rows by
    physical page, bit for bit."""
    w = W.composed(1231, B=2)
    say(f"shared documents, per-sequence rotary rows: lens {w.seq_lens.tolist()}")
    page_in_doc = w.extra["page_in_doc"].numpy()
    doc_of_page = w.extra["doc_of_page"].numpy()
    start = w.extra["doc_start"].numpy()  # [B][documents]
    n_rows = int(start.max()) + max(w.extra["doc_lens"]) + w.P
    cos, sin = K.rope_table(w.extra["theta"], w.D, 0, n_rows, torch.device("cuda"))
    kv_raw = composed_kv(K, w)
    enc = K.rope_shift(kv_raw, K.Rope(cos, sin, torch.from_numpy((page_in_doc * w.P).astype(np.int32)).cuda(), 1))
    kv = K.PagedKV(enc, kv_raw.v_pool, kv_raw.page_table, kv_raw.seq_lens, w.Hq,
                   page_fill=kv_raw.page_fill)
    table = w.page_table.numpy()
    rows = np.zeros(table.shape, dtype=np.int32)
    for b in range(w.B):
        for n in range(w.n_pages(b)):
            rows[b, n] = start[b, doc_of_page[table[b, n]]]
    per_seq = K.Rope(cos, sin, torch.from_numpy(rows).cuda(), 0, per_sequence=True)
    q = w.q.cuda()
    summ = K.build_summaries(kv, rope=per_seq)
    both = K.select_attend(kv, summ, q, w.k, rope=per_seq)
    torch.cuda.synchronize()
    for b in range(w.B):
        phys = K.Rope(cos, sin, torch.from_numpy(start[b][doc_of_page].astype(np.int32)).cuda(), 0)
        one = K.PagedKV(enc, kv_raw.v_pool, kv_raw.page_table[b:b + 1].contiguous(),
                        kv_raw.seq_lens[b:b + 1].contiguous(), w.Hq, page_fill=kv_raw.page_fill)
        s1 = K.build_summaries(one, rope=phys)
        alone = K.select_attend(one, s1, q[b:b + 1].contiguous(), w.k, rope=phys)
        torch.cuda.synchronize()
        assert torch.equal(summ[b], s1[0]), f"sequence {b}: summaries"
        for x, y, name in zip(both, alone, ("sel", "cnt", "out", "lse")):
            assert torch.equal(x[b], y[0]), f"sequence {b}: {name}"
    assert not torch.equal(both[2][0], both[2][1])  # the two placements differ
