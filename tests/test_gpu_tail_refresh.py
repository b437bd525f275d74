"""The decode-time tail refresh of the score kernel on every block shape, through the C ABI: the
block that holds a sequence's last page rebuilds that page's summary with all of its waves (each
folds a share of the tile's rows; the shares meet in LDS). After a call with the refresh on, every
live summary must equal a fresh summary build of the same keys (and, without the rotary gather,
the oracle's), and the selection must equal the selection over the fresh build. Shapes: 8, 16
and 32 lanes per key row (bf16 D 64, bf16 D 128 / f32 D 64, f32 D 128), pages of 16 and 32 rows,
blocks of up to 128 pages (the tail's page id in a lane's second page-id load), one, two and four
pages per lane group (where the tail block scores its pages before the fold), fp8 pools, the
rotary gather, full, one-row and empty tails; the same through kvsel_select_attend and through
the speculative step's shared launch (2- and 4-wave blocks) against its serial calls."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_common import assert_scores_close, assert_summaries_equal, kv_of, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from query_aware_sparse_page_amd import kvsel as K
    K.lib()  # raises if libkvsel.so is missing: no fallback
    return K


# (name, dtype, D, P, Hq, Hkv, k, lens, pool): pool "fp8" quantizes the bf16 / f32 keys
CASES = [
    ("bf16-D128-P32", "bf16", 128, 32, 32, 8, 6, [700, 64, 33, 1], None),
    ("bf16-D64-P16-wide", "bf16", 64, 16, 8, 2, 12, [16 * 2147 + 5, 300, 16], None),
    ("f32-D128-P32", "f32", 128, 32, 16, 4, 9, [32 * 250 + 7, 40, 32], None),
    ("f32-D64-P16", "f32", 64, 16, 8, 4, 7, [16 * 100 + 3, 17, 0], None),
    ("bf16-D128-P16", "bf16", 128, 16, 16, 2, 10, [16 * 300 + 1, 32, 5], None),
    ("bf16-D128-P16-U2", "bf16", 128, 16, 16, 4, 10, [16 * 1500 + 7, 900], None),
    ("f32-D64-P32-U2", "f32", 64, 32, 8, 4, 8, [32 * 1300 + 1, 64], None),
    ("fp8-D128-P32", "bf16", 128, 32, 32, 8, 6, [40 * 32 - 3, 9 * 32 + 1, 1], "fp8"),
    ("fp8-D64-P16-wide", "bf16", 64, 16, 8, 2, 12, [16 * 2147 + 9, 16 * 3], "fp8"),
]


def rope_for(K, w, n_rows=4):
    """A rotary table and a per-physical-page row map: half the pages shifted (row_step 0), the
    rest left as stored."""
    cos, sin = K.rope_table(500000.0, w.D, 4096, n_rows, torch.device("cuda"))
    page_row = torch.full((w.num_phys_pages,), -1, dtype=torch.int32)
    half = w.num_phys_pages // 2
    page_row[:half] = torch.arange(half, dtype=torch.int32) % n_rows
    return K.Rope(cos, sin, page_row.cuda(), row_step=0)


def setup(K, case, seed):
    name, dtype, D, P, Hq, Hkv, k, lens, pool = case
    w = W.custom(seed, B=len(lens), Hq=Hq, Hkv=Hkv, D=D, P=P, k=k, lens=lens, dtype=dtype)
    gen = torch.Generator().manual_seed(seed)
    for b in range(w.B):  # a decode step wrote new keys into each tail page
        if w.n_pages(b):
            p = int(w.page_table[b, w.n_pages(b) - 1])
            w.k_pool[p] = torch.randn(w.k_pool[p].shape, generator=gen).to(w.k_pool.dtype)
    kv = kv_of(K, w)
    if pool == "fp8":
        kv = K.quantize_pages(kv)
    return w, kv


def poison_tails(summ, w):
    for b in range(w.B):
        if w.n_pages(b):
            summ[b, :, w.n_pages(b) - 1] = 0
    return summ


def assert_live_equal(a, b, w):
    for i in range(w.B):
        n = w.n_pages(i)
        assert torch.equal(a[i, :, :n], b[i, :, :n]), f"sequence {i}: summaries differ"


def oracle_summaries(w, kv):
    if kv.is_fp8:
        return O.page_summaries_fp8(kv.k_pool.cpu().numpy(), kv.k_scale.cpu().numpy(),
                                    w.page_table, w.seq_lens, w.P)
    return O.page_summaries(w.k_pool, w.page_table, w.seq_lens, w.P)


@pytest.mark.parametrize("rotary", [False, True], ids=["plain", "rotary"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_refresh_equals_fresh_build(K, case, rotary):
    if rotary and case[8] == "fp8":
        pytest.skip("fp8 pools have no rotary gather")
    w, kv = setup(K, case, 1500 + CASES.index(case))
    rope = rope_for(K, w) if rotary else None
    q = w.q.cuda() if not kv.is_fp8 else w.q.to(torch.bfloat16).cuda()
    say(f"tail refresh {case[0]} ({'rotary' if rotary else 'plain'}): lens {case[7]}")
    fresh = K.build_summaries(kv, rope=rope)
    summ = poison_tails(fresh.clone(), w)
    sc = torch.full((w.B, w.Hkv, w.max_pages), float("nan"), device="cuda")
    sel, cnt = K.score_topk(kv, summ, q, w.k, refresh_tail=True, rope=rope, scores=sc)
    sc2 = torch.full_like(sc, float("nan"))
    sel2, cnt2 = K.score_topk(kv, fresh, q, w.k, rope=rope, scores=sc2)
    torch.cuda.synchronize()
    assert_live_equal(summ, fresh, w)
    if not rotary:
        assert_summaries_equal(summ, oracle_summaries(w, kv), w)
    assert torch.equal(cnt, cnt2)
    assert torch.equal(sel, sel2)
    assert_scores_close(sc, sc2.cpu().numpy(), w, exact=True)
    # the one-call form: scores (with the refresh) and the fused selection + attention
    summ3 = poison_tails(fresh.clone(), w)
    out = K.select_attend(kv, summ3, q, w.k, refresh_tail=True, rope=rope)
    torch.cuda.synchronize()
    assert_live_equal(summ3, fresh, w)
    assert torch.equal(out[0], sel) and torch.equal(out[1], cnt)


# (dtype, D, P, Hq, Hkv, k, lens): the shared launch's block shapes (bf16 P 32: 4 waves; bf16
# P 16: 2 waves; f32: 4 waves)
SPEC_SHAPES = [
    ("bf16", 128, 32, 32, 8, 16, [4000, 3000, 2017, 33]),
    ("bf16", 64, 16, 16, 8, 12, [16 * 250 + 3, 16 * 40, 1]),
    ("f32", 128, 32, 16, 8, 16, [32 * 120 + 31, 32 * 7]),
    ("f32", 64, 16, 8, 8, 9, [16 * 300 + 8, 100]),
]


@pytest.mark.parametrize("shape", SPEC_SHAPES, ids=lambda s: f"{s[0]}-D{s[1]}-P{s[2]}")
def test_speculative_step_refresh_matches_serial(K, shape):
    dtype, D, P, Hq, Hkv, k, lens = shape
    case = (f"spec-{dtype}", dtype, D, P, Hq, Hkv, k, lens, None)
    w, kv = setup(K, case, 1600 + SPEC_SHAPES.index(shape))
    say(f"speculative step with the tail refresh: {shape}")
    q = w.q.cuda()
    gen = torch.Generator().manual_seed(1700)
    q_prev = (w.q.float() + 0.05 * torch.randn(w.q.shape, generator=gen)).to(w.q.dtype).cuda()
    fresh = K.build_summaries(kv)
    prev_idx, prev_cnt = K.score_topk(kv, fresh, q_prev, k)
    for first in (False, True):
        reuse = K.Reuse(q_prev, prev_idx, prev_cnt, 0.8, first_step=first)
        sa = poison_tails(fresh.clone(), w)
        sb = poison_tails(fresh.clone(), w)
        spec = K.speculative_step(kv, sa, q, k, reuse, refresh_tail=True)
        sel, cnt, used, ucnt, corr, sim = K.score_topk(kv, sb, q, k, reuse=reuse, refresh_tail=True)
        out, lse = K.sparse_decode_attn(kv, q, used, ucnt, k,
                                        pages_per_split=K.step_pages_per_split(kv, k))
        torch.cuda.synchronize()
        assert_live_equal(sa, fresh, w)
        assert_live_equal(sb, fresh, w)
        for x, y, n in zip(spec, (sel, cnt, used, ucnt, corr, sim, out, lse),
                           ("sel_idx", "sel_cnt", "used_idx", "used_cnt", "corrected",
                            "similarity", "out", "lse")):
            assert torch.equal(x, y), f"{n} differs between the speculative step and the serial calls"
    assert np.isfinite(spec[7].cpu().numpy()[np.asarray(lens)[:, None].repeat(w.Hq, 1) > 0]).all()
