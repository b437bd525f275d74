"""kvsel_speculative_step (attention over the previous pages in the scoring launch, corrected
lists attended again by the fused selection) against the serial calls, bit for bit, and the
oracle; every block shape of the co-scheduled launch, the rotary gather, the serial fallback, and
capture in a HIP graph."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_common import (assert_attention_close, assert_selection_equal, fp32_boundary, kv_of, say,
                        scale_of)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from query_aware_sparse_page_amd import kvsel as K
    K.lib()
    return K


def setup_case(K, k, seed=601, dtype="bf16", Hq=32, Hkv=8, D=128, P=32,
               lens=(4000, 3000, 2017, 5000), rope=None):
    w = W.custom(seed, B=len(lens), Hq=Hq, Hkv=Hkv, D=D, P=P, k=k, lens=list(lens), dtype=dtype)
    kv = kv_of(K, w)
    summ = K.build_summaries(kv, rope=rope)
    gen = torch.Generator().manual_seed(seed)
    q = w.q.clone().float()
    q_prev = q.clone()
    # the first half of the KV heads of every sequence keep a close previous query, the rest get
    # a fresh one
    G = Hq // Hkv
    h = (Hkv // 2) * G
    q_prev[:, :h] = q[:, :h] + 0.05 * torch.randn(q[:, :h].shape, generator=gen)
    q_prev[:, h:] = torch.randn(q_prev[:, h:].shape, generator=gen)
    q = q.to(w.q.dtype).cuda()
    q_prev = q_prev.to(w.q.dtype).cuda()
    prev_idx, prev_cnt = K.score_topk(kv, summ, q_prev, k)  # the previous step's fresh pages
    torch.cuda.synchronize()
    return w, kv, summ, q, q_prev, prev_idx, prev_cnt


def serial(K, kv, summ, q, k, reuse, rope=None):
    sel, cnt, used, ucnt, corr, sim = K.score_topk(kv, summ, q, k, reuse=reuse)
    out, lse = K.sparse_decode_attn(kv, q, used, ucnt, k, rope=rope,
                                    pages_per_split=K.step_pages_per_split(kv, k))
    return sel, cnt, used, ucnt, corr, sim, out, lse


NAMES = ("sel_idx", "sel_cnt", "used_idx", "used_cnt", "corrected", "similarity", "out", "lse")


def assert_same(a, b):
    for x, y, n in zip(a, b, NAMES):
        assert torch.equal(x, y), f"{n} differs between the speculative step and the serial calls"


def check_both_outcomes(K, kv, summ, q, q_prev, prev_idx, prev_cnt, k, rope=None, specs=None):
    Hkv = kv.num_kv_heads
    for first in (False, True):
        reuse = K.Reuse(q_prev, prev_idx, prev_cnt, 0.8, first_step=first)
        spec = K.speculative_step(kv, summ, q, k, reuse, rope=rope)
        ref = serial(K, kv, summ, q, k, reuse, rope=rope)
        torch.cuda.synchronize()
        assert_same(spec, ref)
        corr = spec[4].cpu().numpy()
        if first:
            assert corr.all()
        else:  # both outcomes occur
            assert corr[:, Hkv // 2:].all() and not corr[:, :Hkv // 2].any()
        if specs is not None:
            specs[first] = spec
    return spec


def check_against_oracle(w, q, q_prev, k, tau, first, spec):
    """The step's fresh selection, similarity, decision and used lists against the oracle's (its
    previous selection being the oracle's top-k for q_prev), and the attention against the oracle
    over the oracle's own used lists."""
    summ = O.page_summaries(w.k_pool, w.page_table, w.seq_lens, w.P)
    qc, pc = q.cpu(), q_prev.cpu()
    sc = O.page_scores(qc, summ, w.page_table, w.seq_lens, w.P)
    f_sel, f_cnt = O.top_pages(sc, w.seq_lens, w.P, k)
    psc = O.page_scores(pc, summ, w.page_table, w.seq_lens, w.P)
    p_sel, p_cnt = O.top_pages(psc, w.seq_lens, w.P, k)
    C = O.query_similarity(qc, pc, w.Hkv)
    u_sel, u_cnt, corr = O.speculative_choice(f_sel, f_cnt, p_sel, p_cnt, C, tau, first)
    assert_selection_equal(spec[0], spec[1], f_sel, f_cnt,
                           fp32_boundary(w.dtype, sc, w.seq_lens, w.P, k))
    assert np.abs(spec[5].cpu().numpy() - C).max() < 1e-12
    np.testing.assert_array_equal(spec[4].cpu().numpy(), corr)
    used_sc = np.where(corr[:, :, None].astype(bool), sc, psc)
    assert_selection_equal(spec[2], spec[3], u_sel, u_cnt,
                           fp32_boundary(w.dtype, used_sc, w.seq_lens, w.P, k))
    o_out, o_lse = O.sparse_decode_attention(qc, w.k_pool, w.v_pool, w.page_table, w.seq_lens,
                                             u_sel, u_cnt, w.P, scale_of(w.D))
    assert_attention_close(spec[6], spec[7], o_out, o_lse, w.dtype)


# (dtype, P, D, Hq, Hkv, k): every block shape of the co-scheduled launch (bf16 P 32: 4 waves;
# bf16 P 16: 2 waves; fp32 P 32: 4 waves x 2 tiles; fp32 P 16), group sizes 1..8, one split
# (direct writes, no merge) and many
SHAPES = [
    ("bf16", 32, 128, 32, 8, 16),
    ("bf16", 32, 128, 32, 8, 4),
    ("bf16", 16, 64, 64, 8, 12),
    ("f32", 32, 128, 16, 8, 16),
    ("f32", 16, 64, 8, 8, 9),
    ("bf16", 32, 64, 8, 4, 40),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_speculative_step_matches_serial(K, shape):
    dtype, P, D, Hq, Hkv, k = shape
    say(f"speculative step {shape}")
    w, kv, summ, q, q_prev, prev_idx, prev_cnt = setup_case(K, k, dtype=dtype, Hq=Hq, Hkv=Hkv,
                                                              D=D, P=P)
    specs = {}
    check_both_outcomes(K, kv, summ, q, q_prev, prev_idx, prev_cnt, k, specs=specs)
    for first, spec in specs.items():  # both decision outcomes, and the first step
        check_against_oracle(w, q, q_prev, k, 0.8, first, spec)


def test_speculative_step_empty_and_short_sequences(K):
    k = 16
    say("speculative step: empty, one-page and short sequences")
    w, kv, summ, q, q_prev, prev_idx, prev_cnt = setup_case(K, k, seed=605,
                                                              lens=(0, 31, 4000, 33, 512))
    spec = check_both_outcomes(K, kv, summ, q, q_prev, prev_idx, prev_cnt, k)
    assert int(spec[1][0].max()) == 0 and int(spec[3][0].max()) == 0
    assert bool((spec[7][0] == float("-inf")).all()) and not bool(spec[6][0].float().any())


def test_speculative_step_rotary_gather(K):
    k = 16
    n_rows = 4
    lens = (4000, 3000, 2017, 5000)
    n_phys = sum(-(-L // 32) for L in lens)
    cos, sin = K.rope_table(500000.0, 128, 4096, n_rows, torch.device("cuda"))
    page_row = torch.full((n_phys,), -1, dtype=torch.int32)
    page_row[: n_phys // 2] = torch.arange(n_phys // 2, dtype=torch.int32) % n_rows
    rope = K.Rope(cos, sin, page_row.cuda(), row_step=0)
    say("speculative step with the rotary gather")
    w, kv, summ, q, q_prev, prev_idx, prev_cnt = setup_case(K, k, seed=603, lens=lens, rope=rope)
    check_both_outcomes(K, kv, summ, q, q_prev, prev_idx, prev_cnt, k, rope=rope)


def test_speculative_step_serial_fallback(K):
    # k above 1024 needs splits larger than the fused selection's: the two calls run serially
    k = 1100
    say("speculative step fallback: k = 1100")
    w, kv, summ, q, q_prev, prev_idx, prev_cnt = setup_case(K, k, seed=604, Hq=8, Hkv=2, D=64,
                                                              P=16, lens=(16 * 1500,))
    check_both_outcomes(K, kv, summ, q, q_prev, prev_idx, prev_cnt, k)


def test_speculative_step_wide_table(K):
    # 2100 pages: 16 score keys per thread in the fused select (a form kvsel_select_attend does
    # not take), with the previous pages attended in the shared launch
    k = 32
    say("speculative step: 2100-page table")
    w, kv, summ, q, q_prev, prev_idx, prev_cnt = setup_case(K, k, seed=606, Hq=16, Hkv=4,
                                                              lens=(32 * 2100 - 9, 32 * 700))
    check_both_outcomes(K, kv, summ, q, q_prev, prev_idx, prev_cnt, k)


def test_speculative_step_in_a_graph(K):
    k = 16
    w, kv, summ, q, q_prev, prev_idx, prev_cnt = setup_case(K, k, seed=602)
    reuse = K.Reuse(q_prev, prev_idx, prev_cnt, 0.8, first_step=False)
    ref = serial(K, kv, summ, q, k, reuse)
    torch.cuda.synchronize()
    say("speculative step captured in a graph")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        K.speculative_step(kv, summ, q, k, reuse)  # warm-up
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        res = K.speculative_step(kv, summ, q, k, reuse)
    for rep in range(3):  # replays, with eager work in between
        for t in res:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert_same(res, ref)
        _ = serial(K, kv, summ, q, k, reuse)
        torch.cuda.synchronize()
