"""kvsel_speculative_step (attention over the previous pages overlapped with the selection on a
side stream, corrected lists attended again) against the serial calls, bit for bit, and the
oracle; eager and captured in a HIP graph."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_common import assert_attention_close, kv_of, say, scale_of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from query_aware_sparse_page_amd import kvsel as K
    K.lib()
    return K


def setup_case(K, k, seed=601, dtype="bf16"):
    w = W.custom(seed, B=4, Hq=32, Hkv=8, D=128, P=32, k=k, lens=[4000, 3000, 2017, 5000],
                 dtype=dtype)
    kv = kv_of(K, w)
    summ = K.build_summaries(kv)
    gen = torch.Generator().manual_seed(seed)
    q = w.q.clone().float()
    q_prev = q.clone()
    # KV heads 0..3 of every sequence keep a close previous query, 4..7 a fresh one
    G = w.Hq // w.Hkv
    close = q[:, : 4 * G] + 0.05 * torch.randn(q[:, : 4 * G].shape, generator=gen)
    q_prev[:, : 4 * G] = close
    q_prev[:, 4 * G:] = torch.randn(q_prev[:, 4 * G:].shape, generator=gen)
    q = q.to(w.q.dtype).cuda()
    q_prev = q_prev.to(w.q.dtype).cuda()
    prev_idx, prev_cnt = K.score_topk(kv, summ, q_prev, k)  # the previous step's fresh pages
    torch.cuda.synchronize()
    return w, kv, summ, q, q_prev, prev_idx, prev_cnt


def serial(K, kv, summ, q, k, reuse):
    sel, cnt, used, ucnt, corr, sim = K.score_topk(kv, summ, q, k, reuse=reuse)
    out, lse = K.sparse_decode_attn(kv, q, used, ucnt, k)
    return sel, cnt, used, ucnt, corr, sim, out, lse


NAMES = ("sel_idx", "sel_cnt", "used_idx", "used_cnt", "corrected", "similarity", "out", "lse")


def assert_same(a, b):
    for x, y, n in zip(a, b, NAMES):
        assert torch.equal(x, y), f"{n} differs between the speculative step and the serial calls"


@pytest.mark.parametrize("k", [16, 4])  # 4 splits (merge) and a single split (direct writes)
def test_speculative_step_matches_serial(K, k):
    w, kv, summ, q, q_prev, prev_idx, prev_cnt = setup_case(K, k)
    for first in (False, True):
        say(f"speculative step k={k} first_step={first}")
        reuse = K.Reuse(q_prev, prev_idx, prev_cnt, 0.8, first_step=first)
        spec = K.speculative_step(kv, summ, q, k, reuse)
        ref = serial(K, kv, summ, q, k, reuse)
        torch.cuda.synchronize()
        assert_same(spec, ref)
        corr = spec[4].cpu().numpy()
        if first:
            assert corr.all()
        else:
            assert corr[:, 4:].all() and not corr[:, :4].any()  # both outcomes occur
    # the used pages' attention against the oracle
    out, lse = spec[6], spec[7]
    o_out, o_lse = O.sparse_decode_attention(q.cpu(), w.k_pool, w.v_pool, w.page_table, w.seq_lens,
                                             spec[2].cpu().numpy(), spec[3].cpu().numpy(), w.P,
                                             scale_of(w.D))
    assert_attention_close(out, lse, o_out, o_lse, "bf16")


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
        K.speculative_step(kv, summ, q, k, reuse)  # warm-up (creates the side objects)
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
