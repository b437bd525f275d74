"""Parity of the speculative-reuse decision and the rotary re-positioning with the CPU oracle.

The speculative workload: a 32K Llama-shaped cache built from eight 4096-token blocks, each
rotary-encoded at positions 0..4095 and re-rotated to its absolute offset, then 64 decode steps
with AR(1)-correlated queries; step t attends over the pages chosen at step t-1 unless the
group-mean query similarity is below tau.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_common import (assert_attention_close, assert_selection_equal, assert_summaries_equal,
                        kv_of, orderable32, referenced_pages, say, scale_of)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from query_aware_sparse_page_amd import kvsel as K
    K.lib()
    return K


def table_agreement(gc, gs, oc, os_):
    dc = np.abs(orderable32(gc.cpu().numpy()) - orderable32(oc))
    ds = np.abs(orderable32(gs.cpu().numpy()) - orderable32(os_))
    assert dc.max() <= 1 and ds.max() <= 1, "rotary table differs from the oracle's by > 1 ulp"
    return (dc == 0) & (ds == 0)


def test_rope_table_matches_oracle(K):
    say("rope_table theta=500000 D=128 rows=32768")
    gc, gs = K.rope_table(500000.0, 128, 0, 32768, "cuda")
    torch.cuda.synchronize()
    oc, os_ = O.rope_table(500000.0, 128, 0, 32768)
    same = table_agreement(gc, gs, oc, os_)
    say(f"rope table: {int(same.sum())}/{same.size} entries bit-identical")
    # both sides round the same fp64 angle's cos/sin; two libms can differ only when the value
    # sits within an fp64 ulp of an fp32 rounding boundary: every differing entry must be one
    assert same.size - int(same.sum()) <= 4
    gcn, gsn = gc.cpu().numpy(), gs.cpu().numpy()
    for r, i in zip(*np.nonzero(~same)):
        ang = float(r) * math.pow(500000.0, -(2.0 * i) / 128)
        for v64, got, ref in ((math.cos(ang), gcn[r, i], oc[r, i]), (math.sin(ang), gsn[r, i], os_[r, i])):
            if got == ref:
                continue
            lo, hi = sorted((float(got), float(ref)))  # adjacent fp32 values around the fp64 value
            mid = 0.5 * (lo + hi)
            assert abs(v64 - mid) <= 4.0 * np.spacing(abs(v64)), (r, i, v64, got, ref)


@pytest.mark.parametrize("dtype,D,P,row_step,in_place", [
    ("bf16", 128, 32, 1, False), ("bf16", 128, 32, 0, True), ("bf16", 64, 16, 1, True),
    ("f32", 64, 16, 0, False), ("f32", 128, 32, 1, False),
])
def test_rope_shift_matches_oracle(K, dtype, D, P, row_step, in_place):
    w = W.custom(201, B=1, Hq=4, Hkv=2, D=D, P=P, k=2, lens=[P * 40], dtype=dtype)
    rng = np.random.Generator(np.random.PCG64(5))
    page_row = rng.integers(0, 3000, size=w.num_phys_pages).astype(np.int32)
    page_row[::7] = -1
    say(f"rope_shift dtype={dtype} D={D} P={P} row_step={row_step} in_place={in_place}")
    gc, gs = K.rope_table(10000.0, D, 0, 3100, "cuda")
    kv = kv_of(K, w)
    rope = K.Rope(gc, gs, torch.from_numpy(page_row).cuda(), row_step)
    out = K.rope_shift(kv, rope, out=kv.k_pool if in_place else None)
    torch.cuda.synchronize()
    oc, os_ = O.rope_table(10000.0, D, 0, 3100)
    same = table_agreement(gc, gs, oc, os_)
    ref = O.rope_rotate(w.k_pool, oc, os_, page_row, row_step, dtype)
    got = out.float().cpu().numpy()
    # bit-exact wherever both sides used identical table entries
    half = D // 2
    rows = page_row[:, None] + row_step * np.arange(P)[None, :]  # [Npp][P]
    ok_rows = np.where(rows[..., None] >= 0, same[np.clip(rows, 0, None)], True)  # [Npp][P][half]
    mask = np.concatenate([ok_rows, ok_rows], axis=-1)[:, None, :, :]  # [Npp][1][P][D]
    mask = np.broadcast_to(mask, got.shape)
    assert np.array_equal(got[mask], ref[mask])
    # pages with page_row < 0 are untouched
    np.testing.assert_array_equal(got[page_row < 0], w.k_pool.float().numpy()[page_row < 0])


@pytest.fixture(scope="module")
def spec(K):
    """The speculative workload rotated on both sides. The library encodes and shifts the blocks
    twice: with its own rotary table (kvsel_rope_table), and with the oracle's table handed to it
    as data (so both sides rotate with identical cos / sin bits and the rotated keys must agree
    bit for bit)."""
    w = W.speculative_rope()
    blocks = w.extra["block_tokens"] // w.P  # pages per block
    npg = w.num_phys_pages
    enc_row = ((np.arange(npg) % blocks) * w.P).astype(np.int32)
    shift_row = ((np.arange(npg) // blocks) * w.extra["block_tokens"]).astype(np.int32)
    say("speculative workload: rope table + encode + shift (GPU)")
    gc, gs = K.rope_table(w.extra["theta"], w.D, 0, 8 * w.extra["block_tokens"], "cuda")
    kv_raw = kv_of(K, w)
    enc = K.rope_shift(kv_raw, K.Rope(gc, gs, torch.from_numpy(enc_row).cuda(), 1))
    kv_enc = K.PagedKV(enc, kv_raw.v_pool, kv_raw.page_table, kv_raw.seq_lens, w.Hq)
    shift = K.Rope(gc, gs, torch.from_numpy(shift_row).cuda(), 0)
    absk = K.rope_shift(kv_enc, shift)
    torch.cuda.synchronize()
    oc, os_ = O.rope_table(w.extra["theta"], w.D, 0, 8 * w.extra["block_tokens"])
    same = table_agreement(gc, gs, oc, os_)
    o_enc = O.rope_rotate(w.k_pool, oc, os_, enc_row, 1, "bf16")
    o_abs = O.rope_rotate(torch.from_numpy(o_enc).to(torch.bfloat16), oc, os_, shift_row, 0, "bf16")
    # the oracle's table as the library's input data
    dc, ds = torch.from_numpy(oc).cuda(), torch.from_numpy(os_).cuda()
    enc_d = K.rope_shift(kv_raw, K.Rope(dc, ds, torch.from_numpy(enc_row).cuda(), 1))
    kv_enc_d = K.PagedKV(enc_d, kv_raw.v_pool, kv_raw.page_table, kv_raw.seq_lens, w.Hq)
    absk_d = K.rope_shift(kv_enc_d, K.Rope(dc, ds, torch.from_numpy(shift_row).cuda(), 0))
    torch.cuda.synchronize()
    return dict(w=w, kv_enc=kv_enc, shift=shift, absk=absk, o_enc=o_enc, o_abs=o_abs,
                table_same=bool(same.all()), same=same, enc_row=enc_row, shift_row=shift_row,
                enc_gpu=enc, enc_d=enc_d, absk_d=absk_d)


def test_speculative_rope_blocks_match_oracle(spec):
    w = spec["w"]
    # with the oracle's table as data: bit for bit, unconditionally
    np.testing.assert_array_equal(spec["enc_d"].float().cpu().numpy(), spec["o_enc"])
    np.testing.assert_array_equal(spec["absk_d"].float().cpu().numpy(), spec["o_abs"])
    # with the library's own table
    g_enc = spec["enc_gpu"].float().cpu().numpy()
    g_abs = spec["absk"].float().cpu().numpy()
    if spec["table_same"]:
        np.testing.assert_array_equal(g_enc, spec["o_enc"])
        np.testing.assert_array_equal(g_abs, spec["o_abs"])
        return
    # bit-exact wherever every table entry a value depends on agrees; 1 bf16 ulp elsewhere
    same = spec["same"]
    half = w.D // 2
    enc_rows = spec["enc_row"][:, None] + np.arange(w.P)[None, :]
    ok_enc = same[enc_rows]  # [Npp][P][half]
    ok_abs = ok_enc & same[spec["shift_row"]][:, None, :]
    for got, ref, ok in ((g_enc, spec["o_enc"], ok_enc), (g_abs, spec["o_abs"], ok_abs)):
        m = np.broadcast_to(np.concatenate([ok, ok], axis=-1)[:, None], got.shape)
        assert np.array_equal(got[m], ref[m])
        assert (np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-30).all()


def test_fused_rope_is_bit_identical_to_materialized(K, spec):
    w = spec["w"]
    kv_enc = spec["kv_enc"]
    kv_abs = K.PagedKV(spec["absk"], kv_enc.v_pool, kv_enc.page_table, kv_enc.seq_lens, w.Hq)
    say("fused rope: summaries + attention on encoded blocks vs materialized keys")
    s_mat = K.build_summaries(kv_abs)
    s_fused = K.build_summaries(kv_enc, rope=spec["shift"])
    q = w.q.cuda()
    sel, cnt = K.score_topk(kv_abs, s_mat, q, w.k)
    o_mat, l_mat = K.sparse_decode_attn(kv_abs, q, sel, cnt, w.k)
    o_fused, l_fused = K.sparse_decode_attn(kv_enc, q, sel, cnt, w.k, rope=spec["shift"])
    torch.cuda.synchronize()
    assert torch.equal(s_mat, s_fused)
    assert torch.equal(o_mat, o_fused) and torch.equal(l_mat, l_fused)


@pytest.mark.parametrize("tau", [None, 0.85], ids=["tau0.8", "tau0.85"])
def test_speculative_decode_loop_matches_oracle(K, spec, tau):
    """64 decode steps, each run as the serial calls (kvsel_score_topk with reuse, then
    kvsel_sparse_decode_attn over the used pages) and as one kvsel_speculative_step, both against
    the oracle's fresh selection, similarity, decision, used lists and attention over its own used
    lists. tau 0.8 is the workload's (no correction fires); at tau 0.85 about half the decisions
    correct."""
    w = spec["w"]
    tau = w.extra["tau"] if tau is None else tau
    qs = w.extra["q_steps"]
    o_pool = torch.from_numpy(spec["o_abs"]).to(torch.bfloat16)
    # the keys the library encoded and shifted itself (kvsel_rope_shift with the oracle's table as
    # data), end to end through summaries, selection, reuse and attention
    kv = K.PagedKV(spec["absk_d"], spec["kv_enc"].v_pool, spec["kv_enc"].page_table,
                   spec["kv_enc"].seq_lens, w.Hq)
    say("speculative loop: summaries")
    summ = K.build_summaries(kv)
    o_summ = O.page_summaries(o_pool, w.page_table, w.seq_lens, w.P)
    torch.cuda.synchronize()
    assert_summaries_equal(summ, o_summ, w)
    scale = scale_of(w.D)
    prev = (torch.zeros((w.B, w.Hkv, w.k), dtype=torch.int32, device="cuda"),
            torch.zeros((w.B, w.Hkv), dtype=torch.int32, device="cuda"))
    sprev = prev
    o_prev = None
    fires = 0
    for t in range(qs.shape[0]):
        say(f"speculative step {t} (tau {tau})")
        q = qs[t].cuda()
        q_prev = qs[t - 1].cuda() if t > 0 else q
        sel, cnt, used, ucnt, corr, sim = K.score_topk(
            kv, summ, q, w.k, reuse=K.Reuse(q_prev, prev[0], prev[1], tau, first_step=(t == 0)))
        out, lse = K.sparse_decode_attn(kv, q, used, ucnt, w.k,
                                        pages_per_split=K.step_pages_per_split(kv, w.k))
        sp = K.speculative_step(kv, summ, q, w.k,
                                K.Reuse(q_prev, sprev[0], sprev[1], tau, first_step=(t == 0)))
        torch.cuda.synchronize()
        # oracle step
        sc = O.page_scores(qs[t], o_summ, w.page_table, w.seq_lens, w.P)
        f_sel, f_cnt = O.top_pages(sc, w.seq_lens, w.P, w.k)
        C = O.query_similarity(qs[t], qs[t - 1] if t > 0 else qs[t], w.Hkv)
        if o_prev is None:
            o_prev = (f_sel, f_cnt)
        u_sel, u_cnt, o_corr = O.speculative_choice(f_sel, f_cnt, o_prev[0], o_prev[1], C, tau,
                                                    first_step=(t == 0))
        assert_selection_equal(sel, cnt, f_sel, f_cnt)
        assert np.abs(sim.cpu().numpy() - C).max() < 1e-12
        assert np.abs(C - tau).min() > 1e-9, "a correction decision sits on the rounding edge"
        np.testing.assert_array_equal(corr.cpu().numpy(), o_corr)
        assert_selection_equal(used, ucnt, u_sel, u_cnt)
        o_out, o_lse = O.sparse_decode_attention(qs[t], o_pool, w.v_pool, w.page_table, w.seq_lens,
                                                 u_sel, u_cnt, w.P, scale)
        assert_attention_close(out, lse, o_out, o_lse, "bf16")
        # the speculative step against the same oracle results
        assert_selection_equal(sp[0], sp[1], f_sel, f_cnt)
        assert np.abs(sp[5].cpu().numpy() - C).max() < 1e-12
        np.testing.assert_array_equal(sp[4].cpu().numpy(), o_corr)
        assert_selection_equal(sp[2], sp[3], u_sel, u_cnt)
        assert_attention_close(sp[6], sp[7], o_out, o_lse, "bf16")
        fires += int(o_corr.sum()) if t > 0 else 0
        prev = (sel, cnt)
        sprev = (sp[0], sp[1])
        o_prev = (f_sel, f_cnt)
    say(f"speculative loop (tau {tau}): corrections {fires}/{(qs.shape[0] - 1) * w.Hkv}")
    if tau > 0.84:
        assert fires > 0, "no correction fired"
