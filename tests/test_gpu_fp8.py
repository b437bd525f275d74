"""fp8 (E4M3) pages through the C ABI against the oracle: the quantizer bit for bit (codes and
scales), the decoding of every code, summaries bit for bit (outward bf16 rounding), the selection
exactly, attention over the dequantized pages within the bf16 tolerances, and the one-call forms
against the separate calls."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_common import (assert_attention_close, assert_scores_close, assert_selection_equal,
                        assert_summaries_equal, kv_of, say, scale_of)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from query_aware_sparse_page_amd import kvsel as K
    K.lib()  # raises if libkvsel.so is missing: no fallback
    return K


def fp8_reference(w, scale):
    """The oracle's quantization of w's pools and its decode step over the dequantized cache."""
    kc, ks = O.quantize_pages(w.k_pool)
    vc, vs = O.quantize_pages(w.v_pool)  # token-major values; the codes are per element
    q = w.q.to(torch.bfloat16)
    summ = O.page_summaries_fp8(kc, ks, w.page_table, w.seq_lens, w.P)
    sc = O.page_scores(q, summ, w.page_table, w.seq_lens, w.P)
    sel, cnt = O.top_pages(sc, w.seq_lens, w.P, w.k)
    out, lse = O.sparse_decode_attention(q, O.dequantize_pages(kc, ks), O.dequantize_pages(vc, vs),
                                         w.page_table, w.seq_lens, sel, cnt, w.P, scale)
    return dict(kc=kc, ks=ks, vc=vc, vs=vs, q=q, summ=summ, scores=sc, sel=sel, cnt=cnt,
                fp32=None, out=out, lse=lse)


def check_quantized(kv8, ref):
    assert np.array_equal(kv8.k_pool.cpu().numpy(), ref["kc"]), "key codes differ"
    assert np.array_equal(kv8.k_scale.cpu().numpy(), ref["ks"]), "key scales differ"
    assert np.array_equal(kv8.v_pool.permute(0, 1, 3, 2).cpu().numpy(), ref["vc"]), "value codes differ"
    assert np.array_equal(kv8.v_scale.cpu().numpy(), ref["vs"]), "value scales differ"


CASES = [
    dict(seed=901, B=3, Hq=32, Hkv=8, D=128, P=32, k=16, lens=[40 * 32 - 3, 9 * 32 + 1, 1], dtype="bf16"),
    dict(seed=902, B=2, Hq=8, Hkv=2, D=64, P=16, k=12, lens=[100 * 16 + 5, 33], dtype="bf16"),  # G=4
    dict(seed=903, B=2, Hq=16, Hkv=2, D=128, P=16, k=20, lens=[300, 1000], dtype="bf16"),       # G=8
    dict(seed=904, B=2, Hq=8, Hkv=8, D=64, P=32, k=5, lens=[600, 64], dtype="f32"),             # G=1, f32 source
    dict(seed=905, B=3, Hq=8, Hkv=4, D=128, P=32, k=8, lens=[0, 50, 7 * 32], dtype="bf16"),     # empty sequence
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c['seed']}")
def test_fp8_path_matches_oracle(K, case):
    w = W.custom(**case)
    say(f"fp8 path {case['seed']}: lens {case['lens']}, D {w.D}, P {w.P}, G {w.G}, from {w.dtype}")
    scale = scale_of(w.D)
    ref = fp8_reference(w, scale)
    kv8 = K.quantize_pages(kv_of(K, w))
    torch.cuda.synchronize()
    check_quantized(kv8, ref)
    q = ref["q"].cuda()
    summ = K.build_summaries(kv8)
    torch.cuda.synchronize()
    assert_summaries_equal(summ, ref["summ"], w)
    scores = torch.empty((w.B, w.Hkv, w.max_pages), dtype=torch.float32, device="cuda")
    sel, cnt = K.score_topk(kv8, summ, q, w.k, scores=scores)
    out, lse = K.sparse_decode_attn(kv8, q, sel, cnt, w.k, scale=scale,
                                    pages_per_split=K.step_pages_per_split(kv8, w.k))
    torch.cuda.synchronize()
    assert_scores_close(scores, ref["scores"], w, exact=False)
    assert_selection_equal(sel, cnt, ref["sel"], ref["cnt"], ref["fp32"])
    err = assert_attention_close(out, lse, ref["out"], ref["lse"], "bf16")
    # the one-call forms (the top-k fused into the attention launch, the speculative
    # co-launch) give the separate calls' outputs bit for bit
    s2, c2, o2, l2 = K.select_attend(kv8, summ, q, w.k, scale=scale)
    zi = torch.zeros((w.B, w.Hkv, w.k), dtype=torch.int32, device="cuda")
    zc = torch.zeros((w.B, w.Hkv), dtype=torch.int32, device="cuda")
    spec = K.speculative_step(kv8, summ, q, w.k, K.Reuse(q, zi, zc, 0.8, first_step=True),
                              scale=scale)
    torch.cuda.synchronize()
    for a, b_, name in ((s2, sel, "sel"), (c2, cnt, "cnt"), (o2, out, "out"), (l2, lse, "lse"),
                        (spec[0], sel, "spec sel"), (spec[6], out, "spec out"),
                        (spec[7], lse, "spec lse")):
        assert torch.equal(a, b_), f"{name} differs from the separate calls"
    # a second speculative step reusing the first's pages where the queries agree (the attention
    # over the previous pages runs in the scoring launch) equals the serial calls bit for bit
    gen = torch.Generator().manual_seed(case["seed"] + 50)
    q2 = (ref["q"].float() + 0.3 * torch.randn(ref["q"].shape, generator=gen)).to(torch.bfloat16).cuda()
    reuse = K.Reuse(q, spec[0].clone(), spec[1].clone(), 0.95)
    s2 = K.speculative_step(kv8, summ, q2, w.k, reuse, scale=scale)
    r2 = K.score_topk(kv8, summ, q2, w.k, reuse=reuse)
    o2, l2 = K.sparse_decode_attn(kv8, q2, r2[2], r2[3], w.k, scale=scale,
                                  pages_per_split=K.step_pages_per_split(kv8, w.k))
    torch.cuda.synchronize()
    for a, b_, name in zip(s2, tuple(r2) + (o2, l2),
                           ("sel", "cnt", "used", "ucnt", "corrected", "similarity", "out", "lse")):
        assert torch.equal(a, b_), f"second speculative step: {name} differs"
    say(f"fp8 {case['seed']}: max abs attention error {err:.3g}, "
        f"{int((~s2[4].bool()).sum())} lists kept on their previous pages")


def test_fp8_tail_refresh(K):
    """A stale tail summary rebuilt by the score call's refresh equals the oracle's summary of the
    grown page, and the selection follows it."""
    c = dict(seed=911, B=2, Hq=8, Hkv=2, D=128, P=32, k=6, lens=[20 * 32 + 5, 3 * 32 + 31],
             dtype="bf16")
    w = W.custom(**c)
    say("fp8 tail refresh")
    ref = fp8_reference(w, scale_of(w.D))
    kv8 = K.quantize_pages(kv_of(K, w))
    summ = K.build_summaries(kv8)
    for b in range(w.B):  # poison the tail summaries
        summ[b, :, w.n_pages(b) - 1] = 0
    sel, cnt = K.score_topk(kv8, summ, ref["q"].cuda(), w.k, refresh_tail=True)
    torch.cuda.synchronize()
    assert_summaries_equal(summ, ref["summ"], w)
    assert_selection_equal(sel, cnt, ref["sel"], ref["cnt"], ref["fp32"])


def test_every_code_decodes(K):
    """One-token sequences whose value rows hold every non-NaN code (v_scale 1): the attention
    output is the value row itself, so it must equal the OCP E4M3 value of each code exactly; the
    key rows hold every code too, with scales that make the outward rounding work."""
    D, P = 128, 16
    codes = np.arange(256).reshape(2, D)
    codes[0, 0x7F] = 0x00  # NaN codes are never written by the quantizer
    codes[1, 0x7F] = 0x80
    B, Hkv, Hq = 2, 2, 4
    Npp = B
    kc = np.zeros((Npp, Hkv, P, D), np.uint8)
    vc = np.zeros((Npp, Hkv, P, D), np.uint8)
    for p in range(Npp):
        for j in range(Hkv):
            kc[p, j, 0] = codes[p]
            vc[p, j, 0] = codes[p]
            kc[p, j, 1:] = 0x7F  # NaN poison past the sequence's one token
            vc[p, j, 1:] = 0xFF
    rng = np.random.default_rng(921)
    ks = (rng.random((Npp, Hkv)) * 2.0 ** -3 + 2.0 ** -9).astype(np.float32)
    vs = np.ones((Npp, Hkv), np.float32)
    table = torch.arange(B, dtype=torch.int32).reshape(B, 1)
    lens = torch.ones(B, dtype=torch.int32)
    kv8 = K.PagedKV(torch.from_numpy(kc).cuda(), K.device_v_layout(torch.from_numpy(vc)).cuda(),
                    table.cuda(), lens.cuda(), Hq, 0, torch.from_numpy(ks).cuda(),
                    torch.from_numpy(vs).cuda())
    say("fp8: every code")
    summ = K.build_summaries(kv8)
    q = (torch.randn((B, Hq, D), generator=torch.Generator().manual_seed(922)) * 0.05).to(torch.bfloat16)
    sel = torch.zeros((B, Hkv, 1), dtype=torch.int32, device="cuda")
    cnt = torch.ones((B, Hkv), dtype=torch.int32, device="cuda")
    out, lse = K.sparse_decode_attn(kv8, q.cuda(), sel, cnt, 1)
    torch.cuda.synchronize()
    want = O.fp8_e4m3_decode(codes)  # [B][D]
    got = out.double().cpu().numpy()  # [B][Hq][D]
    for b in range(B):
        assert np.array_equal(got[b], np.broadcast_to(want[b], (Hq, D))), f"sequence {b}"
    w = W.Workload("codes", "bf16", B, Hq, Hkv, D, P, 1, lens, table, None, None, q)
    assert_summaries_equal(summ, O.page_summaries_fp8(kc, ks, table, lens, P), w)


def restricted(w, seqs):
    """The sub-workload of sequences `seqs`: their pages only, renumbered (every step of the path
    is per page or per sequence, so the oracle on it gives those sequences' results)."""
    pages = sorted({int(x) for b in seqs for x in w.page_table[b, :w.n_pages(b)]})
    where = {p: i for i, p in enumerate(pages)}
    idx = torch.tensor(pages, dtype=torch.long)
    table = torch.zeros((len(seqs), w.max_pages), dtype=torch.int32)
    for i, b in enumerate(seqs):
        for n in range(w.n_pages(b)):
            table[i, n] = where[int(w.page_table[b, n])]
    return W.Workload(w.name, w.dtype, len(seqs), w.Hq, w.Hkv, w.D, w.P, w.k,
                      w.seq_lens[list(seqs)].clone(), table, w.k_pool[idx], w.v_pool[idx],
                      w.q[list(seqs)].clone()), pages


_full = {}


@pytest.mark.parametrize("name,seqs", [("llama8b_32k", None), ("ragged_batch", (0, 1, 2, 3)),
                                       ("ragged_batch", (4, 5, 6, 7)),
                                       ("ragged_batch", (8, 9, 10, 11)),
                                       ("ragged_batch", (12, 13, 14, 15))])
def test_fp8_full_workloads(K, name, seqs):
    """The full-size workloads quantized on the GPU and run in the bench's launch configuration
    (one kvsel_select_attend call, the default split): quantizer, summaries and selection exact,
    attention within tolerance. The ragged batch runs whole on the GPU; the oracle checks its 16
    sequences four at a time (one case each, to bound the oracle's time per test)."""
    if name not in _full:
        _full.clear()
        _full[name] = W.make(name)
    w = _full[name]
    say(f"fp8 full workload {name}, oracle on sequences {seqs or 'all'}")
    scale = scale_of(w.D)
    kv8 = K.quantize_pages(kv_of(K, w))
    summ = K.build_summaries(kv8)
    q = w.q.to(torch.bfloat16).cuda()
    sel, cnt, out, lse = K.select_attend(kv8, summ, q, w.k, scale=scale)
    torch.cuda.synchronize()
    ws, pages = (w, None) if seqs is None else restricted(w, seqs)
    ref = fp8_reference(ws, scale)
    if seqs is None:
        check_quantized(kv8, ref)
        rows = slice(None)
    else:
        idx = torch.tensor(pages, dtype=torch.long, device="cuda")
        sub = K.PagedKV(kv8.k_pool[idx], kv8.v_pool[idx], None, None, w.Hq, 0, kv8.k_scale[idx],
                        kv8.v_scale[idx])
        check_quantized(sub, ref)
        rows = list(seqs)
    assert_summaries_equal(summ[rows], ref["summ"], ws)
    assert_selection_equal(sel[rows], cnt[rows], ref["sel"], ref["cnt"], ref["fp32"])
    err = assert_attention_close(out[rows], lse[rows], ref["out"], ref["lse"], "bf16")
    say(f"fp8 {name}: max abs attention error {err:.3g}")
