"""C ABI on the CPU: the library loads, exports every symbol include/kvsel.h declares, and its
host-side validation returns the documented status codes before touching any device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvsel.h")


@pytest.fixture(scope="module")
def K():
    from query_aware_sparse_page_amd import kvsel as K
    if not os.path.exists(K.LIB_PATH):
        from query_aware_sparse_page_amd.build import build
        build()
    K.lib()
    return K


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvsel_[a-z_]+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ["kvsel_build_summaries", "kvsel_score_topk", "kvsel_sparse_decode_attn",
              "kvsel_rope_shift"]:
        assert n in names


def test_every_declared_symbol_is_exported(K):
    lib = K.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(K.EXPORTS)


def test_version_and_status_strings(K):
    lib = K.lib()
    assert lib.kvsel_abi_version() == K.ABI_VERSION == 7
    for code, tag in [(0, "KVSEL_OK"), (1, "INVALID_ARGUMENT"), (2, "UNSUPPORTED"),
                      (3, "WORKSPACE"), (4, "DEVICE"), (5, "LAUNCH"), (6, "SCRATCH"),
                      (99, "UNKNOWN")]:
        assert tag in lib.kvsel_status_str(code).decode()


def _desc(K, **kw):
    base = dict(dtype=K.KVSEL_BF16, batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128,
                page_size=32, num_phys_pages=1024, max_pages_per_seq=1024,
                k_pool=0x1000, v_pool=0x2000, page_table=0x3000, seq_lens=0x4000,
                max_seq_len=0, k_scale=None, v_scale=None, page_fill=None)
    base.update(kw)
    return K.PagedKVDesc(*[base[f] for f, _ in K.PagedKVDesc._fields_])


def test_workspace_sizes(K):
    lib = K.lib()
    d = _desc(K)
    ws = lib.kvsel_workspace_bytes(ctypes.byref(d), 64, K.KVSEL_OP_SCORE_TOPK, 0)
    assert ws == 1 * 8 * 1024 * 4  # room for the scores
    # 64 pages in splits of 2 -> 32 partials per (b, KV head, query head of the group): the
    # accumulator rows, then (m, l, lu, unused) as 4 floats
    parts = 1 * 8 * 32 * 4
    acc = parts * 128 * 4
    assert lib.kvsel_workspace_bytes(ctypes.byref(d), 64, K.KVSEL_OP_ATTENTION, 2) == \
        ((acc + 255) // 256) * 256 + parts * 16
    # one split needs no workspace
    assert lib.kvsel_workspace_bytes(ctypes.byref(d), 2, K.KVSEL_OP_ATTENTION, 2) == 0
    assert lib.kvsel_workspace_bytes(None, 64, K.KVSEL_OP_SCORE_TOPK, 0) == 0
    assert lib.kvsel_workspace_bytes(ctypes.byref(d), 0, K.KVSEL_OP_SCORE_TOPK, 0) == 0


def _attn_ws(lib, d, k, pps):
    return lib.kvsel_workspace_bytes(ctypes.byref(d), k, 2, pps)  # KVSEL_OP_ATTENTION


def test_default_and_step_splits(K):
    """The library's split choices, read through the workspace sizes and the step-split query:
    below 64 lists 2 pages when lists x ceil(k / 2) <= 256, else 4; 8 from 64 lists on. The
    select-attend and speculative calls run 4-page splits below 64 lists (their fused launches'),
    the default from 64 lists on."""
    lib = K.lib()
    one = _desc(K)  # 8 lists of 1024 pages
    assert _attn_ws(lib, one, 64, 0) == _attn_ws(lib, one, 64, 2)  # 8 x 32 = 256 blocks
    assert _attn_ws(lib, one, 128, 0) == _attn_ws(lib, one, 128, 4)  # 8 x 64 > 256
    assert lib.kvsel_step_pages_per_split(ctypes.byref(one), 64) == 4
    assert lib.kvsel_step_pages_per_split(ctypes.byref(one), 128) == 4
    scores = 8 * 1024 * 4
    assert lib.kvsel_workspace_bytes(ctypes.byref(one), 64, K.KVSEL_OP_SELECT_ATTEND, 0) == \
        scores + _attn_ws(lib, one, 64, 4)
    two = _desc(K, batch=2, num_phys_pages=2048)  # 16 lists: 16 x 32 > 256
    assert _attn_ws(lib, two, 64, 0) == _attn_ws(lib, two, 64, 4)
    many = _desc(K, batch=8, num_phys_pages=8192)  # 64 lists
    assert _attn_ws(lib, many, 64, 0) == _attn_ws(lib, many, 64, 8)
    assert lib.kvsel_step_pages_per_split(ctypes.byref(many), 64) == 8
    assert lib.kvsel_workspace_bytes(ctypes.byref(many), 64, K.KVSEL_OP_SPECULATIVE_STEP, 0) == \
        8 * 8 * 1024 * 4 + _attn_ws(lib, many, 64, 8)
    # a k that needs more than 256 splits of 4 raises the split
    assert lib.kvsel_step_pages_per_split(ctypes.byref(one), 1024) == 4
    assert lib.kvsel_step_pages_per_split(ctypes.byref(one), 0) == 0
    assert lib.kvsel_step_pages_per_split(None, 64) == 0


@pytest.mark.parametrize("field,value,status", [
    ("num_q_heads", 30, 1),          # Hq % Hkv != 0
    ("batch", 0, 1),
    ("k_pool", None, 1),
    ("head_dim", 96, 2),
    ("page_size", 64, 2),
    ("num_q_heads", 8 * 16, 2),      # G = 16
    ("dtype", 7, 2),
    ("batch", 65536, 2),             # beyond the launch-grid limits
    ("max_pages_per_seq", (1 << 20) + 1, 2),
    ("max_seq_len", -1, 1),
    ("dtype", 2, 1),                 # fp8 without k_scale
])
def test_descriptor_validation(K, field, value, status):
    lib = K.lib()
    d = _desc(K, **{field: value})
    st = lib.kvsel_build_summaries(ctypes.byref(d), None, 0, ctypes.c_void_p(0x5000), None)
    assert st == status


def test_call_argument_validation(K):
    lib = K.lib()
    d = _desc(K)
    p = ctypes.c_void_p(0x5000)
    assert lib.kvsel_build_summaries(None, None, 0, p, None) == 1
    assert lib.kvsel_build_summaries(ctypes.byref(d), None, 0, None, None) == 1
    # score/top-k: k < 1, NULL outputs, unknown flags, missing or short workspace
    st = lib.kvsel_score_topk
    assert st(ctypes.byref(d), None, p, p, 0, 0, p, p, p, None, p, 1 << 20, None) == 1
    assert st(ctypes.byref(d), None, p, p, 64, 0, None, p, p, None, p, 1 << 20, None) == 1
    assert st(ctypes.byref(d), None, p, p, 64, 4, p, p, p, None, p, 1 << 20, None) == 1
    assert st(ctypes.byref(d), None, p, p, 64, 0, p, p, None, None, None, 0, None) == 3
    assert st(ctypes.byref(d), None, p, p, 64, 0, p, p, None, None, p, 1024, None) == 3
    bad_reuse = K.ReuseDesc(None, 1, 1, 0.8, 0, 1, 1, 1, None)
    assert st(ctypes.byref(d), None, p, p, 64, 0, p, p, p, ctypes.byref(bad_reuse), p, 1 << 20,
              None) == 1
    bad_rope = K.RopeDesc(0x10, None, 0x30, 4, 0)
    assert st(ctypes.byref(d), ctypes.byref(bad_rope), p, p, 64, 1, p, p, p, None, p, 1 << 20,
              None) == 1
    # attention: missing V pool, bad split request, workspace too small
    dv = _desc(K, v_pool=None)
    assert lib.kvsel_sparse_decode_attn(ctypes.byref(dv), None, p, p, p, 64, 0.1, 0, p, None, p,
                                        1 << 30, None) == 1
    assert lib.kvsel_sparse_decode_attn(ctypes.byref(d), None, p, p, p, 64, 0.1, -1, p, None, p,
                                        1 << 30, None) == 1
    assert lib.kvsel_sparse_decode_attn(ctypes.byref(d), None, p, p, p, 64, 0.1, 2, p, None, p,
                                        100, None) == 3
    # rope descriptors
    bad_rope = K.RopeDesc(0x10, 0x20, 0x30, 4, 2)
    assert lib.kvsel_rope_shift(ctypes.byref(d), ctypes.byref(bad_rope), p, None) == 1
    # per-sequence rows cannot be materialized into shared physical pages
    per_seq = K.RopeDesc(0x10, 0x20, 0x30, 4, 0, 1)
    assert lib.kvsel_rope_shift(ctypes.byref(d), ctypes.byref(per_seq), p, None) == 2
    assert lib.kvsel_rope_shift(ctypes.byref(d), None, p, None) == 1
    assert lib.kvsel_rope_table(500000.0, 127, 0, 4, p, p, None) == 1
    assert lib.kvsel_rope_table(-1.0, 128, 0, 4, p, p, None) == 1


def test_select_attend_static_validation(K):
    """The entry point without a workspace rejects a call whose scores and partials exceed the
    library's static scratch before touching any device, and checks its arguments."""
    lib = K.lib()
    p = ctypes.c_void_p(0x5000)
    fn = lib.kvsel_select_attend_static
    big = _desc(K, batch=64, num_phys_pages=64 * 4096, max_pages_per_seq=4096)
    need = lib.kvsel_workspace_bytes(ctypes.byref(big), 64, K.KVSEL_OP_SELECT_ATTEND, 0)
    assert need > K.KVSEL_STATIC_SCRATCH_BYTES
    assert fn(ctypes.byref(big), None, p, p, 64, 0, 0.1, p, p, p, p, None) == K.KVSEL_ERR_SCRATCH
    d = _desc(K)
    assert lib.kvsel_workspace_bytes(ctypes.byref(d), 64, K.KVSEL_OP_SELECT_ATTEND, 0) <= \
        K.KVSEL_STATIC_SCRATCH_BYTES
    assert fn(ctypes.byref(d), None, None, p, 64, 0, 0.1, p, p, p, p, None) == 1  # no summaries
    assert fn(ctypes.byref(d), None, p, p, 0, 0, 0.1, p, p, p, p, None) == 1      # k < 1
    assert fn(ctypes.byref(d), None, p, p, 64, 4, 0.1, p, p, p, p, None) == 1     # unknown flag
    assert fn(ctypes.byref(d), None, p, p, 64, 0, 0.1, p, p, None, p, None) == 1  # no output


def test_gather_probe_validation(K):
    lib = K.lib()
    p = ctypes.c_void_p(0x5000)
    assert lib.kvsel_gather_probe(None, 4, 8192, p, None) == 1
    assert lib.kvsel_gather_probe(p, 4, 8192, None, None) == 1
    assert lib.kvsel_gather_probe(p, 0, 8192, p, None) == 1
    for bad in (0, 512, 3072, 65536, 8193):
        assert lib.kvsel_gather_probe(p, 4, bad, p, None) == 1


def test_check_inputs_validation(K):
    lib = K.lib()
    d = _desc(K)
    p = ctypes.c_void_p(0x5000)
    assert lib.kvsel_check_inputs(ctypes.byref(d), None, None, 0, None, None) == 1   # no flags
    assert lib.kvsel_check_inputs(ctypes.byref(d), p, None, 64, p, None) == 1        # no counts
    assert lib.kvsel_check_inputs(ctypes.byref(d), p, p, 0, p, None) == 1            # k < 1
    dn = _desc(K, page_table=None)
    assert lib.kvsel_check_inputs(ctypes.byref(dn), None, None, 0, p, None) == 1


def test_append_validation(K):
    lib = K.lib()
    d = _desc(K)
    p = ctypes.c_void_p(0x5000)
    ap = lib.kvsel_append_kv
    assert ap(ctypes.byref(d), None, p, p, p, None, None, None) == 1      # no k_new
    assert ap(ctypes.byref(d), p, None, p, p, None, None, None) == 1      # no v_new
    assert ap(ctypes.byref(d), p, p, None, None, None, None, None) == 1   # no lengths out
    dv = _desc(K, v_pool=None)
    assert ap(ctypes.byref(dv), p, p, None, p, None, None, None) == 1     # no V pool
    dn = _desc(K, page_table=None)
    assert ap(ctypes.byref(dn), p, p, None, p, None, None, None) == 1
    assert ap(ctypes.byref(_desc(K, head_dim=96)), p, p, None, p, None, None, None) == 2
    # free-page list: ids, count and a positive capacity required
    for fp in (K.FreePagesDesc(None, 0x6000, 4), K.FreePagesDesc(0x6000, None, 4),
               K.FreePagesDesc(0x6000, 0x7000, 0)):
        assert ap(ctypes.byref(d), p, p, None, p, ctypes.byref(fp), None, None) == 1


def test_fp8_validation(K):
    """fp8 caches: scales required, no rotary argument, no append or rotary shift; the quantizer
    takes an f32 / bf16 source and needs its outputs."""
    lib = K.lib()
    p = ctypes.c_void_p(0x5000)
    f8 = _desc(K, dtype=K.KVSEL_FP8_E4M3, k_scale=0x8000, v_scale=0x9000)
    no_v = _desc(K, dtype=K.KVSEL_FP8_E4M3, k_scale=0x8000)
    rope = K.RopeDesc(0x10, 0x20, 0x30, 4, 0)
    # attention needs the value scales
    assert lib.kvsel_sparse_decode_attn(ctypes.byref(no_v), None, p, p, p, 64, 0.1, 0, p, None, p,
                                        1 << 30, None) == 1
    assert lib.kvsel_build_summaries(ctypes.byref(f8), ctypes.byref(rope), 0, p, None) == 2
    assert lib.kvsel_rope_shift(ctypes.byref(f8), ctypes.byref(rope), p, None) == 2
    assert lib.kvsel_append_kv(ctypes.byref(f8), p, p, None, p, None, None, None) == 2
    q = lib.kvsel_quantize_pages
    assert q(ctypes.byref(f8), p, p, p, p, None) == 2          # source already fp8
    assert q(ctypes.byref(_desc(K)), None, p, None, None, None) == 1
    assert q(ctypes.byref(_desc(K)), p, p, p, None, None) == 1  # v codes without v scales
    assert q(ctypes.byref(_desc(K, v_pool=None)), p, p, p, p, None) == 1
