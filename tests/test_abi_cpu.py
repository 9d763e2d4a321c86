"""The C-ABI library on the CPU: it loads, exports what include/eagle_verify.h
declares, and validates/plans without touching the device."""
import ctypes as C
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ev = pytest.importorskip("eagle_draft_tree_attention_amd")


def test_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "eagle_verify.h")).read()
    declared = set(re.findall(r"EAGLE_API\s+[\w\s\*]+?\b(eagle_verify_\w+)\s*\(", header))
    assert declared == set(ev.EXPORTED_SYMBOLS)
    lib = ev.library()
    for name in declared:
        assert hasattr(lib, name), name


def _desc(**kw):
    d = dict(max_batch=4, num_q_heads=32, num_kv_heads=8, head_dim=128, max_tree_rows=61, vocab_size=128256,
             kv_dtype="bf16", logits_dtype="bf16")
    d.update(kw)
    return ev.make_desc(**d)


def _attn_args(B=1, T=61, lens=(8192,), rows=None, **over):
    a = ev.TreeAttentionArgs()
    a.batch, a.tree_rows = B, T
    lens = np.asarray(lens, dtype=np.int32)
    a.num_kv_rows = int(rows if rows is not None else lens.sum() + B * T)
    fake = 1 << 20   # aligned non-null addresses: never dereferenced by the check
    a.q = a.k = a.v = a.out = fake
    a.kv_indptr = fake
    a.parents = a.flags = fake
    a.prefix_lens_host = lens.ctypes.data_as(C.POINTER(C.c_int32))
    a.sm_scale = 1.0 / np.sqrt(128.0)
    for k, v in over.items():
        setattr(a, k, v)
    return a, lens


def test_plan_for_the_workload_shapes():
    # 8B/8K: R = 61*4 = 244 rows per KV head -> four 64-row MFMA tiles
    a, keep = _attn_args()
    st, plan = ev.eagle_verify_check_tree_attention(_desc(), a)
    assert st == ev.EAGLE_OK
    assert plan.path == 1 and plan.rows_per_kv_head == 244
    assert plan.row_tiles == 4 and plan.rows_per_tile == 64
    assert plan.chunk_keys % 64 == 0 and plan.total_splits == -(-8192 // plan.chunk_keys)
    assert plan.workgroups == plan.total_splits * 8 * 4
    assert plan.merge_workgroups == (8 * 4 if plan.total_splits > 1 else 0)
    assert plan.merge_in_kernel == 0      # only a handle's call knows the device
    # 70B batch of four: R = 488 -> eight 64-row tiles per KV head
    a, keep = _attn_args(B=4, lens=(1024, 2048, 3072, 4096))
    st, plan = ev.eagle_verify_check_tree_attention(_desc(num_q_heads=64), a)
    assert st == ev.EAGLE_OK and plan.row_tiles == 8 and plan.rows_per_tile == 64
    # tiny fp32 goes to the FMA path, one row per workgroup
    a, keep = _attn_args(T=11, lens=(128,))
    st, plan = ev.eagle_verify_check_tree_attention(
        _desc(num_q_heads=4, num_kv_heads=4, head_dim=64, kv_dtype="f32", logits_dtype="f32"), a)
    assert st == ev.EAGLE_OK and plan.path == 0 and plan.row_tiles == 11
    # bf16 with fewer than 16 rows per KV head also takes the FMA path
    a, keep = _attn_args(T=3, lens=(300,))
    st, plan = ev.eagle_verify_check_tree_attention(_desc(num_q_heads=8, num_kv_heads=8), a)
    assert st == ev.EAGLE_OK and plan.path == 0


def test_attention_argument_errors():
    d = _desc()
    a, keep = _attn_args(T=65)
    assert ev.eagle_verify_check_tree_attention(d, a)[0] == ev.EAGLE_ERR_CAPACITY
    a, keep = _attn_args(B=5, lens=(1,) * 5)
    assert ev.eagle_verify_check_tree_attention(d, a)[0] == ev.EAGLE_ERR_CAPACITY
    a, keep = _attn_args(B=0, lens=())
    assert ev.eagle_verify_check_tree_attention(d, a)[0] == ev.EAGLE_ERR_ARG
    a, keep = _attn_args(q=None)
    assert ev.eagle_verify_check_tree_attention(d, a)[0] == ev.EAGLE_ERR_ARG
    a, keep = _attn_args(k=(1 << 20) + 8)
    assert ev.eagle_verify_check_tree_attention(d, a)[0] == ev.EAGLE_ERR_ARG
    a, keep = _attn_args(sm_scale=float("nan"))
    assert ev.eagle_verify_check_tree_attention(d, a)[0] == ev.EAGLE_ERR_ARG
    a, keep = _attn_args(lens=(-1,))
    assert ev.eagle_verify_check_tree_attention(d, a)[0] == ev.EAGLE_ERR_ARG
    a, keep = _attn_args(rows=100)
    assert ev.eagle_verify_check_tree_attention(d, a)[0] == ev.EAGLE_ERR_CAPACITY
    assert "KV rows" in ev.eagle_verify_last_error()
    assert ev.eagle_verify_check_tree_attention(_desc(head_dim=96), _attn_args()[0])[0] == \
        ev.EAGLE_ERR_UNSUPPORTED
    assert ev.eagle_verify_check_tree_attention(_desc(num_kv_heads=7), _attn_args()[0])[0] == ev.EAGLE_ERR_ARG


def _sa_args(**over):
    a = ev.SpecAcceptArgs()
    a.batch, a.tree_rows = 1, 61
    fake = 1 << 20
    a.target_logits = a.draft_logits = fake
    a.parents = a.tokens = a.accept_len = a.accepted_nodes = a.out_tokens = a.flags = a.near_ties = fake
    a.temperature, a.seed, a.offset = 1.0, 1, 0
    for k, v in over.items():
        setattr(a, k, v)
    return a


def test_last_attention_plan_needs_a_call():
    import ctypes as C
    lib = ev.library()
    plan = ev.verify.AttentionPlan()
    assert lib.eagle_verify_last_attention_plan(None, C.byref(plan)) == ev.EAGLE_ERR_ARG
    assert lib.eagle_verify_last_attention_plan(None, None) == ev.EAGLE_ERR_ARG


def test_last_accept_paths_needs_a_call():
    import ctypes as C
    lib = ev.library()
    paths = C.c_int(0)
    assert lib.eagle_verify_last_accept_paths(None, C.byref(paths)) == ev.EAGLE_ERR_ARG
    assert lib.eagle_verify_last_accept_paths(None, None) == ev.EAGLE_ERR_ARG


def test_set_timeline_needs_a_handle():
    lib = ev.library()
    assert lib.eagle_verify_set_timeline(None, None, 0) == ev.EAGLE_ERR_ARG
    assert lib.eagle_verify_set_timeline(None, 64, 32) == ev.EAGLE_ERR_ARG


def test_spec_accept_argument_errors():
    d = _desc()
    assert ev.eagle_verify_check_spec_accept(d, _sa_args()) == ev.EAGLE_OK
    assert ev.eagle_verify_check_spec_accept(d, _sa_args(temperature=-1.0)) == ev.EAGLE_ERR_ARG
    assert ev.eagle_verify_check_spec_accept(d, _sa_args(temperature=float("nan"))) == ev.EAGLE_ERR_ARG
    assert ev.eagle_verify_check_spec_accept(d, _sa_args(draft_logits=None)) == ev.EAGLE_ERR_ARG
    assert ev.eagle_verify_check_spec_accept(d, _sa_args(draft_logits=None, temperature=0.0)) == ev.EAGLE_OK
    assert ev.eagle_verify_check_spec_accept(d, _sa_args(tree_rows=62)) == ev.EAGLE_ERR_CAPACITY
    assert ev.eagle_verify_check_spec_accept(d, _sa_args(batch=9)) == ev.EAGLE_ERR_CAPACITY
    assert ev.eagle_verify_check_spec_accept(d, _sa_args(target_logits=(1 << 20) + 4)) == ev.EAGLE_ERR_ARG
    assert ev.eagle_verify_check_spec_accept(d, _sa_args(near_ties=None)) == ev.EAGLE_ERR_ARG


def _kc_args(lens=(5, 9), T=61, **over):
    a = ev.KvCommitArgs()
    lens = np.asarray(lens, dtype=np.int32)
    a.batch, a.tree_rows = len(lens), T
    a.num_kv_rows = int(lens.sum() + len(lens) * T)
    fake = 1 << 20
    a.k = a.v = a.kv_indptr = a.accept_len = a.accepted_nodes = a.new_lens = a.flags = fake
    a.prefix_lens_host = lens.ctypes.data_as(C.POINTER(C.c_int32))
    a.num_layers, a.layer_stride = 1, 0
    for k, v in over.items():
        setattr(a, k, v)
    return a, lens


def test_kv_commit_argument_errors():
    d = _desc()
    a, keep = _kc_args()
    assert ev.eagle_verify_check_kv_commit(d, a) == ev.EAGLE_OK
    for over, want in ((dict(batch=0), ev.EAGLE_ERR_ARG), (dict(batch=9), ev.EAGLE_ERR_CAPACITY),
                       (dict(tree_rows=0), ev.EAGLE_ERR_ARG), (dict(tree_rows=62), ev.EAGLE_ERR_CAPACITY),
                       (dict(num_kv_rows=-1), ev.EAGLE_ERR_ARG), (dict(k=None), ev.EAGLE_ERR_ARG),
                       (dict(new_lens=None), ev.EAGLE_ERR_ARG), (dict(v=(1 << 20) + 8), ev.EAGLE_ERR_ARG),
                       (dict(kv_indptr=(1 << 20) + 4), ev.EAGLE_ERR_ARG),
                       (dict(accepted_nodes=(1 << 20) + 2), ev.EAGLE_ERR_ARG),
                       (dict(num_layers=0), ev.EAGLE_ERR_ARG),
                       (dict(num_layers=32, layer_stride=1000), ev.EAGLE_ERR_ARG),
                       (dict(num_layers=32, layer_stride=(5 + 9 + 122) * 8 * 128 + 4), ev.EAGLE_ERR_ARG),
                       (dict(num_layers=32, layer_stride=(5 + 9 + 122) * 8 * 128), ev.EAGLE_OK)):
        a, keep = _kc_args(**over)
        assert ev.eagle_verify_check_kv_commit(d, a) == want, over
    a, keep = _kc_args(lens=(5, -1))
    assert ev.eagle_verify_check_kv_commit(d, a) == ev.EAGLE_ERR_ARG
    assert "prefix_lens_host[1]" in ev.eagle_verify_last_error()


def _te_args(**over):
    a = ev.TreeExpandArgs()
    a.batch, a.frontier = 2, 8
    fake = 1 << 20
    a.draft_logits = a.scores = a.parent = a.token = a.value = a.flags = a.near_ties = fake
    a.temperature, a.top_k, a.keep = 1.0, 8, 16
    for k, v in over.items():
        setattr(a, k, v)
    return a


def test_tree_expand_argument_errors():
    d = _desc()
    assert ev.eagle_verify_check_tree_expand(d, _te_args()) == ev.EAGLE_OK
    for over, want in ((dict(batch=0), ev.EAGLE_ERR_ARG), (dict(batch=9), ev.EAGLE_ERR_CAPACITY),
                       (dict(frontier=0), ev.EAGLE_ERR_ARG), (dict(frontier=62), ev.EAGLE_ERR_CAPACITY),
                       (dict(top_k=0), ev.EAGLE_ERR_ARG), (dict(top_k=17), ev.EAGLE_ERR_ARG),
                       (dict(keep=0), ev.EAGLE_ERR_ARG), (dict(keep=65), ev.EAGLE_ERR_ARG),
                       (dict(temperature=0.0), ev.EAGLE_ERR_ARG), (dict(temperature=float("inf")), ev.EAGLE_ERR_ARG),
                       (dict(scores=None), ev.EAGLE_ERR_ARG), (dict(value=(1 << 20) + 2), ev.EAGLE_ERR_ARG)):
        assert ev.eagle_verify_check_tree_expand(d, _te_args(**over)) == want, over
    assert ev.eagle_verify_check_tree_expand(_desc(vocab_size=64 * 8192 + 1), _te_args()) == ev.EAGLE_ERR_UNSUPPORTED


def test_tree_rerank_argument_errors():
    d = _desc()

    def args(**over):
        a = ev.TreeRerankArgs()
        a.batch, a.steps, a.keep, a.nodes = 2, 6, 8, 60
        fake = 1 << 20
        a.parent = a.token = a.value = a.root_tokens = a.parents = a.tokens = a.rows = fake
        for k, v in over.items():
            setattr(a, k, v)
        return a

    assert ev.eagle_verify_check_tree_rerank(d, args()) == ev.EAGLE_OK
    for over, want in ((dict(batch=0), ev.EAGLE_ERR_ARG), (dict(steps=0), ev.EAGLE_ERR_ARG),
                       (dict(steps=65), ev.EAGLE_ERR_ARG), (dict(keep=65), ev.EAGLE_ERR_ARG),
                       (dict(nodes=61), ev.EAGLE_ERR_CAPACITY), (dict(nodes=-1), ev.EAGLE_ERR_ARG),
                       (dict(rows=None), ev.EAGLE_ERR_ARG), (dict(tokens=(1 << 20) + 2), ev.EAGLE_ERR_ARG)):
        assert ev.eagle_verify_check_tree_rerank(d, args(**over)) == want, over


def test_descriptor_errors():
    for kw in (dict(max_batch=0), dict(max_batch=257), dict(max_tree_rows=65), dict(vocab_size=1),
               dict(num_q_heads=0)):
        assert ev.eagle_verify_check_spec_accept(_desc(**kw), _sa_args()) == ev.EAGLE_ERR_ARG, kw
    with pytest.raises(ev.EagleVerifyError) as e:
        ev.eagle_verify_create(_desc(max_batch=0))
    assert e.value.status == ev.EAGLE_ERR_ARG


def test_paged_kv_argument_errors():
    """Paged K/V (page_size > 0): a page size that is not a multiple of 64, a
    row count it does not divide, a table row too short for a sequence's
    L + T rows or a missing table are argument errors; kv_indptr may be NULL."""
    d = _desc()
    fake = 1 << 20
    rows = 64 * 200                                      # 8192 + 61 rows need 129 pages of 64
    ok = dict(page_table=fake, page_size=64, pages_per_seq=129, kv_indptr=None, rows=rows)
    a, keep = _attn_args(**ok)
    st, _ = ev.eagle_verify_check_tree_attention(d, a)
    assert st == ev.EAGLE_OK, ev.eagle_verify_last_error()
    for over in (dict(page_size=96), dict(page_size=-64), dict(pages_per_seq=128), dict(page_table=None),
                 dict(rows=rows + 1), dict(page_table=fake + 2)):
        a, keep = _attn_args(**{**ok, **over})
        assert ev.eagle_verify_check_tree_attention(d, a)[0] == ev.EAGLE_ERR_ARG, over
    a, keep = _attn_args(**{**ok, "page_size": 0})        # contiguous again: kv_indptr is required
    assert ev.eagle_verify_check_tree_attention(d, a)[0] == ev.EAGLE_ERR_ARG
    # the KV commit: T = 61 rows behind prefixes 5 and 9 need one page of 128 each
    a, keep = _kc_args(page_table=fake, page_size=128, pages_per_seq=1, kv_indptr=None)
    a.num_kv_rows = 128 * 4
    assert ev.eagle_verify_check_kv_commit(d, a) == ev.EAGLE_OK, ev.eagle_verify_last_error()
    a.page_size = 64
    assert ev.eagle_verify_check_kv_commit(d, a) == ev.EAGLE_ERR_ARG


def test_spec_accept_noalloc_rejects_before_any_launch():
    """Argument and capacity errors come back without touching the device."""
    from eagle_draft_tree_attention_amd import verify
    d = _desc(max_batch=64, max_tree_rows=64, vocab_size=128256)
    a = _sa_args(batch=64, tree_rows=64)
    lib = ev.library()
    st = lib.eagle_verify_spec_accept_noalloc(C.byref(d), C.byref(a), None)
    assert st == ev.EAGLE_ERR_CAPACITY
    assert "scratch" in verify.eagle_verify_last_error()
    assert lib.eagle_verify_spec_accept_noalloc(C.byref(d), C.byref(_sa_args(near_ties=None)), None) == \
        ev.EAGLE_ERR_ARG
    bad = _desc(vocab_size=1)
    assert lib.eagle_verify_spec_accept_noalloc(C.byref(bad), C.byref(_sa_args()), None) == ev.EAGLE_ERR_ARG
