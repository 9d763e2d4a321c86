"""The bounded waits of the self-synchronising kernels (the fused acceptance
kernel, tree attention with its split merge inside), through the C ABI.

With the host-side spin limit forced to 0 (EAGLE_VERIFY_SPIN_LIMIT, read
when a handle is created) a wait that is not satisfied at its first poll
gives up.  Every kernel must still finish, and every sequence must come back
either flagged EAGLE_FLAG_INTERNAL with poisoned outputs (-1 integers, NaN
attention rows) or with exactly the oracle's result.  A handle created
afterwards with the normal limit must give the oracle's results again."""
import numpy as np
import pytest

import synth
from gpu_util import (ATTN_TOL, FLAGS_SENTINEL, compare_accept, dev, log, make_verifier, row_error, run_attention,
                      sentinel_accept_outputs, small_spec)
from oracle import accept as oacc
from oracle import attention as oa

pytestmark = pytest.mark.gpu

SEED = 0x5EED0000
INTERNAL = 64


def test_acceptance_waits_that_give_up(monkeypatch):
    import torch
    spec = small_spec("waits_accept", B=8, V=20000, levels=(10, 10, 10))
    inp = synth.make_inputs(spec, with_kv=False)
    monkeypatch.setenv("EAGLE_VERIFY_SPIN_LIMIT", "0")
    # the fused kernel's waits (the node-parallel kernels, which never wait,
    # are kept out)
    monkeypatch.setenv("EAGLE_VERIFY_NODE_PARALLEL", "0")
    ver = make_verifier(spec, inp.T)
    B, T = inp.parents.shape
    internal = 0
    for off in range(3):
        log(f"[waits] acceptance with spin limit 0, offset {off}")
        outs = sentinel_accept_outputs(B, T)
        ver.spec_accept(dev(inp.target, "bf16"), dev(inp.draft, "bf16"), dev(inp.parents), dev(inp.tokens), 1.0,
                        SEED, off, outputs=outs)
        torch.cuda.synchronize()
        got = {k: v.cpu().numpy() for k, v in outs.items()}
        got["flags"] = got["flags"].astype(np.uint32)
        ref = oacc.spec_accept(inp.target64(), inp.draft64(), inp.parents, inp.tokens, 1.0, SEED, off)
        for b in range(B):
            if got["flags"][b] & INTERNAL:
                internal += 1
                assert got["accept_len"][b] == -1 and (got["accepted_nodes"][b] == -1).all() and \
                    (got["out_tokens"][b] == -1).all(), f"seq {b}: flagged but not poisoned"
            else:
                one = {k: v[b:b + 1] for k, v in got.items()}
                want = {k: v[b:b + 1] for k, v in ref.items()}
                assert compare_accept(one, want, f"seq {b}", inp.parents[b:b + 1], inp.tokens[b:b + 1],
                                      spec.vocab) == 0
    log(f"    sequences that gave up: {internal} of {3 * B}")
    assert internal > 0
    ver.close()
    monkeypatch.delenv("EAGLE_VERIFY_SPIN_LIMIT")
    ver = make_verifier(spec, inp.T)
    from gpu_util import run_accept
    got = run_accept(ver, inp, 1.0, SEED, 0)
    ref = oacc.spec_accept(inp.target64(), inp.draft64(), inp.parents, inp.tokens, 1.0, SEED, 0)
    assert compare_accept(got, ref, "after", inp.parents, inp.tokens, spec.vocab) <= 1
    ver.close()


def test_attention_merge_waits_that_give_up(monkeypatch):
    spec = small_spec("waits_attn", B=2, Hq=32, Hkv=8, lens=(2048, 2048), levels=(10,) * 6)
    inp = synth.make_inputs(spec, with_logits=False)
    scale = 1.0 / np.sqrt(spec.head_dim)
    ref, _ = oa.tree_attention(inp.q64(), inp.k64(), inp.v64(), inp.kv_indptr, inp.prefix_lens, inp.parents, scale)
    monkeypatch.setenv("EAGLE_VERIFY_SPIN_LIMIT", "0")
    ver = make_verifier(spec, inp.T)
    log("[waits] attention with spin limit 0")
    got, flags = run_attention(ver, inp)   # every output row written (NaN or a result)
    plan = ver.last_attention_plan()
    assert plan.merge_in_kernel == 1 and plan.total_splits > spec.batch
    ver.close()
    nan_rows = np.isnan(got).all(axis=-1)
    assert not (np.isnan(got).any(axis=-1) & ~nan_rows).any(), "a row partly NaN"
    ok = ~nan_rows
    assert (row_error(got[ok], ref[ok]) <= ATTN_TOL["bf16"]).all()
    assert ((flags & ~np.uint32(INTERNAL)) == 0).all()
    log(f"    rows poisoned: {int(nan_rows.sum())} of {nan_rows.size}; flags {flags.tolist()}")
    assert nan_rows.any() or (flags & INTERNAL).any()
    monkeypatch.delenv("EAGLE_VERIFY_SPIN_LIMIT")
    ver = make_verifier(spec, inp.T)
    got, flags = run_attention(ver, inp)
    ver.close()
    assert (flags == 0).all() and row_error(got, ref).max() <= ATTN_TOL["bf16"]
    assert FLAGS_SENTINEL


def test_cooperative_launches_match_the_oracle(monkeypatch):
    """EAGLE_VERIFY_COOPERATIVE=1: the two self-synchronising kernels are
    launched cooperatively (every workgroup resident, or the launch is
    refused and the non-waiting paths run); results as without it."""
    from gpu_util import run_accept
    monkeypatch.setenv("EAGLE_VERIFY_COOPERATIVE", "1")
    spec = small_spec("coop", B=2, Hq=32, Hkv=8, lens=(2048, 2048), levels=(10,) * 6, V=20000)
    inp = synth.make_inputs(spec)
    ver = make_verifier(spec, inp.T)
    log("[waits] cooperative launches")
    got, flags = run_attention(ver, inp)
    assert ver.last_attention_plan().merge_in_kernel == 1
    scale = 1.0 / np.sqrt(spec.head_dim)
    ref, _ = oa.tree_attention(inp.q64(), inp.k64(), inp.v64(), inp.kv_indptr, inp.prefix_lens, inp.parents, scale)
    assert (flags == 0).all() and row_error(got, ref).max() <= ATTN_TOL["bf16"]
    for off in range(3):
        acc = run_accept(ver, inp, 1.0, SEED, off)
        want = oacc.spec_accept(inp.target64(), inp.draft64(), inp.parents, inp.tokens, 1.0, SEED, off)
        assert compare_accept(acc, want, f"cooperative offset {off}", inp.parents, inp.tokens, spec.vocab) <= 1
    ver.close()
