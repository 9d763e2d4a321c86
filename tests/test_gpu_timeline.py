"""The diagnostic phase timeline (eagle_verify_set_timeline), through the C
ABI: calls with a timeline buffer set give exactly the results of calls
without one, and every workgroup's marks are in phase order."""
import numpy as np
import pytest

import synth
from gpu_util import compare_accept, log, make_verifier, run_accept, run_attention, small_spec
from oracle import accept as oacc

pytestmark = pytest.mark.gpu

SLOTS = 32


def _ordered(w, marks):
    """Each workgroup's reached marks (nonzero words) never go back in time."""
    for row in w:
        seen = [row[k] for k in marks if row[k] != 0]
        assert all(x <= y for x, y in zip(seen, seen[1:])), row[:24]


def test_timeline_leaves_results_unchanged():
    import torch
    spec = small_spec("timeline", B=2, Hq=16, Hkv=4, lens=(1500, 700), levels=(4, 6, 10), V=20000)
    inp = synth.make_inputs(spec)
    ver = make_verifier(spec, inp.T)
    log("[timeline] attention and acceptance without a timeline")
    ref_o, ref_f = run_attention(ver, inp)
    ref_a = run_accept(ver, inp, 1.0, 0x5EED0000, 3)
    plan = ver.last_attention_plan()
    assert plan.path == 1 and plan.merge_in_kernel == 1
    words = torch.zeros(1 << 16, dtype=torch.int64, device="cuda")
    ver.set_timeline(words)
    log("[timeline] attention with the timeline")
    got_o, got_f = run_attention(ver, inp)
    assert np.array_equal(got_o, ref_o) and np.array_equal(got_f, ref_f)
    w = words[: plan.workgroups * SLOTS].view(-1, SLOTS).cpu().numpy()
    assert (w[:, :5] > 0).all(), "a workgroup missed an attention mark"
    _ordered(w, range(8))
    assert (w[:, 30] >= 1).all()
    words.zero_()
    log("[timeline] acceptance with the timeline")
    got_a = run_accept(ver, inp, 1.0, 0x5EED0000, 3)
    for k in ref_a:
        assert np.array_equal(got_a[k], ref_a[k]), k
    T = inp.T
    NC = (spec.vocab + 8191) // 8192
    w = words[: spec.batch * T * NC * SLOTS].view(-1, SLOTS).cpu().numpy()
    assert (w[:, :5] > 0).all(), "a workgroup missed an acceptance mark"
    _ordered(w, [0, 1, 2, 3, 4] + list(range(5, 17)) + [17, 18, 19, 20, 21])
    # one workgroup per sequence writes the outputs
    assert int((w[:, 21] > 0).sum()) == spec.batch
    ref = oacc.spec_accept(inp.target64(), inp.draft64(), inp.parents, inp.tokens, 1.0, 0x5EED0000, 3)
    diverged = compare_accept(got_a, ref, "timeline", inp.parents, inp.tokens, spec.vocab)
    assert diverged <= 1
    ver.set_timeline(None)
    ver.close()
