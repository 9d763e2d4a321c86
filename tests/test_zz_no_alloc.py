"""The acceptance entry point that allocates nothing
(eagle_verify_spec_accept_noalloc, its scratch in a static device array)
against the handle-based eagle_verify_spec_accept, through the C ABI: two
calls in a row, the second on a smaller batch, tree and temperature; every
output identical."""
import numpy as np
import pytest

import synth
from gpu_util import dev, host_accept, log, sentinel_accept_outputs, small_spec

pytestmark = pytest.mark.gpu

SEED = 0x5EED0000


def _args(ev, tgt, drf, par, tok, temp, offset, outs, without_replacement=False):
    a = ev.SpecAcceptArgs()
    a.batch, a.tree_rows = int(tgt.shape[0]), int(tgt.shape[1])
    a.target_logits, a.draft_logits = tgt.data_ptr(), drf.data_ptr()
    a.parents, a.tokens = par.data_ptr(), tok.data_ptr()
    a.temperature = float(temp)
    a.seed, a.offset = SEED, int(offset)
    for name in ("accept_len", "accepted_nodes", "out_tokens", "flags", "near_ties"):
        setattr(a, name, outs[name].data_ptr())
    a.without_replacement = 1 if without_replacement else 0
    return a


def _both(ev, ver, spec, inp, temp, offset):
    import torch
    tgt, drf = dev(inp.target, spec.ldtype), dev(inp.draft, spec.ldtype)
    par, tok = dev(inp.parents), dev(inp.tokens)
    B, T = inp.parents.shape
    stream = int(torch.cuda.current_stream().cuda_stream)
    ref_out, new_out = sentinel_accept_outputs(B, T), sentinel_accept_outputs(B, T)
    ev.verify.eagle_verify_spec_accept(ver.handle, _args(ev, tgt, drf, par, tok, temp, offset, ref_out), stream)
    ev.verify.eagle_verify_spec_accept_noalloc(ver.desc, _args(ev, tgt, drf, par, tok, temp, offset, new_out), stream)
    torch.cuda.synchronize()
    return host_accept(ref_out), host_accept(new_out)


def test_noalloc_matches_the_handle_entry_point_twice():
    import eagle_draft_tree_attention_amd as ev
    big = small_spec("noalloc_big", B=6, V=20000, levels=(10, 10, 10, 10), sigma_d=1.0)
    small = small_spec("noalloc_small", B=2, V=20000, levels=(4, 6), sigma_d=1.0)
    ver = ev.Verifier(6, 8, 8, 128, 41, 20000, kv_dtype="bf16", logits_dtype="bf16")
    for spec, temp, off in ((big, 1.0, 3), (small, 0.7, 4), (small, 0.0, 5)):
        log(f"[noalloc] {spec.name} temperature {temp}")
        inp = synth.make_inputs(spec, with_kv=False)
        ref, got = _both(ev, ver, spec, inp, temp, off)
        for key in ref:
            assert np.array_equal(ref[key], got[key]), (spec.name, key)
        assert (ref["accept_len"] >= 0).all()
    ver.close()


def test_noalloc_fused_slices_and_workload_shape():
    """The 8B workload's shape (one 61-row tree over 128256 tokens) and a
    batch verified in several fused slices."""
    import eagle_draft_tree_attention_amd as ev
    for spec in (synth.config_spec(2), small_spec("noalloc_slices", B=24, V=32000, levels=(10,) * 6)):
        log(f"[noalloc] {spec.name}")
        inp = synth.make_inputs(spec, with_kv=False)
        ver = ev.Verifier(spec.batch, 8, 8, 128, inp.T, spec.vocab, kv_dtype="bf16", logits_dtype="bf16")
        for off in range(2):
            ref, got = _both(ev, ver, spec, inp, spec.temperature, off)
            for key in ref:
                assert np.array_equal(ref[key], got[key]), (spec.name, key)
        ver.close()
