"""Argument marshalling for the libeagle_verify entry points.

The functions named like the C entry points take plain integers (device
addresses, host arrays, a stream handle) and return the C status, raising
EagleVerifyError on failure.  `Verifier` wraps a handle and accepts torch
tensors that already live on the GPU; it allocates the output tensors when
none are given.  No computation happens here.
"""
import ctypes as C

import numpy as np

from . import _abi
from ._abi import (EAGLE_BF16, EAGLE_F32, EagleVerifyError, KvCommitArgs, SpecAcceptArgs, TreeAttentionArgs,
                   TreeExpandArgs, TreeRerankArgs, VerifyDesc, AttentionPlan)


def _lib():
    from . import _lib as lib
    return lib


def _check(status, handle=None):
    if status != _abi.EAGLE_OK:
        msg = _lib().eagle_verify_last_error(handle)
        raise EagleVerifyError(status, (msg or b"").decode(errors="replace"))
    return status


def make_desc(max_batch, num_q_heads, num_kv_heads, head_dim, max_tree_rows, vocab_size,
              kv_dtype="bf16", logits_dtype="bf16") -> VerifyDesc:
    dt = {"bf16": EAGLE_BF16, "f32": EAGLE_F32}
    return VerifyDesc(int(max_batch), int(num_q_heads), int(num_kv_heads), int(head_dim),
                      int(max_tree_rows), int(vocab_size), dt[kv_dtype], dt[logits_dtype])


# ---------------------------------------------------------------- C names
def eagle_verify_create(desc: VerifyDesc) -> int:
    h = C.c_void_p()
    _check(_lib().eagle_verify_create(C.byref(desc), C.byref(h)))
    return h.value


def eagle_verify_destroy(handle: int) -> None:
    _check(_lib().eagle_verify_destroy(handle))


def eagle_verify_last_error(handle=None) -> str:
    return (_lib().eagle_verify_last_error(handle) or b"").decode(errors="replace")


def eagle_verify_tree_attention(handle: int, args: TreeAttentionArgs, stream: int) -> int:
    return _check(_lib().eagle_verify_tree_attention(handle, C.byref(args), C.c_void_p(stream)), handle)


def eagle_verify_spec_accept(handle: int, args: SpecAcceptArgs, stream: int) -> int:
    return _check(_lib().eagle_verify_spec_accept(handle, C.byref(args), C.c_void_p(stream)), handle)


def eagle_verify_spec_accept_noalloc(desc: VerifyDesc, args: SpecAcceptArgs, stream: int) -> int:
    return _check(_lib().eagle_verify_spec_accept_noalloc(C.byref(desc), C.byref(args), C.c_void_p(stream)))


def eagle_verify_kv_commit(handle: int, args: KvCommitArgs, stream: int) -> int:
    return _check(_lib().eagle_verify_kv_commit(handle, C.byref(args), C.c_void_p(stream)), handle)


def eagle_verify_check_kv_commit(desc: VerifyDesc, args: KvCommitArgs) -> int:
    return _lib().eagle_verify_check_kv_commit(C.byref(desc), C.byref(args))


def eagle_verify_tree_expand(handle: int, args: TreeExpandArgs, stream: int) -> int:
    return _check(_lib().eagle_verify_tree_expand(handle, C.byref(args), C.c_void_p(stream)), handle)


def eagle_verify_check_tree_expand(desc: VerifyDesc, args: TreeExpandArgs) -> int:
    return _lib().eagle_verify_check_tree_expand(C.byref(desc), C.byref(args))


def eagle_verify_tree_rerank(handle: int, args: TreeRerankArgs, stream: int) -> int:
    return _check(_lib().eagle_verify_tree_rerank(handle, C.byref(args), C.c_void_p(stream)), handle)


def eagle_verify_check_tree_rerank(desc: VerifyDesc, args: TreeRerankArgs) -> int:
    return _lib().eagle_verify_check_tree_rerank(C.byref(desc), C.byref(args))


def eagle_verify_check_tree_attention(desc: VerifyDesc, args: TreeAttentionArgs):
    """(status, AttentionPlan) without touching the device."""
    plan = AttentionPlan()
    st = _lib().eagle_verify_check_tree_attention(C.byref(desc), C.byref(args), C.byref(plan))
    return st, plan


def eagle_verify_check_spec_accept(desc: VerifyDesc, args: SpecAcceptArgs) -> int:
    return _lib().eagle_verify_check_spec_accept(C.byref(desc), C.byref(args))


def eagle_verify_last_attention_plan(handle: int) -> AttentionPlan:
    """Plan of the handle's last successful tree-attention call."""
    plan = AttentionPlan()
    _check(_lib().eagle_verify_last_attention_plan(handle, C.byref(plan)), handle)
    return plan


# kernels of a spec_accept call (bits of eagle_verify_last_accept_paths)
ACCEPT_PATH_THREE_KERNEL, ACCEPT_PATH_FUSED, ACCEPT_PATH_NODE_PARALLEL = 1, 2, 4


def eagle_verify_last_accept_paths(handle: int) -> int:
    """ACCEPT_PATH_* bits of the handle's last successful spec_accept call."""
    paths = C.c_int(0)
    _check(_lib().eagle_verify_last_accept_paths(handle, C.byref(paths)), handle)
    return paths.value


# ---------------------------------------------------------------- torch layer
def eagle_verify_set_timeline(handle: int, device_words: int, num_words: int) -> int:
    return _check(_lib().eagle_verify_set_timeline(handle, device_words, num_words), handle)


def _ptr(t):
    return None if t is None else int(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _paging(a, page_table, page_size):
    """page_table: [B, pages_per_seq] int32 device tensor (paged K/V), or None."""
    if page_table is None:
        a.page_table, a.page_size, a.pages_per_seq = None, 0, 0
    else:
        a.page_table = _ptr(page_table)
        a.page_size, a.pages_per_seq = int(page_size), int(page_table.shape[1])


def tree_attention_args(q, k, v, kv_indptr, prefix_lens, parents, sm_scale, out, flags, page_table=None,
                        page_size=0):
    lens = np.ascontiguousarray(np.asarray(prefix_lens, dtype=np.int32))
    a = TreeAttentionArgs()
    a.batch, a.tree_rows = int(q.shape[0]), int(q.shape[1])
    a.num_kv_rows = int(k.shape[0])
    a.q, a.k, a.v = _ptr(q), _ptr(k), _ptr(v)
    a.kv_indptr = None if kv_indptr is None else _ptr(kv_indptr)
    a.prefix_lens_host = lens.ctypes.data_as(C.POINTER(C.c_int32))
    a.parents = _ptr(parents)
    a.sm_scale = float(sm_scale)
    a.out, a.flags = _ptr(out), _ptr(flags)
    _paging(a, page_table, page_size)
    return a, lens          # keep lens alive while the call runs


def kv_commit_args(k, v, kv_indptr, prefix_lens, accept_len, accepted_nodes, new_lens, flags, page_table=None,
                   page_size=0):
    """k, v: [rows, Hkv, D] (one layer) or [layers, rows, Hkv, D] (every layer, contiguous)."""
    lens = np.ascontiguousarray(np.asarray(prefix_lens, dtype=np.int32))
    a = KvCommitArgs()
    a.batch, a.tree_rows = int(accepted_nodes.shape[0]), int(accepted_nodes.shape[1])
    if k.dim() == 4:
        a.num_layers, a.layer_stride = int(k.shape[0]), int(k.stride(0))
        a.num_kv_rows = int(k.shape[1])
    else:
        a.num_layers, a.layer_stride = 1, 0
        a.num_kv_rows = int(k.shape[0])
    a.k, a.v = _ptr(k), _ptr(v)
    a.kv_indptr = None if kv_indptr is None else _ptr(kv_indptr)
    a.prefix_lens_host = lens.ctypes.data_as(C.POINTER(C.c_int32))
    a.accept_len, a.accepted_nodes = _ptr(accept_len), _ptr(accepted_nodes)
    a.new_lens, a.flags = _ptr(new_lens), _ptr(flags)
    _paging(a, page_table, page_size)
    return a, lens          # keep lens alive while the call runs


class Verifier:
    """One handle (one stream at a time).  Tensors must be CUDA/HIP tensors."""

    def __init__(self, max_batch, num_q_heads, num_kv_heads, head_dim, max_tree_rows, vocab_size,
                 kv_dtype="bf16", logits_dtype="bf16"):
        self.desc = make_desc(max_batch, num_q_heads, num_kv_heads, head_dim, max_tree_rows, vocab_size,
                              kv_dtype, logits_dtype)
        self.handle = eagle_verify_create(self.desc)

    def close(self):
        if self.handle:
            eagle_verify_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def tree_attention(self, q, k, v, kv_indptr, prefix_lens, parents, sm_scale=None, out=None,
                       flags=None, stream=None, page_table=None, page_size=0):
        """kv_indptr [B+1] int64 for contiguous K/V; or page_table [B, pages_per_seq]
        int32 with page_size rows per page (kv_indptr may be None)."""
        import torch
        B, T, Hq, D = q.shape
        if sm_scale is None:
            sm_scale = 1.0 / float(D) ** 0.5
        if out is None:
            out = torch.empty((B, T, Hq, D), dtype=torch.float32, device=q.device)
        if flags is None:
            flags = torch.empty((B,), dtype=torch.int32, device=q.device)
        a, _keep = tree_attention_args(q, k, v, kv_indptr, prefix_lens, parents, sm_scale, out, flags,
                                       page_table, page_size)
        eagle_verify_tree_attention(self.handle, a, _stream(stream))
        return out, flags

    def last_attention_plan(self) -> AttentionPlan:
        return eagle_verify_last_attention_plan(self.handle)

    def last_accept_paths(self) -> int:
        return eagle_verify_last_accept_paths(self.handle)

    def set_timeline(self, words=None):
        """Diagnostic phase timeline: a contiguous int64 device tensor (32
        words per workgroup), or None to switch it off."""
        if words is None:
            return eagle_verify_set_timeline(self.handle, None, 0)
        assert words.is_contiguous() and words.element_size() == 8
        return eagle_verify_set_timeline(self.handle, words.data_ptr(), words.numel())

    def spec_accept(self, target, draft, parents, tokens, temperature, seed, offset, outputs=None,
                    stream=None, without_replacement=False, top_k=0, top_p=0.0):
        import torch
        B, T, V = target.shape
        dev = target.device
        if outputs is None:
            outputs = {
                "accept_len": torch.empty((B,), dtype=torch.int32, device=dev),
                "accepted_nodes": torch.empty((B, T), dtype=torch.int32, device=dev),
                "out_tokens": torch.empty((B, T), dtype=torch.int32, device=dev),
                "flags": torch.empty((B,), dtype=torch.int32, device=dev),
                "near_ties": torch.empty((B,), dtype=torch.int32, device=dev),
            }
        a = SpecAcceptArgs()
        a.batch, a.tree_rows = int(B), int(T)
        a.target_logits, a.draft_logits = _ptr(target), _ptr(draft)
        a.parents, a.tokens = _ptr(parents), _ptr(tokens)
        a.temperature = float(temperature)
        a.seed, a.offset = int(seed), int(offset)
        a.accept_len = _ptr(outputs["accept_len"])
        a.accepted_nodes = _ptr(outputs["accepted_nodes"])
        a.out_tokens = _ptr(outputs["out_tokens"])
        a.flags = _ptr(outputs["flags"])
        a.near_ties = _ptr(outputs["near_ties"])
        a.without_replacement = 1 if without_replacement else 0
        a.top_k, a.top_p = int(top_k), float(top_p)
        eagle_verify_spec_accept(self.handle, a, _stream(stream))
        return outputs

    def kv_commit(self, k, v, kv_indptr, prefix_lens, accept_len, accepted_nodes, new_lens=None, flags=None,
                  stream=None, page_table=None, page_size=0):
        """Commit the accepted path into k and v in place; returns (new_lens, flags)."""
        import torch
        B = int(accepted_nodes.shape[0])
        if new_lens is None:
            new_lens = torch.empty((B,), dtype=torch.int32, device=k.device)
        if flags is None:
            flags = torch.empty((B,), dtype=torch.int32, device=k.device)
        a, _keep = kv_commit_args(k, v, kv_indptr, prefix_lens, accept_len, accepted_nodes, new_lens, flags,
                                  page_table, page_size)
        eagle_verify_kv_commit(self.handle, a, _stream(stream))
        return new_lens, flags

    def tree_expand(self, logits, scores, temperature, top_k, keep, outputs=None, stream=None):
        """One dynamic draft-tree expansion step: logits [B, F, V], scores [B, F] float32."""
        import torch
        B, F = int(logits.shape[0]), int(logits.shape[1])
        dev = logits.device
        if outputs is None:
            outputs = {
                "parent": torch.empty((B, keep), dtype=torch.int32, device=dev),
                "token": torch.empty((B, keep), dtype=torch.int32, device=dev),
                "value": torch.empty((B, keep), dtype=torch.float32, device=dev),
                "flags": torch.empty((B,), dtype=torch.int32, device=dev),
                "near_ties": torch.empty((B,), dtype=torch.int32, device=dev),
            }
        a = TreeExpandArgs()
        a.batch, a.frontier = B, F
        a.draft_logits, a.scores = _ptr(logits), _ptr(scores)
        a.temperature, a.top_k, a.keep = float(temperature), int(top_k), int(keep)
        a.parent, a.token, a.value = _ptr(outputs["parent"]), _ptr(outputs["token"]), _ptr(outputs["value"])
        a.flags, a.near_ties = _ptr(outputs["flags"]), _ptr(outputs["near_ties"])
        eagle_verify_tree_expand(self.handle, a, _stream(stream))
        return outputs

    def tree_rerank(self, parent, token, value, root_tokens, nodes, stream=None):
        """Final tree from chained expansion steps: parent/token/value [steps, B, keep]."""
        import torch
        D, B, M = (int(x) for x in parent.shape)
        dev = parent.device
        out = {"parents": torch.empty((B, nodes + 1), dtype=torch.int32, device=dev),
               "tokens": torch.empty((B, nodes + 1), dtype=torch.int32, device=dev),
               "rows": torch.empty((B,), dtype=torch.int32, device=dev)}
        a = TreeRerankArgs()
        a.batch, a.steps, a.keep, a.nodes = B, D, M, int(nodes)
        a.parent, a.token, a.value, a.root_tokens = _ptr(parent), _ptr(token), _ptr(value), _ptr(root_tokens)
        a.parents, a.tokens, a.rows = _ptr(out["parents"]), _ptr(out["tokens"]), _ptr(out["rows"])
        eagle_verify_tree_rerank(self.handle, a, _stream(stream))
        return out
