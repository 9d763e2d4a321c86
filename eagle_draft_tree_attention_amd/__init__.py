"""Python binding of libeagle_verify (EAGLE draft-tree verification on MI355X).

A thin ctypes layer over the C ABI in include/eagle_verify.h: the functions
below carry the C names and only marshal arguments (device pointers, sizes,
the caller's stream).  Every step of the computation runs in the HIP kernels
of the library; torch is used for device memory and streams only.

Importing this package fails loudly if the library has not been built
(python eagle_draft_tree_attention_amd/build.py).
"""
import ctypes
import os

from ._abi import (  # noqa: F401
    EAGLE_OK, EAGLE_ERR_ARG, EAGLE_ERR_UNSUPPORTED, EAGLE_ERR_CAPACITY, EAGLE_ERR_HIP, EAGLE_ERR_OOM,
    EAGLE_F32, EAGLE_BF16, FLAG_BAD_TREE, FLAG_BAD_TOKEN, FLAG_NONFINITE, FLAG_P_ZERO,
    FLAG_DEGENERATE_RESIDUAL, FLAG_BAD_KV_RANGE, MAX_TREE_ROWS, EXPORTED_SYMBOLS,
    VerifyDesc, TreeAttentionArgs, SpecAcceptArgs, KvCommitArgs, TreeExpandArgs, TreeRerankArgs,
    AttentionPlan, EagleVerifyError,
)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libeagle_verify.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python eagle_draft_tree_attention_amd/build.py); there is no fallback path")

# torch ships its own HIP runtime (same SONAME as the system one).  Load it
# first so the library binds to the runtime torch's tensors and streams live
# in: one process must not carry two HIP runtimes.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

from . import _abi  # noqa: E402

_abi.bind(_lib)

from .verify import (  # noqa: E402,F401
    eagle_verify_create, eagle_verify_destroy, eagle_verify_tree_attention, eagle_verify_spec_accept,
    eagle_verify_last_error, eagle_verify_check_tree_attention, eagle_verify_check_spec_accept,
    eagle_verify_last_attention_plan, eagle_verify_last_accept_paths, eagle_verify_kv_commit, eagle_verify_check_kv_commit,
    eagle_verify_tree_expand, eagle_verify_check_tree_expand, eagle_verify_tree_rerank,
    eagle_verify_check_tree_rerank, eagle_verify_set_timeline, Verifier, make_desc,
    ACCEPT_PATH_THREE_KERNEL, ACCEPT_PATH_FUSED, ACCEPT_PATH_NODE_PARALLEL,
)


def library():
    """The loaded ctypes library (for symbol checks)."""
    return _lib
