"""ctypes mirror of include/eagle_verify.h (structs, constants, prototypes)."""
import ctypes as C

EAGLE_OK, EAGLE_ERR_ARG, EAGLE_ERR_UNSUPPORTED, EAGLE_ERR_CAPACITY, EAGLE_ERR_HIP, EAGLE_ERR_OOM = range(6)
EAGLE_F32, EAGLE_BF16 = 0, 1

FLAG_BAD_TREE = 1
FLAG_BAD_TOKEN = 2
FLAG_NONFINITE = 4
FLAG_P_ZERO = 8
FLAG_DEGENERATE_RESIDUAL = 16
FLAG_BAD_KV_RANGE = 32
MAX_TREE_ROWS = 64

STATUS_NAMES = {0: "EAGLE_OK", 1: "EAGLE_ERR_ARG", 2: "EAGLE_ERR_UNSUPPORTED", 3: "EAGLE_ERR_CAPACITY",
                4: "EAGLE_ERR_HIP", 5: "EAGLE_ERR_OOM"}

EXPORTED_SYMBOLS = (
    "eagle_verify_create", "eagle_verify_tree_attention", "eagle_verify_spec_accept",
    "eagle_verify_destroy", "eagle_verify_last_error", "eagle_verify_check_tree_attention",
    "eagle_verify_check_spec_accept", "eagle_verify_last_attention_plan", "eagle_verify_last_accept_paths", "eagle_verify_kv_commit",
    "eagle_verify_check_kv_commit", "eagle_verify_tree_expand", "eagle_verify_check_tree_expand",
    "eagle_verify_tree_rerank", "eagle_verify_check_tree_rerank", "eagle_verify_spec_accept_noalloc",
    "eagle_verify_set_timeline",
)


class VerifyDesc(C.Structure):
    _fields_ = [("max_batch", C.c_int32), ("num_q_heads", C.c_int32), ("num_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("max_tree_rows", C.c_int32), ("vocab_size", C.c_int32),
                ("kv_dtype", C.c_int), ("logits_dtype", C.c_int)]


class TreeAttentionArgs(C.Structure):
    _fields_ = [("batch", C.c_int32), ("tree_rows", C.c_int32), ("num_kv_rows", C.c_int64),
                ("q", C.c_void_p), ("k", C.c_void_p), ("v", C.c_void_p),
                ("kv_indptr", C.c_void_p), ("prefix_lens_host", C.POINTER(C.c_int32)),
                ("parents", C.c_void_p), ("sm_scale", C.c_float), ("out", C.c_void_p),
                ("flags", C.c_void_p), ("page_table", C.c_void_p), ("page_size", C.c_int32),
                ("pages_per_seq", C.c_int32)]


class SpecAcceptArgs(C.Structure):
    _fields_ = [("batch", C.c_int32), ("tree_rows", C.c_int32),
                ("target_logits", C.c_void_p), ("draft_logits", C.c_void_p),
                ("parents", C.c_void_p), ("tokens", C.c_void_p), ("temperature", C.c_float),
                ("seed", C.c_uint64), ("offset", C.c_uint64),
                ("accept_len", C.c_void_p), ("accepted_nodes", C.c_void_p), ("out_tokens", C.c_void_p),
                ("flags", C.c_void_p), ("near_ties", C.c_void_p), ("without_replacement", C.c_int32),
                ("top_k", C.c_int32), ("top_p", C.c_float)]


class KvCommitArgs(C.Structure):
    _fields_ = [("batch", C.c_int32), ("tree_rows", C.c_int32), ("num_kv_rows", C.c_int64),
                ("k", C.c_void_p), ("v", C.c_void_p), ("kv_indptr", C.c_void_p),
                ("prefix_lens_host", C.POINTER(C.c_int32)), ("accept_len", C.c_void_p),
                ("accepted_nodes", C.c_void_p), ("new_lens", C.c_void_p), ("flags", C.c_void_p),
                ("num_layers", C.c_int32), ("layer_stride", C.c_int64),
                ("page_table", C.c_void_p), ("page_size", C.c_int32), ("pages_per_seq", C.c_int32)]


class TreeExpandArgs(C.Structure):
    _fields_ = [("batch", C.c_int32), ("frontier", C.c_int32), ("draft_logits", C.c_void_p),
                ("scores", C.c_void_p), ("temperature", C.c_float), ("top_k", C.c_int32), ("keep", C.c_int32),
                ("parent", C.c_void_p), ("token", C.c_void_p), ("value", C.c_void_p), ("flags", C.c_void_p),
                ("near_ties", C.c_void_p)]


class TreeRerankArgs(C.Structure):
    _fields_ = [("batch", C.c_int32), ("steps", C.c_int32), ("keep", C.c_int32), ("nodes", C.c_int32),
                ("parent", C.c_void_p), ("token", C.c_void_p), ("value", C.c_void_p), ("root_tokens", C.c_void_p),
                ("parents", C.c_void_p), ("tokens", C.c_void_p), ("rows", C.c_void_p)]


class AttentionPlan(C.Structure):
    _fields_ = [("path", C.c_int32), ("rows_per_kv_head", C.c_int32), ("row_tiles", C.c_int32),
                ("rows_per_tile", C.c_int32), ("chunk_keys", C.c_int32), ("total_splits", C.c_int32),
                ("workgroups", C.c_int32), ("merge_workgroups", C.c_int32), ("merge_in_kernel", C.c_int32)]


class EagleVerifyError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def bind(lib):
    H = C.c_void_p
    lib.eagle_verify_create.argtypes = [C.POINTER(VerifyDesc), C.POINTER(H)]
    lib.eagle_verify_create.restype = C.c_int
    lib.eagle_verify_tree_attention.argtypes = [H, C.POINTER(TreeAttentionArgs), C.c_void_p]
    lib.eagle_verify_tree_attention.restype = C.c_int
    lib.eagle_verify_spec_accept.argtypes = [H, C.POINTER(SpecAcceptArgs), C.c_void_p]
    lib.eagle_verify_spec_accept.restype = C.c_int
    lib.eagle_verify_spec_accept_noalloc.argtypes = [C.POINTER(VerifyDesc), C.POINTER(SpecAcceptArgs), C.c_void_p]
    lib.eagle_verify_spec_accept_noalloc.restype = C.c_int
    lib.eagle_verify_destroy.argtypes = [H]
    lib.eagle_verify_destroy.restype = C.c_int
    lib.eagle_verify_last_error.argtypes = [H]
    lib.eagle_verify_last_error.restype = C.c_char_p
    lib.eagle_verify_check_tree_attention.argtypes = [C.POINTER(VerifyDesc), C.POINTER(TreeAttentionArgs),
                                                      C.POINTER(AttentionPlan)]
    lib.eagle_verify_check_tree_attention.restype = C.c_int
    lib.eagle_verify_check_spec_accept.argtypes = [C.POINTER(VerifyDesc), C.POINTER(SpecAcceptArgs)]
    lib.eagle_verify_check_spec_accept.restype = C.c_int
    lib.eagle_verify_last_attention_plan.argtypes = [H, C.POINTER(AttentionPlan)]
    lib.eagle_verify_last_attention_plan.restype = C.c_int
    lib.eagle_verify_last_accept_paths.argtypes = [H, C.POINTER(C.c_int)]
    lib.eagle_verify_last_accept_paths.restype = C.c_int
    lib.eagle_verify_set_timeline.argtypes = [H, C.c_void_p, C.c_int64]
    lib.eagle_verify_set_timeline.restype = C.c_int
    lib.eagle_verify_kv_commit.argtypes = [H, C.POINTER(KvCommitArgs), C.c_void_p]
    lib.eagle_verify_kv_commit.restype = C.c_int
    lib.eagle_verify_check_kv_commit.argtypes = [C.POINTER(VerifyDesc), C.POINTER(KvCommitArgs)]
    lib.eagle_verify_check_kv_commit.restype = C.c_int
    lib.eagle_verify_tree_expand.argtypes = [H, C.POINTER(TreeExpandArgs), C.c_void_p]
    lib.eagle_verify_tree_expand.restype = C.c_int
    lib.eagle_verify_check_tree_expand.argtypes = [C.POINTER(VerifyDesc), C.POINTER(TreeExpandArgs)]
    lib.eagle_verify_check_tree_expand.restype = C.c_int
    lib.eagle_verify_tree_rerank.argtypes = [H, C.POINTER(TreeRerankArgs), C.c_void_p]
    lib.eagle_verify_tree_rerank.restype = C.c_int
    lib.eagle_verify_check_tree_rerank.argtypes = [C.POINTER(VerifyDesc), C.POINTER(TreeRerankArgs)]
    lib.eagle_verify_check_tree_rerank.restype = C.c_int
