"""ctypes binding of the C ABI in include/csmla.h (argument marshalling only).

Every step of the attention runs inside libcsmla.so on the GPU.  This module
only converts Python / torch objects into the ABI's plain structs and
pointers; it has no compute path of its own and raises if the library is
missing.  torch provides device memory and the HIP stream.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# CSMLA_LIB points the binding at another build of the same ABI (the host-only
# sanitizer build the host ABI tests use); by default the in-tree HIP library.
LIB_PATH = os.environ.get("CSMLA_LIB") or os.path.join(_HERE, "libcsmla.so")

CSMLA_METADATA_WORDS = 1024
LAYOUTS = {"BSND": 0, "TND": 1, "PA_BBND": 2}

STATUS = {0: "CSMLA_OK", 1: "CSMLA_ERR_INVALID_ARG", 2: "CSMLA_ERR_UNSUPPORTED", 3: "CSMLA_ERR_WORKSPACE",
          4: "CSMLA_ERR_METADATA_MISMATCH", 5: "CSMLA_ERR_HIP"}

_i32 = ctypes.c_int32
_p = ctypes.c_void_p


class CsmlaProblem(ctypes.Structure):
    _fields_ = [(n, _i32) for n in (
        "batch", "n1", "n2", "d", "layout_q", "layout_kv", "q_s", "t1", "ori_s", "cmp_s",
        "ori_block_size", "cmp_block_size", "ori_num_blocks", "cmp_num_blocks",
        "ori_table_cols", "cmp_table_cols", "has_cmp", "topk")] + [("softmax_scale", ctypes.c_float)] + [
        (n, _i32) for n in ("cmp_ratio", "ori_mask_mode", "cmp_mask_mode", "ori_win_left", "ori_win_right",
                            "kv_scale_mode", "q_descale_per_head", "topk_value_mode", "return_softmax_lse",
                            "q_dtype", "kv_dtype", "ori_topk")]

Q_DTYPES = {"fp8": 0, "bf16": 1}
KV_DTYPES = {"fp8": 0, "bf16": 1, "packed640": 2}


class CsmlaHostLengths(ctypes.Structure):
    _fields_ = [(n, _p) for n in (
        "cu_seqlens_q", "seqused_q", "seqused_ori_kv", "cu_seqlens_ori_kv", "seqused_cmp_kv",
        "cu_seqlens_cmp_kv", "cmp_residual_kv", "cmp_topk_length", "ori_topk_length")]


TENSOR_FIELDS = ("q", "q_descale", "ori_kv", "ori_kv_descale", "cmp_kv", "cmp_kv_descale", "cmp_sparse_indices",
                 "ori_block_table", "cmp_block_table", "cu_seqlens_q", "cu_seqlens_ori_kv", "cu_seqlens_cmp_kv",
                 "seqused_q", "seqused_ori_kv", "seqused_cmp_kv", "cmp_residual_kv", "cmp_topk_length", "sinks",
                 "attn_out", "softmax_lse", "workspace")


TENSOR_FIELDS_TAIL = ("ori_sparse_indices", "ori_topk_length")


class CsmlaTensors(ctypes.Structure):
    _fields_ = ([(n, _p) for n in TENSOR_FIELDS] + [("workspace_bytes", ctypes.c_size_t)]
                + [(n, _p) for n in TENSOR_FIELDS_TAIL])


class CsmlaError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: {STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH):
    """Load libcsmla.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    lib.csmla_abi_version.restype = ctypes.c_int
    lib.csmla_status_string.restype = ctypes.c_char_p
    lib.csmla_status_string.argtypes = [ctypes.c_int]
    lib.csmla_last_error.restype = ctypes.c_char_p
    lib.csmla_metadata_words.restype = ctypes.c_size_t
    lib.csmla_validate.restype = ctypes.c_int
    lib.csmla_validate.argtypes = [ctypes.POINTER(CsmlaProblem)]
    lib.csmla_plan.restype = ctypes.c_int
    lib.csmla_plan.argtypes = [ctypes.POINTER(CsmlaProblem), ctypes.POINTER(CsmlaHostLengths),
                               ctypes.POINTER(_i32), ctypes.c_size_t, ctypes.POINTER(ctypes.c_size_t)]
    lib.csmla_plan_check.restype = ctypes.c_int
    lib.csmla_plan_check.argtypes = [ctypes.POINTER(CsmlaProblem), ctypes.POINTER(CsmlaHostLengths),
                                     ctypes.POINTER(_i32)]
    for fn in (lib.csmla_forward, lib.csmla_forward_noalloc):
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.POINTER(CsmlaProblem), ctypes.POINTER(CsmlaTensors), ctypes.POINTER(_i32), _p]
    for fn in (lib.csmla_debug_resolve, lib.csmla_debug_resolve_whole_token):
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.POINTER(CsmlaProblem), ctypes.POINTER(CsmlaTensors), _p, _p, _i32, _p]
    _lib = lib
    return lib


def _check(st: int, where: str):
    if st != 0:
        raise CsmlaError(st, where, load().csmla_last_error().decode())


# ---------------------------------------------------------------------------
# the C entry points, same names
# ---------------------------------------------------------------------------

def csmla_abi_version() -> int:
    return load().csmla_abi_version()


def csmla_status_string(status: int) -> str:
    return load().csmla_status_string(status).decode()


def csmla_last_error() -> str:
    return load().csmla_last_error().decode()


def csmla_metadata_words() -> int:
    return int(load().csmla_metadata_words())


def csmla_validate(problem: CsmlaProblem) -> int:
    return load().csmla_validate(ctypes.byref(problem))


def csmla_plan(problem: CsmlaProblem, lengths: Optional[CsmlaHostLengths] = None,
               raise_on_error: bool = True) -> Tuple[int, np.ndarray, int]:
    """Returns (status, int32[1024] metadata, workspace bytes)."""
    md = np.zeros(CSMLA_METADATA_WORDS, dtype=np.int32)
    ws = ctypes.c_size_t(0)
    st = load().csmla_plan(ctypes.byref(problem), ctypes.byref(lengths) if lengths is not None else None,
                           md.ctypes.data_as(ctypes.POINTER(_i32)), md.size, ctypes.byref(ws))
    if raise_on_error:
        _check(st, "csmla_plan")
    return st, md, int(ws.value)


# (array, pointer) of the last metadata array passed in that needed no
# conversion, one slot for the attention entry points and one for the
# indexer's: numpy's ctypes pointer takes a few microseconds to form, as
# much as the launch itself, so a caller that passes the same plan again
# reuses it.  The pointer points into the caller's own buffer, so in-place
# edits are seen; the reference held here keeps that buffer alive.
_md_last = [(None, None), (None, None)]


def _md_pointer(metadata, slot: int = 0):
    last = _md_last[slot]
    if metadata is last[0]:
        return last[1]
    md = np.ascontiguousarray(metadata, dtype=np.int32)
    ptr = md.ctypes.data_as(ctypes.POINTER(_i32))
    if md is metadata:
        _md_last[slot] = (metadata, ptr)
    return ptr


def csmla_forward(problem: CsmlaProblem, tensors: CsmlaTensors, metadata: np.ndarray, stream: int = 0,
                  raise_on_error: bool = True) -> int:
    st = load().csmla_forward(ctypes.byref(problem), ctypes.byref(tensors), _md_pointer(metadata), _p(stream))
    if raise_on_error:
        _check(st, "csmla_forward")
    return st


def csmla_plan_check(problem: CsmlaProblem, lengths: Optional[CsmlaHostLengths], metadata: np.ndarray) -> int:
    """CSMLA_OK (0) if `metadata` was planned for this problem and these host
    lengths, else CSMLA_ERR_METADATA_MISMATCH (4) or a validation status."""
    md = np.ascontiguousarray(metadata, dtype=np.int32)
    return load().csmla_plan_check(ctypes.byref(problem), ctypes.byref(lengths) if lengths is not None else None,
                                   md.ctypes.data_as(ctypes.POINTER(_i32)))


def csmla_forward_noalloc(problem: CsmlaProblem, tensors: CsmlaTensors, metadata: np.ndarray, stream: int = 0,
                          raise_on_error: bool = True) -> int:
    """csmla_forward with the split partials in the library's static device
    scratch (tensors.workspace is ignored); allocates nothing."""
    st = load().csmla_forward_noalloc(ctypes.byref(problem), ctypes.byref(tensors), _md_pointer(metadata),
                                      _p(stream))
    if raise_on_error:
        _check(st, "csmla_forward_noalloc")
    return st


def csmla_debug_resolve(problem: CsmlaProblem, tensors: CsmlaTensors, keys_ptr: int, counts_ptr: int,
                        max_keys: int, stream: int = 0) -> int:
    st = load().csmla_debug_resolve(ctypes.byref(problem), ctypes.byref(tensors), _p(keys_ptr), _p(counts_ptr),
                                    max_keys, _p(stream))
    _check(st, "csmla_debug_resolve")
    return st


def csmla_debug_resolve_whole_token(problem: CsmlaProblem, tensors: CsmlaTensors, keys_ptr: int, counts_ptr: int,
                                    max_keys: int, stream: int = 0) -> int:
    st = load().csmla_debug_resolve_whole_token(ctypes.byref(problem), ctypes.byref(tensors), _p(keys_ptr),
                                                _p(counts_ptr), max_keys, _p(stream))
    _check(st, "csmla_debug_resolve_whole_token")
    return st


# ---------------------------------------------------------------------------
# marshalling helpers for torch tensors
# ---------------------------------------------------------------------------

def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    return int(x.data_ptr())


def problem_from(inp) -> CsmlaProblem:
    """Fill the problem struct from an object with the pages' tensor names
    (q, ori_kv, ... as torch tensors) and attributes."""
    p = CsmlaProblem()
    p.batch = int(inp.batch)
    p.n1 = int(inp.q.shape[1])
    p.n2 = 1
    p.d = int(inp.q.shape[2])
    p.layout_q = LAYOUTS[inp.layout_q]
    p.layout_kv = LAYOUTS[inp.layout_kv]
    p.q_s = int(inp.q_s)
    p.t1 = int(inp.q.shape[0])
    if inp.layout_kv == "PA_BBND":
        p.ori_block_size = int(inp.ori_kv.shape[1])
        p.ori_num_blocks = int(inp.ori_kv.shape[0])
        p.ori_table_cols = int(inp.ori_block_table.shape[1])
    elif inp.layout_kv == "BSND":
        p.ori_s = int(inp.ori_kv.shape[1])
    else:
        p.ori_s = int(inp.ori_kv.shape[0])
    if inp.cmp_kv is not None:
        p.has_cmp = 1
        if inp.layout_kv == "PA_BBND":
            p.cmp_block_size = int(inp.cmp_kv.shape[1])
            p.cmp_num_blocks = int(inp.cmp_kv.shape[0])
            p.cmp_table_cols = int(inp.cmp_block_table.shape[1])
        elif inp.layout_kv == "BSND":
            p.cmp_s = int(inp.cmp_kv.shape[1])
        else:
            p.cmp_s = int(inp.cmp_kv.shape[0])
    p.topk = 0 if inp.cmp_sparse_indices is None else int(inp.cmp_sparse_indices.shape[-1])
    p.softmax_scale = float(inp.softmax_scale)
    p.cmp_ratio = int(inp.cmp_ratio)
    p.ori_mask_mode = int(inp.ori_mask_mode)
    p.cmp_mask_mode = int(inp.cmp_mask_mode)
    p.ori_win_left = int(inp.ori_win_left) if inp.ori_mask_mode == 4 else -1
    p.ori_win_right = int(inp.ori_win_right) if inp.ori_mask_mode == 4 else -1
    p.kv_scale_mode = int(inp.kv_scale_mode)
    p.q_descale_per_head = 1 if (inp.q_descale is not None and inp.q_descale.dim() == 2) else 0
    p.q_dtype = Q_DTYPES[getattr(inp, "q_format", "fp8")]
    p.kv_dtype = KV_DTYPES[getattr(inp, "kv_format", "fp8")]
    oi = getattr(inp, "ori_sparse_indices", None)
    p.ori_topk = 0 if oi is None else int(oi.shape[-1])
    p.topk_value_mode = 0
    p.return_softmax_lse = 1 if inp.return_lse else 0
    return p


_LEN_NAMES = ("cu_seqlens_q", "seqused_q", "seqused_ori_kv", "cu_seqlens_ori_kv", "seqused_cmp_kv",
              "cu_seqlens_cmp_kv", "cmp_residual_kv", "cmp_topk_length", "ori_topk_length")


def host_lengths_from(inp):
    """Host copies of the length tensors (kept alive by the returned list)."""
    keep = []
    hl = CsmlaHostLengths()
    for n in _LEN_NAMES:
        x = getattr(inp, n, None)
        if x is None:
            continue
        arr = np.ascontiguousarray(x.detach().cpu().numpy().astype(np.int32))
        keep.append(arr)
        setattr(hl, n, arr.ctypes.data)
    return hl, keep


def tensors_from(inp, out, lse, workspace=None) -> CsmlaTensors:
    """Device pointers of the inputs (attributes of `inp`) and the outputs."""
    t = CsmlaTensors()
    for n in TENSOR_FIELDS + TENSOR_FIELDS_TAIL:
        if n in ("attn_out", "softmax_lse", "workspace"):
            continue
        v = getattr(inp, n, None)
        if v is not None:
            setattr(t, n, _ptr(v))
    t.attn_out = _ptr(out)
    t.softmax_lse = _ptr(lse)
    if workspace is not None:
        t.workspace = _ptr(workspace)
        t.workspace_bytes = int(workspace.numel() * workspace.element_size())
    return t


class Plan:
    """A planned call: problem struct, metadata and workspace size."""

    def __init__(self, inp, lengths: bool = True):
        self.problem = problem_from(inp)
        hl, keep = host_lengths_from(inp) if lengths else (None, [])
        _, self.metadata, self.workspace_bytes = csmla_plan(self.problem, hl)
        self._keep = keep

    @property
    def splits(self) -> int:
        return int(self.metadata[5])

    @property
    def grid(self) -> int:
        return int(self.metadata[7])

    @property
    def split_key(self) -> bool:
        """The split-key decode kernel (64 heads, <= 128 keys per unit, the
        splits merged inside the kernel)."""
        return bool(self.metadata[13])

    @property
    def head_group(self) -> int:
        """Heads per work unit: 8 or 16 (head-split decode kernel), 64 (whole-token
        prefill kernel), or 0 (key-split kernel)."""
        return int(self.metadata[12])

    @property
    def dk_parts(self) -> int:
        """Key parts per (token, head group) of the head-split kernel (1: none);
        the last part of a group merges the others' partials inside the kernel."""
        return int(self.metadata[14])


def forward(inp, out=None, lse=None, workspace=None, plan: Optional[Plan] = None, stream=None):
    """Run the attention on inputs already on the GPU.  Allocates the outputs
    (and the workspace) with torch when they are not given.  A plan passed in
    is checked against the inputs' host lengths (csmla_plan_check).  Returns
    (out, lse)."""
    import torch
    if plan is not None:
        hl, keep = host_lengths_from(inp)
        _check(csmla_plan_check(plan.problem, hl, plan.metadata), "csmla_plan_check")
    plan = plan or Plan(inp)
    dev = inp.q.device
    if out is None:
        out = torch.empty(inp.q.shape, dtype=torch.bfloat16, device=dev)
    if lse is None and inp.return_lse:
        lse = torch.empty(inp.q.shape[:2], dtype=torch.float32, device=dev)
    if workspace is None and plan.workspace_bytes > 0:
        workspace = torch.zeros(plan.workspace_bytes, dtype=torch.uint8, device=dev)
    t = tensors_from(inp, out, lse, workspace)
    s = torch.cuda.current_stream(dev).cuda_stream if stream is None else int(stream)
    csmla_forward(plan.problem, t, plan.metadata, s)
    return out, lse


def debug_resolve(inp, max_keys: int, stream=None, whole_token: bool = False):
    """Resolved physical rows per query token (the kernels' resolution code:
    the key-split / head-split kernels' functions, or with whole_token the
    whole-token kernel's own).  Returns (keys int32 [t1, max_keys], counts
    int32 [t1, 2]) on the GPU."""
    import torch
    dev = inp.q.device
    keys = torch.full((inp.q.shape[0], max_keys), -1, dtype=torch.int32, device=dev)
    counts = torch.zeros((inp.q.shape[0], 2), dtype=torch.int32, device=dev)
    p = problem_from(inp)
    t = tensors_from(inp, None, None)
    s = torch.cuda.current_stream(dev).cuda_stream if stream is None else int(stream)
    fn = csmla_debug_resolve_whole_token if whole_token else csmla_debug_resolve
    fn(p, t, _ptr(keys), _ptr(counts), max_keys, s)
    return keys, counts


# ---------------------------------------------------------------------------
# the lightning-indexer top-k (include/csmla_indexer.h)
# ---------------------------------------------------------------------------

CSMLA_INDEXER_METADATA_WORDS = 32


class CsmlaIndexerProblem(ctypes.Structure):
    _fields_ = [(n, _i32) for n in (
        "batch", "g", "n2", "d", "layout_q", "layout_k", "q_s", "t1", "k_s", "block_size", "num_blocks",
        "table_cols", "topk", "mask_mode", "cmp_ratio", "quant_mode")]


class CsmlaIndexerHostLengths(ctypes.Structure):
    _fields_ = [(n, _p) for n in ("cu_seqlens_q", "seqused_q", "cu_seqlens_k", "seqused_k", "cmp_residual_k")]


INDEXER_TENSOR_FIELDS = ("query", "key", "weights", "query_dequant_scale", "key_dequant_scale", "cu_seqlens_q",
                         "cu_seqlens_k", "seqused_q", "seqused_k", "cmp_residual_k", "block_table",
                         "sparse_indices", "workspace")


class CsmlaIndexerTensors(ctypes.Structure):
    _fields_ = [(n, _p) for n in INDEXER_TENSOR_FIELDS] + [("workspace_bytes", ctypes.c_size_t)]


def _load_indexer():
    lib = load()
    if not getattr(lib, "_indexer_ready", False):
        lib.csmla_indexer_metadata_words.restype = ctypes.c_size_t
        lib.csmla_indexer_validate.restype = ctypes.c_int
        lib.csmla_indexer_validate.argtypes = [ctypes.POINTER(CsmlaIndexerProblem)]
        lib.csmla_indexer_plan.restype = ctypes.c_int
        lib.csmla_indexer_plan.argtypes = [ctypes.POINTER(CsmlaIndexerProblem),
                                           ctypes.POINTER(CsmlaIndexerHostLengths), ctypes.POINTER(_i32),
                                           ctypes.c_size_t, ctypes.POINTER(ctypes.c_size_t)]
        lib.csmla_indexer_forward.restype = ctypes.c_int
        lib.csmla_indexer_forward.argtypes = [ctypes.POINTER(CsmlaIndexerProblem),
                                              ctypes.POINTER(CsmlaIndexerTensors), ctypes.POINTER(_i32), _p]
        lib._indexer_ready = True
    return lib


def csmla_indexer_metadata_words() -> int:
    return int(_load_indexer().csmla_indexer_metadata_words())


def csmla_indexer_validate(problem: CsmlaIndexerProblem) -> int:
    return _load_indexer().csmla_indexer_validate(ctypes.byref(problem))


def csmla_indexer_plan(problem: CsmlaIndexerProblem, lengths: Optional[CsmlaIndexerHostLengths] = None,
                       raise_on_error: bool = True) -> Tuple[int, np.ndarray, int]:
    """Returns (status, int32 plan, workspace bytes)."""
    md = np.zeros(CSMLA_INDEXER_METADATA_WORDS, dtype=np.int32)
    ws = ctypes.c_size_t(0)
    st = _load_indexer().csmla_indexer_plan(ctypes.byref(problem),
                                            ctypes.byref(lengths) if lengths is not None else None,
                                            md.ctypes.data_as(ctypes.POINTER(_i32)), md.size, ctypes.byref(ws))
    if raise_on_error:
        _check(st, "csmla_indexer_plan")
    return st, md, int(ws.value)


def csmla_indexer_forward(problem: CsmlaIndexerProblem, tensors: CsmlaIndexerTensors, metadata: np.ndarray,
                          stream: int = 0, raise_on_error: bool = True) -> int:
    st = _load_indexer().csmla_indexer_forward(ctypes.byref(problem), ctypes.byref(tensors),
                                               _md_pointer(metadata, 1), _p(stream))
    if raise_on_error:
        _check(st, "csmla_indexer_forward")
    return st


def indexer_problem_from(inp) -> CsmlaIndexerProblem:
    """Problem struct of an object carrying the page's indexer tensors (q,
    q_scale, weights, key, key_scale, ... as torch tensors) and attributes."""
    p = CsmlaIndexerProblem()
    p.batch = int(inp.batch)
    p.g = int(inp.q.shape[1])
    p.n2 = 1
    p.d = int(inp.q.shape[2])
    p.layout_q = LAYOUTS[inp.layout_q]
    p.layout_k = LAYOUTS[inp.layout_k]
    p.q_s = int(inp.q_s)
    p.t1 = int(inp.q.shape[0])
    if inp.layout_k == "PA_BBND":
        p.block_size = int(inp.key.shape[1])
        p.num_blocks = int(inp.key.shape[0])
        p.table_cols = int(inp.block_table.shape[1])
    elif inp.layout_k == "BSND":
        p.k_s = int(inp.key.shape[1])
    else:
        p.k_s = int(inp.key.shape[0])
    p.topk = int(inp.topk)
    p.mask_mode = int(inp.mask_mode)
    p.cmp_ratio = int(inp.cmp_ratio)
    p.quant_mode = 1
    return p


_IDX_LEN_NAMES = ("cu_seqlens_q", "seqused_q", "cu_seqlens_k", "seqused_k", "cmp_residual_k")


def indexer_host_lengths_from(inp):
    keep = []
    hl = CsmlaIndexerHostLengths()
    for n in _IDX_LEN_NAMES:
        x = getattr(inp, n, None)
        if x is None:
            continue
        arr = np.ascontiguousarray(x.detach().cpu().numpy().astype(np.int32))
        keep.append(arr)
        setattr(hl, n, arr.ctypes.data)
    return hl, keep


def indexer_tensors_from(inp, sparse_indices, workspace) -> CsmlaIndexerTensors:
    t = CsmlaIndexerTensors()
    t.query = _ptr(inp.q)
    t.key = _ptr(inp.key)
    t.weights = _ptr(inp.weights)
    t.query_dequant_scale = _ptr(inp.q_scale)
    t.key_dequant_scale = _ptr(inp.key_scale)
    for n in ("cu_seqlens_q", "cu_seqlens_k", "seqused_q", "seqused_k", "cmp_residual_k", "block_table"):
        v = getattr(inp, n, None)
        if v is not None:
            setattr(t, n, _ptr(v))
    t.sparse_indices = _ptr(sparse_indices)
    if workspace is not None:
        t.workspace = _ptr(workspace)
        t.workspace_bytes = int(workspace.numel() * workspace.element_size())
    return t


class IndexerPlan:
    """A planned indexer call: problem struct, plan words and workspace size."""

    def __init__(self, inp, lengths: bool = True):
        self.problem = indexer_problem_from(inp)
        hl, keep = indexer_host_lengths_from(inp) if lengths else (None, [])
        _, self.metadata, self.workspace_bytes = csmla_indexer_plan(self.problem, hl)
        self._keep = keep

    @property
    def stride(self) -> int:
        """floats per score row in the workspace"""
        return int(self.metadata[9])


def indexer_forward(inp, out=None, workspace=None, plan: Optional[IndexerPlan] = None, stream=None):
    """Run the indexer on inputs already on the GPU.  Returns (sparse_indices
    int32 [t1, 1, topk], workspace); the workspace holds the float32 scores,
    row t at t * plan.stride floats."""
    import torch
    plan = plan or IndexerPlan(inp)
    dev = inp.q.device
    if out is None:
        out = torch.empty((inp.q.shape[0], 1, int(inp.topk)), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
    t = indexer_tensors_from(inp, out, workspace)
    s = torch.cuda.current_stream(dev).cuda_stream if stream is None else int(stream)
    csmla_indexer_forward(plan.problem, t, plan.metadata, s)
    return out, workspace
