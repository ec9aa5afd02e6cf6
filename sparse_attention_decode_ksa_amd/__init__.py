"""Block top-k / vote-union sparse decode attention for AMD MI355X (gfx950).

Thin Python binding over ``libksa.so`` (C ABI in ``include/ksa.h``).  It only
marshals arguments: it checks tensor dtype, shape, contiguity and device,
passes raw device pointers and the current HIP stream, and allocates the
workspace the library asks for.  Every step of the computation runs in the
library's HIP kernels; there is no CPU or PyTorch fallback, and a missing or
unloadable library raises :class:`KsaLibraryError` on first use.

Function names match the C entry points: ``ksa_block_summaries``,
``ksa_select_topk``, ``ksa_sparse_decode`` (and ``ksa_sparse_decode_noalloc``, no workspace), ``ksa_block_topk_decode`` (and
``ksa_block_topk_decode_varlen``, one length per sequence), ``ksa_vote_select``, ``ksa_dense_decode``, the paged-cache calls
``ksa_paged_block_summaries``, ``ksa_paged_block_topk_decode`` and
``ksa_paged_dense_decode``, ``ksa_paged_vote_select``, ``ksa_paged_sparse_decode``,
``ksa_paged_vote_layer_decode``, ``ksa_paged_select_topk_ex``,
``ksa_paged_vote_select_heads`` and ``ksa_paged_vote_select_per_head``, the selection
variants ``ksa_select_topk_ex``, ``ksa_vote_select_heads`` and
``ksa_vote_select_per_head``, the diagnostic ``ksa_attention_recall``, the
selection layer ``ksa_vote_layer_decode``, ``ksa_workspace_bytes``,
``ksa_status_string`` and ``ksa_version``.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build (python -m sparse_attention_decode_ksa_amd.build)
LIB_PATH = os.path.join(_HERE, "libksa.so")

KSA_OK, KSA_ERR_INVALID_ARGUMENT, KSA_ERR_UNSUPPORTED, KSA_ERR_WORKSPACE_TOO_SMALL, KSA_ERR_HIP = range(5)
KSA_F32, KSA_BF16 = 0, 1
KSA_SEL_BLOCKS, KSA_SEL_TOKENS, KSA_SEL_HEAD_TOKENS = 0, 1, 2
(KSA_OP_SELECT_TOPK, KSA_OP_SPARSE_BLOCKS, KSA_OP_SPARSE_TOKENS, KSA_OP_VOTE_SELECT,
 KSA_OP_DENSE, KSA_OP_PAGED_DENSE, KSA_OP_VOTE_LAYER, KSA_OP_SPARSE_HEAD_TOKENS,
 KSA_OP_PAGED_VOTE_LAYER) = range(9)
SIZE_MAX = ctypes.c_size_t(-1).value

EXPORTED = ("ksa_block_summaries", "ksa_select_topk", "ksa_sparse_decode",
            "ksa_block_topk_decode", "ksa_vote_select", "ksa_dense_decode",
            "ksa_paged_block_summaries", "ksa_paged_block_topk_decode", "ksa_paged_dense_decode",
            "ksa_select_topk_ex", "ksa_vote_select_heads", "ksa_attention_recall",
            "ksa_vote_layer_decode", "ksa_vote_select_per_head", "ksa_paged_vote_select",
            "ksa_paged_sparse_decode", "ksa_paged_vote_layer_decode", "ksa_paged_select_topk_ex",
            "ksa_paged_vote_select_heads", "ksa_paged_vote_select_per_head",
            "ksa_block_topk_decode_varlen", "ksa_sparse_decode_noalloc", "ksa_workspace_bytes",
            "ksa_status_string", "ksa_version")
NOALLOC_SCRATCH_BYTES = 4 << 20  # KSA_NOALLOC_SCRATCH_BYTES
KSA_AGG_SUM, KSA_AGG_MAX = 0, 1


class KsaLibraryError(RuntimeError):
    """libksa.so is missing or cannot be loaded."""


class KsaError(RuntimeError):
    """A libksa call returned a status other than KSA_OK."""

    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__("%s: %s" % (call, ksa_status_string(status)))


class Problem(ctypes.Structure):
    """Mirror of ``ksa_problem``."""
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("seq_len", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("sm_scale", ctypes.c_float)]


class Selection(ctypes.Structure):
    """Mirror of ``ksa_selection``."""
    _fields_ = [("kind", ctypes.c_int32), ("idx", ctypes.c_void_p), ("count", ctypes.c_int32)]


class SelectOptions(ctypes.Structure):
    """Mirror of ``ksa_select_options``."""
    _fields_ = [("top_k", ctypes.c_int32), ("aggregate", ctypes.c_int32),
                ("force_last_block", ctypes.c_int32)]


class PagedKv(ctypes.Structure):
    """Mirror of ``ksa_paged_kv``."""
    _fields_ = [("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("max_blocks", ctypes.c_int32), ("num_pages", ctypes.c_int32)]


_lock = threading.Lock()
_lib = None


def load_library(path: str = LIB_PATH):
    """Load libksa.so once and declare its signatures."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise KsaLibraryError(
                "libksa.so not found at %s; build it with "
                "`python -m sparse_attention_decode_ksa_amd.build`" % path)
        try:
            lib = ctypes.CDLL(path)
        except OSError as e:
            raise KsaLibraryError("cannot load %s: %s" % (path, e)) from e
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        PP = ctypes.POINTER(Problem)
        lib.ksa_block_summaries.argtypes = [PP, P, P, I32, I32, P]
        lib.ksa_select_topk.argtypes = [PP, P, P, I32, P, P, P, SZ, P]
        lib.ksa_sparse_decode.argtypes = [PP, P, P, P, ctypes.POINTER(Selection), P, P, P, SZ, P]
        lib.ksa_block_topk_decode.argtypes = [PP, P, P, P, P, I32, I32, P, P, P, P]
        lib.ksa_vote_select.argtypes = [PP, P, P, I32, I32, P, P, P, SZ, P]
        lib.ksa_dense_decode.argtypes = [PP, P, P, P, P, P, P, SZ, P]
        PG = ctypes.POINTER(PagedKv)
        lib.ksa_paged_block_summaries.argtypes = [PP, PG, P, P, I32, I32, P]
        lib.ksa_paged_block_topk_decode.argtypes = [PP, PG, P, P, P, P, I32, I32, P, P, P, P]
        lib.ksa_paged_dense_decode.argtypes = [PP, PG, P, P, P, P, P, P, SZ, P]
        lib.ksa_select_topk_ex.argtypes = [PP, P, P, ctypes.POINTER(SelectOptions), P, P, P, SZ, P]
        lib.ksa_vote_select_heads.argtypes = [PP, P, P, I32, I32, P, I32, P, P, P, SZ, P]
        lib.ksa_attention_recall.argtypes = [P, P, P, I32, P]
        lib.ksa_vote_layer_decode.argtypes = [PP, P, P, P, I32, I32, P, P, P, P, P, SZ, P]
        lib.ksa_vote_select_per_head.argtypes = [PP, P, P, I32, I32, P, P, SZ, P]
        lib.ksa_paged_vote_select.argtypes = [PP, PG, P, P, I32, I32, P, P, P, SZ, P]
        lib.ksa_paged_sparse_decode.argtypes = [PP, PG, P, P, P, ctypes.POINTER(Selection), P, P,
                                                P, SZ, P]
        lib.ksa_paged_vote_layer_decode.argtypes = [PP, PG, P, P, P, I32, I32, P, P, P, P, P, SZ,
                                                    P]
        lib.ksa_paged_select_topk_ex.argtypes = [PP, PG, P, P, ctypes.POINTER(SelectOptions), P, P,
                                                 P, SZ, P]
        lib.ksa_paged_vote_select_heads.argtypes = [PP, PG, P, P, I32, I32, P, I32, P, P, P, SZ, P]
        lib.ksa_paged_vote_select_per_head.argtypes = [PP, PG, P, P, I32, I32, P, P, SZ, P]
        lib.ksa_block_topk_decode_varlen.argtypes = [PP, P, P, P, P, P, I32, I32, P, P, P, P]
        lib.ksa_sparse_decode_noalloc.argtypes = [PP, P, P, P, ctypes.POINTER(Selection), P, P, P]
        lib.ksa_workspace_bytes.argtypes = [PP, I32, I32]
        lib.ksa_workspace_bytes.restype = SZ
        lib.ksa_status_string.argtypes = [ctypes.c_int]
        lib.ksa_status_string.restype = ctypes.c_char_p
        lib.ksa_version.argtypes = []
        lib.ksa_version.restype = ctypes.c_char_p
        for name in EXPORTED[:-3]:  # every call but the three below returns a status
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
        return lib


def ksa_status_string(status: int) -> str:
    return load_library().ksa_status_string(int(status)).decode()


def ksa_version() -> str:
    return load_library().ksa_version().decode()


# ----------------------------------------------------------------------------- marshalling
def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KSA_BF16
    if t.dtype == torch.float32:
        return KSA_F32
    raise TypeError("KV dtype must be bfloat16 or float32, got %s" % t.dtype)


def make_problem(q: torch.Tensor, k: torch.Tensor, seq_len: int, block_size: int = 1,
                 sm_scale: float = 0.0) -> Problem:
    """Problem for q [B,Hq,D] and k [B,Hkv,T_cap,D] with T = seq_len."""
    if q.dim() != 3 or k.dim() != 4:
        raise ValueError("q must be [B,Hq,D] and k [B,Hkv,T_cap,D]")
    B, Hq, D = q.shape
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError("q %s and k %s disagree" % (tuple(q.shape), tuple(k.shape)))
    return Problem(B, Hq, k.shape[1], D, int(seq_len), k.shape[2], int(block_size),
                   _dtype_code(k), float(sm_scale))


def _dev(t: Optional[torch.Tensor], name: str, dtype=None, shape=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int, call: str):
    if status != KSA_OK:
        raise KsaError(status, call)


def ksa_workspace_bytes(problem: Problem, op: int, param: int) -> int:
    n = load_library().ksa_workspace_bytes(ctypes.byref(problem), int(op), int(param))
    if n == SIZE_MAX:
        raise KsaError(KSA_ERR_INVALID_ARGUMENT, "ksa_workspace_bytes")
    return n


def new_workspace(nbytes: int, device) -> torch.Tensor:
    """A device workspace of at least nbytes (its contents do not matter)."""
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def _workspace(problem: Problem, op: int, param: int, device, workspace):
    need = ksa_workspace_bytes(problem, op, param)
    if workspace is None:
        workspace = new_workspace(need, device)
    elif workspace.numel() * workspace.element_size() < need:
        raise KsaError(KSA_ERR_WORKSPACE_TOO_SMALL, "workspace")
    return workspace, ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()


def nblocks(n: int, bs: int) -> int:
    return (n + bs - 1) // bs


# ----------------------------------------------------------------------------- entry points
def ksa_block_summaries(k: torch.Tensor, summaries: torch.Tensor, seq_len: int, block_size: int,
                        first_block: int = 0, num_blocks: Optional[int] = None,
                        stream=None) -> torch.Tensor:
    """Mean key of blocks [first_block, first_block + num_blocks) of every
    (sequence, KV head), written into summaries [B,Hkv,ceil(T_cap/Bs),D]."""
    lib = load_library()
    B, Hkv, Tcap, D = k.shape
    prob = Problem(B, Hkv, Hkv, D, int(seq_len), Tcap, int(block_size), _dtype_code(k), 0.0)
    if num_blocks is None:
        num_blocks = nblocks(seq_len, block_size) - first_block
    pk = _dev(k, "k")
    ps = _dev(summaries, "summaries", k.dtype, (B, Hkv, nblocks(Tcap, block_size), D))
    _check(lib.ksa_block_summaries(ctypes.byref(prob), pk, ps, int(first_block), int(num_blocks),
                                   _stream(stream)), "ksa_block_summaries")
    return summaries


def ksa_select_topk(q: torch.Tensor, summaries: torch.Tensor, seq_len: int, block_size: int,
                    top_k: int, max_seq_len: Optional[int] = None, block_idx=None,
                    block_scores=None, want_scores: bool = False, sm_scale: float = 0.0,
                    workspace=None, stream=None):
    """Top-k blocks per (sequence, KV head) -> block_idx [B,Hkv,min(k,NB)] int32
    (and block_scores [B,Hkv,NB] fp32 when asked)."""
    lib = load_library()
    B, Hkv, nbcap, D = summaries.shape
    Tcap = max_seq_len if max_seq_len is not None else nbcap * block_size
    prob = Problem(B, q.shape[1], Hkv, D, int(seq_len), int(Tcap), int(block_size),
                   _dtype_code(summaries), float(sm_scale))
    nb = nblocks(seq_len, block_size)
    keff = min(top_k, nb)
    if block_idx is None:
        block_idx = torch.empty((B, Hkv, keff), dtype=torch.int32, device=q.device)
    if want_scores and block_scores is None:
        block_scores = torch.empty((B, Hkv, nb), dtype=torch.float32, device=q.device)
    ws, pws, nws = _workspace(prob, KSA_OP_SELECT_TOPK, top_k, q.device, workspace)
    _check(lib.ksa_select_topk(ctypes.byref(prob), _dev(q, "q", summaries.dtype, (B, prob.num_q_heads, D)),
                               _dev(summaries, "summaries"), int(top_k),
                               _dev(block_idx, "block_idx", torch.int32, (B, Hkv, keff)),
                               _dev(block_scores, "block_scores", torch.float32, (B, Hkv, nb)),
                               pws, nws, _stream(stream)), "ksa_select_topk")
    return (block_idx, block_scores) if block_scores is not None else block_idx


def ksa_sparse_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seq_len: int,
                      idx: torch.Tensor, kind: int = KSA_SEL_BLOCKS, block_size: int = 1,
                      out=None, lse=None, want_lse: bool = True, sm_scale: float = 0.0,
                      workspace=None, stream=None):
    """Attention of every query head over the selected blocks (kind BLOCKS,
    idx [B,Hkv,count]), the shared token list (kind TOKENS, idx [B,count]) or
    a list per query head (kind HEAD_TOKENS, idx [B,Hq,count]).
    Returns (out [B,Hq,D] fp32, lse [B,Hq] fp32 or None)."""
    lib = load_library()
    prob = make_problem(q, k, seq_len, block_size, sm_scale)
    B, Hq, D = q.shape
    count = idx.shape[-1]
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    ishape = {KSA_SEL_BLOCKS: (B, prob.num_kv_heads, count), KSA_SEL_TOKENS: (B, count),
              KSA_SEL_HEAD_TOKENS: (B, Hq, count)}[kind]
    sel = Selection(int(kind), _dev(idx, "idx", torch.int32, ishape), int(count))
    op = {KSA_SEL_BLOCKS: KSA_OP_SPARSE_BLOCKS, KSA_SEL_TOKENS: KSA_OP_SPARSE_TOKENS,
          KSA_SEL_HEAD_TOKENS: KSA_OP_SPARSE_HEAD_TOKENS}[kind]
    ws, pws, nws = _workspace(prob, op, count, q.device, workspace)
    _check(lib.ksa_sparse_decode(ctypes.byref(prob), _dev(q, "q", k.dtype), _dev(k, "k"),
                                 _dev(v, "v", k.dtype, k.shape), ctypes.byref(sel),
                                 _dev(out, "out", torch.float32, (B, Hq, D)),
                                 _dev(lse, "lse", torch.float32, (B, Hq)), pws, nws,
                                 _stream(stream)), "ksa_sparse_decode")
    return out, lse


def ksa_sparse_decode_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seq_len: int,
                              idx: torch.Tensor, kind: int = KSA_SEL_BLOCKS, block_size: int = 1,
                              out=None, lse=None, want_lse: bool = True, sm_scale: float = 0.0,
                              stream=None):
    """ksa_sparse_decode without a workspace: the library's own per-GPU
    scratch array holds the split rows' state (for callers that cannot
    allocate; calls overlapping on one GPU race).  Pass `out` (and `lse`)
    to allocate nothing at all."""
    lib = load_library()
    prob = make_problem(q, k, seq_len, block_size, sm_scale)
    B, Hq, D = q.shape
    count = idx.shape[-1]
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    ishape = {KSA_SEL_BLOCKS: (B, prob.num_kv_heads, count), KSA_SEL_TOKENS: (B, count),
              KSA_SEL_HEAD_TOKENS: (B, Hq, count)}[kind]
    sel = Selection(int(kind), _dev(idx, "idx", torch.int32, ishape), int(count))
    _check(lib.ksa_sparse_decode_noalloc(ctypes.byref(prob), _dev(q, "q", k.dtype), _dev(k, "k"),
                                         _dev(v, "v", k.dtype, k.shape), ctypes.byref(sel),
                                         _dev(out, "out", torch.float32, (B, Hq, D)),
                                         _dev(lse, "lse", torch.float32, (B, Hq)),
                                         _stream(stream)), "ksa_sparse_decode_noalloc")
    return out, lse


def ksa_block_topk_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                          summaries: torch.Tensor, seq_len: int, block_size: int, top_k: int,
                          refresh_last_block: bool = True, block_idx=None,
                          want_block_idx: bool = False, out=None, lse=None, want_lse: bool = True,
                          sm_scale: float = 0.0, stream=None):
    """One whole decode step in one launch: refresh the newest block's summary
    (in place, when asked), select the top-k blocks, attend them.
    Returns (out [B,Hq,D] fp32, lse [B,Hq] fp32 or None,
    block_idx [B,Hkv,min(k,NB)] int32 or None)."""
    lib = load_library()
    prob = make_problem(q, k, seq_len, block_size, sm_scale)
    B, Hq, D = q.shape
    Hkv, Tcap = k.shape[1], k.shape[2]
    keff = min(top_k, nblocks(seq_len, block_size))
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if block_idx is None and want_block_idx:
        block_idx = torch.empty((B, Hkv, keff), dtype=torch.int32, device=q.device)
    _check(lib.ksa_block_topk_decode(
        ctypes.byref(prob), _dev(q, "q", k.dtype), _dev(k, "k"), _dev(v, "v", k.dtype, k.shape),
        _dev(summaries, "summaries", k.dtype, (B, Hkv, nblocks(Tcap, block_size), D)),
        int(top_k), 1 if refresh_last_block else 0,
        _dev(block_idx, "block_idx", torch.int32, (B, Hkv, keff)),
        _dev(out, "out", torch.float32, (B, Hq, D)), _dev(lse, "lse", torch.float32, (B, Hq)),
        _stream(stream)), "ksa_block_topk_decode")
    return out, lse, block_idx


def ksa_block_topk_decode_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                 summaries: torch.Tensor, seq_lens: torch.Tensor, block_size: int,
                                 top_k: int, max_len: Optional[int] = None,
                                 refresh_last_block: bool = True, block_idx=None,
                                 want_block_idx: bool = False, out=None, lse=None,
                                 want_lse: bool = True, sm_scale: float = 0.0, stream=None):
    """ksa_block_topk_decode with one length per sequence (seq_lens [B] int32
    on the device; max_len, the longest, defaults to the cache capacity).
    block_idx [B,Hkv,min(k,NB(max_len))] holds each row's ids, then -1."""
    lib = load_library()
    B, Hq, D = q.shape
    Hkv, Tcap = k.shape[1], k.shape[2]
    T = int(max_len) if max_len is not None else Tcap
    prob = make_problem(q, k, T, block_size, sm_scale)
    keff = min(top_k, nblocks(T, block_size))
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if block_idx is None and want_block_idx:
        block_idx = torch.empty((B, Hkv, keff), dtype=torch.int32, device=q.device)
    _check(lib.ksa_block_topk_decode_varlen(
        ctypes.byref(prob), _dev(seq_lens, "seq_lens", torch.int32, (B,)), _dev(q, "q", k.dtype),
        _dev(k, "k"), _dev(v, "v", k.dtype, k.shape),
        _dev(summaries, "summaries", k.dtype, (B, Hkv, nblocks(Tcap, block_size), D)),
        int(top_k), 1 if refresh_last_block else 0,
        _dev(block_idx, "block_idx", torch.int32, (B, Hkv, keff)),
        _dev(out, "out", torch.float32, (B, Hq, D)), _dev(lse, "lse", torch.float32, (B, Hq)),
        _stream(stream)), "ksa_block_topk_decode_varlen")
    return out, lse, block_idx


def ksa_vote_select(q: torch.Tensor, k: torch.Tensor, seq_len: int, token_budget: int,
                    recent_window: int, token_idx=None, votes=None, want_votes: bool = False,
                    workspace=None, stream=None):
    """Shared token set [B, min(N,T)] int32 of the vote-union variant (and the
    per-token votes [B,T] uint8 when asked)."""
    lib = load_library()
    prob = make_problem(q, k, seq_len)
    B = q.shape[0]
    n_out = min(token_budget, seq_len)
    if token_idx is None:
        token_idx = torch.empty((B, n_out), dtype=torch.int32, device=q.device)
    if want_votes and votes is None:
        votes = torch.empty((B, seq_len), dtype=torch.uint8, device=q.device)
    ws, pws, nws = _workspace(prob, KSA_OP_VOTE_SELECT, token_budget, q.device, workspace)
    _check(lib.ksa_vote_select(ctypes.byref(prob), _dev(q, "q", k.dtype), _dev(k, "k"),
                               int(token_budget), int(recent_window),
                               _dev(token_idx, "token_idx", torch.int32, (B, n_out)),
                               _dev(votes, "votes", torch.uint8, (B, seq_len)), pws, nws,
                               _stream(stream)), "ksa_vote_select")
    return (token_idx, votes) if votes is not None else token_idx


def ksa_dense_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seq_len: int, out=None,
                     lse=None, want_lse: bool = True, sm_scale: float = 0.0, workspace=None,
                     stream=None):
    """Exact attention of every query head over all T tokens."""
    lib = load_library()
    prob = make_problem(q, k, seq_len, 1, sm_scale)
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    ws, pws, nws = _workspace(prob, KSA_OP_DENSE, 0, q.device, workspace)
    _check(lib.ksa_dense_decode(ctypes.byref(prob), _dev(q, "q", k.dtype), _dev(k, "k"),
                                _dev(v, "v", k.dtype, k.shape),
                                _dev(out, "out", torch.float32, (B, Hq, D)),
                                _dev(lse, "lse", torch.float32, (B, Hq)), pws, nws,
                                _stream(stream)), "ksa_dense_decode")
    return out, lse


# ----------------------------------------------------------------------------- paged cache
def _paged_args(q: torch.Tensor, k_pool: torch.Tensor, block_table: torch.Tensor,
                seq_lens: torch.Tensor, max_len: Optional[int], sm_scale: float):
    """Problem and ksa_paged_kv for q [B,Hq,D], pools [num_pages,Hkv,Bs,D],
    block_table [B,max_blocks] int32 and seq_lens [B] int32.  max_len is the
    longest sequence (read from seq_lens, a device sync, when not given)."""
    if k_pool.dim() != 4 or block_table.dim() != 2 or seq_lens.dim() != 1:
        raise ValueError("pools must be [num_pages,Hkv,Bs,D], block_table [B,max_blocks], "
                         "seq_lens [B]")
    num_pages, Hkv, Bs, D = k_pool.shape
    B = block_table.shape[0]
    max_blocks = block_table.shape[1]
    if max_len is None:
        max_len = int(seq_lens.max().item())
    Hq = q.shape[1] if q is not None else Hkv
    prob = Problem(B, Hq, Hkv, D, int(max_len), max_blocks * Bs, Bs, _dtype_code(k_pool),
                   float(sm_scale))
    pg = PagedKv(_dev(block_table, "block_table", torch.int32, (B, max_blocks)),
                 _dev(seq_lens, "seq_lens", torch.int32, (B,)), max_blocks, num_pages)
    return prob, pg


def ksa_paged_block_summaries(k_pool: torch.Tensor, summaries: torch.Tensor,
                              block_table: torch.Tensor, seq_lens: torch.Tensor,
                              max_len: Optional[int] = None, first_block: int = 0,
                              num_blocks: Optional[int] = None, newest_only: bool = False,
                              stream=None) -> torch.Tensor:
    """Mean key of blocks [first_block, first_block + num_blocks) of every
    sequence (those below its own block count), or of each sequence's newest
    block, into summaries [B,Hkv,max_blocks,D]."""
    lib = load_library()
    prob, pg = _paged_args(None, k_pool, block_table, seq_lens, max_len, 0.0)
    B, max_blocks = block_table.shape
    if newest_only:
        first_block, num_blocks = -1, 1
    elif num_blocks is None:
        num_blocks = max_blocks - first_block
    _check(lib.ksa_paged_block_summaries(
        ctypes.byref(prob), ctypes.byref(pg), _dev(k_pool, "k_pool"),
        _dev(summaries, "summaries", k_pool.dtype, (B, k_pool.shape[1], max_blocks, k_pool.shape[3])),
        int(first_block), int(num_blocks), _stream(stream)), "ksa_paged_block_summaries")
    return summaries


def ksa_paged_block_topk_decode(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                                summaries: torch.Tensor, block_table: torch.Tensor,
                                seq_lens: torch.Tensor, top_k: int,
                                max_len: Optional[int] = None, refresh_last_block: bool = True,
                                block_idx=None, want_block_idx: bool = False, out=None, lse=None,
                                want_lse: bool = True, sm_scale: float = 0.0, stream=None):
    """The one-launch decode step on a paged cache with per-sequence lengths.
    Returns (out [B,Hq,D] fp32, lse [B,Hq] fp32 or None, block_idx
    [B,Hkv,top_k] int32 (-1 past each row's k_eff) or None)."""
    lib = load_library()
    prob, pg = _paged_args(q, k_pool, block_table, seq_lens, max_len, sm_scale)
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if block_idx is None and want_block_idx:
        block_idx = torch.empty((B, Hkv, top_k), dtype=torch.int32, device=q.device)
    _check(lib.ksa_paged_block_topk_decode(
        ctypes.byref(prob), ctypes.byref(pg), _dev(q, "q", k_pool.dtype), _dev(k_pool, "k_pool"),
        _dev(v_pool, "v_pool", k_pool.dtype, k_pool.shape),
        _dev(summaries, "summaries", k_pool.dtype, (B, Hkv, block_table.shape[1], D)),
        int(top_k), 1 if refresh_last_block else 0,
        _dev(block_idx, "block_idx", torch.int32, (B, Hkv, top_k)),
        _dev(out, "out", torch.float32, (B, Hq, D)), _dev(lse, "lse", torch.float32, (B, Hq)),
        _stream(stream)), "ksa_paged_block_topk_decode")
    return out, lse, block_idx


def ksa_paged_dense_decode(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                           block_table: torch.Tensor, seq_lens: torch.Tensor,
                           max_len: Optional[int] = None, out=None, lse=None,
                           want_lse: bool = True, sm_scale: float = 0.0, workspace=None,
                           stream=None):
    """Exact attention of every query head over its sequence's T_b tokens of
    a paged cache.  Returns (out [B,Hq,D] fp32, lse [B,Hq] fp32 or None)."""
    lib = load_library()
    prob, pg = _paged_args(q, k_pool, block_table, seq_lens, max_len, sm_scale)
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    ws, pws, nws = _workspace(prob, KSA_OP_PAGED_DENSE, 0, q.device, workspace)
    _check(lib.ksa_paged_dense_decode(
        ctypes.byref(prob), ctypes.byref(pg), _dev(q, "q", k_pool.dtype), _dev(k_pool, "k_pool"),
        _dev(v_pool, "v_pool", k_pool.dtype, k_pool.shape),
        _dev(out, "out", torch.float32, (B, Hq, D)), _dev(lse, "lse", torch.float32, (B, Hq)),
        pws, nws, _stream(stream)), "ksa_paged_dense_decode")
    return out, lse


# ----------------------------------------------------------------------------- variants, recall
def ksa_select_topk_ex(q: torch.Tensor, summaries: torch.Tensor, seq_len: int, block_size: int,
                       top_k: int, aggregate: int = KSA_AGG_SUM, force_last_block: bool = False,
                       max_seq_len: Optional[int] = None, block_idx=None, block_scores=None,
                       want_scores: bool = False, sm_scale: float = 0.0, workspace=None,
                       stream=None):
    """ksa_select_topk with the selection variants: aggregate KSA_AGG_MAX ranks
    a block by its largest head, force_last_block always keeps the newest block."""
    lib = load_library()
    B, Hkv, nbcap, D = summaries.shape
    Tcap = max_seq_len if max_seq_len is not None else nbcap * block_size
    prob = Problem(B, q.shape[1], Hkv, D, int(seq_len), int(Tcap), int(block_size),
                   _dtype_code(summaries), float(sm_scale))
    nb = nblocks(seq_len, block_size)
    keff = min(top_k, nb)
    if block_idx is None:
        block_idx = torch.empty((B, Hkv, keff), dtype=torch.int32, device=q.device)
    if want_scores and block_scores is None:
        block_scores = torch.empty((B, Hkv, nb), dtype=torch.float32, device=q.device)
    opts = SelectOptions(int(top_k), int(aggregate), 1 if force_last_block else 0)
    ws, pws, nws = _workspace(prob, KSA_OP_SELECT_TOPK, top_k, q.device, workspace)
    _check(lib.ksa_select_topk_ex(ctypes.byref(prob),
                                  _dev(q, "q", summaries.dtype, (B, prob.num_q_heads, D)),
                                  _dev(summaries, "summaries"), ctypes.byref(opts),
                                  _dev(block_idx, "block_idx", torch.int32, (B, Hkv, keff)),
                                  _dev(block_scores, "block_scores", torch.float32, (B, Hkv, nb)),
                                  pws, nws, _stream(stream)), "ksa_select_topk_ex")
    return (block_idx, block_scores) if block_scores is not None else block_idx


def ksa_paged_select_topk_ex(q: torch.Tensor, summaries: torch.Tensor, block_table: torch.Tensor,
                             seq_lens: torch.Tensor, block_size: int, top_k: int,
                             aggregate: int = KSA_AGG_SUM, force_last_block: bool = False,
                             max_len: Optional[int] = None, block_idx=None, block_scores=None,
                             want_scores: bool = False, sm_scale: float = 0.0, workspace=None,
                             stream=None):
    """ksa_select_topk_ex for a paged cache: every row ranks its own NB_b
    blocks of summaries [B,Hkv,max_blocks,D]; block_idx [B,Hkv,top_k] int32
    (ascending, -1 past k_eff_b); force_last_block keeps each row's newest."""
    lib = load_library()
    B, Hkv, max_blocks, D = summaries.shape
    if max_len is None:
        max_len = int(seq_lens.max().item())
    prob = Problem(B, q.shape[1], Hkv, D, int(max_len), max_blocks * int(block_size),
                   int(block_size), _dtype_code(summaries), float(sm_scale))
    pg = PagedKv(_dev(block_table, "block_table", torch.int32, (B, max_blocks)),
                 _dev(seq_lens, "seq_lens", torch.int32, (B,)), max_blocks, 1)
    nb = nblocks(int(max_len), block_size)
    if block_idx is None:
        block_idx = torch.empty((B, Hkv, top_k), dtype=torch.int32, device=q.device)
    if want_scores and block_scores is None:
        block_scores = torch.empty((B, Hkv, nb), dtype=torch.float32, device=q.device)
    opts = SelectOptions(int(top_k), int(aggregate), 1 if force_last_block else 0)
    ws, pws, nws = _workspace(prob, KSA_OP_SELECT_TOPK, top_k, q.device, workspace)
    _check(lib.ksa_paged_select_topk_ex(ctypes.byref(prob), ctypes.byref(pg),
                                        _dev(q, "q", summaries.dtype, (B, prob.num_q_heads, D)),
                                        _dev(summaries, "summaries"), ctypes.byref(opts),
                                        _dev(block_idx, "block_idx", torch.int32, (B, Hkv, top_k)),
                                        _dev(block_scores, "block_scores", torch.float32,
                                             (B, Hkv, nb)),
                                        pws, nws, _stream(stream)), "ksa_paged_select_topk_ex")
    return (block_idx, block_scores) if block_scores is not None else block_idx


def ksa_vote_select_heads(q: torch.Tensor, k: torch.Tensor, seq_len: int, token_budget: int,
                          recent_window: int, voting_heads, token_idx=None, votes=None,
                          want_votes: bool = False, workspace=None, stream=None):
    """ksa_vote_select with only the listed query heads voting."""
    lib = load_library()
    prob = make_problem(q, k, seq_len)
    B = q.shape[0]
    n_out = min(token_budget, seq_len)
    heads = (ctypes.c_int32 * len(voting_heads))(*[int(h) for h in voting_heads])
    if token_idx is None:
        token_idx = torch.empty((B, n_out), dtype=torch.int32, device=q.device)
    if want_votes and votes is None:
        votes = torch.empty((B, seq_len), dtype=torch.uint8, device=q.device)
    ws, pws, nws = _workspace(prob, KSA_OP_VOTE_SELECT, token_budget, q.device, workspace)
    _check(lib.ksa_vote_select_heads(ctypes.byref(prob), _dev(q, "q", k.dtype), _dev(k, "k"),
                                     int(token_budget), int(recent_window),
                                     ctypes.cast(heads, ctypes.c_void_p), len(voting_heads),
                                     _dev(token_idx, "token_idx", torch.int32, (B, n_out)),
                                     _dev(votes, "votes", torch.uint8, (B, seq_len)), pws, nws,
                                     _stream(stream)), "ksa_vote_select_heads")
    return (token_idx, votes) if votes is not None else token_idx


def ksa_attention_recall(lse_selected: torch.Tensor, lse_dense: torch.Tensor, recall=None,
                         stream=None) -> torch.Tensor:
    """Share of each head's dense softmax mass the selection covers:
    exp(lse_selected - lse_dense), elementwise over [B, Hq]."""
    lib = load_library()
    if recall is None:
        recall = torch.empty_like(lse_selected)
    n = lse_selected.numel()
    _check(lib.ksa_attention_recall(_dev(lse_selected, "lse_selected", torch.float32),
                                    _dev(lse_dense, "lse_dense", torch.float32, lse_selected.shape),
                                    _dev(recall, "recall", torch.float32, lse_selected.shape), int(n),
                                    _stream(stream)), "ksa_attention_recall")
    return recall


def ksa_vote_layer_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seq_len: int,
                          token_budget: int, recent_window: int, out=None, lse=None,
                          want_lse: bool = True, token_idx=None, votes=None,
                          want_votes: bool = False, sm_scale: float = 0.0, workspace=None,
                          stream=None):
    """A token-selection layer: dense attention of every head plus the
    vote-union set from the same logits.  Returns (out [B,Hq,D] fp32,
    lse [B,Hq] or None, token_idx [B,min(N,T)] int32, votes [B,T] uint8 or None)."""
    lib = load_library()
    prob = make_problem(q, k, seq_len, 1, sm_scale)
    B, Hq, D = q.shape
    n_out = min(token_budget, seq_len)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if token_idx is None:
        token_idx = torch.empty((B, n_out), dtype=torch.int32, device=q.device)
    if want_votes and votes is None:
        votes = torch.empty((B, seq_len), dtype=torch.uint8, device=q.device)
    ws, pws, nws = _workspace(prob, KSA_OP_VOTE_LAYER, token_budget, q.device, workspace)
    _check(lib.ksa_vote_layer_decode(
        ctypes.byref(prob), _dev(q, "q", k.dtype), _dev(k, "k"), _dev(v, "v", k.dtype, k.shape),
        int(token_budget), int(recent_window), _dev(out, "out", torch.float32, (B, Hq, D)),
        _dev(lse, "lse", torch.float32, (B, Hq)),
        _dev(token_idx, "token_idx", torch.int32, (B, n_out)),
        _dev(votes, "votes", torch.uint8, (B, seq_len)), pws, nws, _stream(stream)),
        "ksa_vote_layer_decode")
    return out, lse, token_idx, votes


def ksa_vote_select_per_head(q: torch.Tensor, k: torch.Tensor, seq_len: int, token_budget: int,
                             recent_window: int, token_idx=None, workspace=None, stream=None):
    """Per-head sets [B, Hq, min(N,T)] int32: every head's own picks plus the
    recency window (attend them with ksa_sparse_decode, KSA_SEL_HEAD_TOKENS)."""
    lib = load_library()
    prob = make_problem(q, k, seq_len)
    B, Hq = q.shape[0], q.shape[1]
    n_out = min(token_budget, seq_len)
    if token_idx is None:
        token_idx = torch.empty((B, Hq, n_out), dtype=torch.int32, device=q.device)
    ws, pws, nws = _workspace(prob, KSA_OP_VOTE_SELECT, token_budget, q.device, workspace)
    _check(lib.ksa_vote_select_per_head(ctypes.byref(prob), _dev(q, "q", k.dtype), _dev(k, "k"),
                                        int(token_budget), int(recent_window),
                                        _dev(token_idx, "token_idx", torch.int32, (B, Hq, n_out)),
                                        pws, nws, _stream(stream)), "ksa_vote_select_per_head")
    return token_idx


def ksa_paged_vote_select(q: torch.Tensor, k_pool: torch.Tensor, block_table: torch.Tensor,
                          seq_lens: torch.Tensor, token_budget: int, recent_window: int,
                          max_len: Optional[int] = None, token_idx=None, votes=None,
                          want_votes: bool = False, workspace=None, stream=None):
    """The vote-union set on a paged cache with per-sequence lengths:
    token_idx [B, min(N, T_max)] int32 (-1 padded), votes [B, T_max] uint8."""
    lib = load_library()
    prob, pg = _paged_args(q, k_pool, block_table, seq_lens, max_len, 0.0)
    B, T = q.shape[0], prob.seq_len
    n_out = min(token_budget, T)
    if token_idx is None:
        token_idx = torch.empty((B, n_out), dtype=torch.int32, device=q.device)
    if want_votes and votes is None:
        votes = torch.empty((B, T), dtype=torch.uint8, device=q.device)
    ws, pws, nws = _workspace(prob, KSA_OP_VOTE_SELECT, token_budget, q.device, workspace)
    _check(lib.ksa_paged_vote_select(ctypes.byref(prob), ctypes.byref(pg),
                                     _dev(q, "q", k_pool.dtype), _dev(k_pool, "k_pool"),
                                     int(token_budget), int(recent_window),
                                     _dev(token_idx, "token_idx", torch.int32, (B, n_out)),
                                     _dev(votes, "votes", torch.uint8, (B, T)), pws, nws,
                                     _stream(stream)), "ksa_paged_vote_select")
    return (token_idx, votes) if votes is not None else token_idx


def ksa_paged_vote_select_heads(q: torch.Tensor, k_pool: torch.Tensor, block_table: torch.Tensor,
                                seq_lens: torch.Tensor, token_budget: int, recent_window: int,
                                voting_heads, max_len: Optional[int] = None, token_idx=None,
                                votes=None, want_votes: bool = False, workspace=None,
                                stream=None):
    """ksa_paged_vote_select with only the listed query heads voting."""
    lib = load_library()
    prob, pg = _paged_args(q, k_pool, block_table, seq_lens, max_len, 0.0)
    B, T = q.shape[0], prob.seq_len
    n_out = min(token_budget, T)
    heads = (ctypes.c_int32 * len(voting_heads))(*[int(h) for h in voting_heads])
    if token_idx is None:
        token_idx = torch.empty((B, n_out), dtype=torch.int32, device=q.device)
    if want_votes and votes is None:
        votes = torch.empty((B, T), dtype=torch.uint8, device=q.device)
    ws, pws, nws = _workspace(prob, KSA_OP_VOTE_SELECT, token_budget, q.device, workspace)
    _check(lib.ksa_paged_vote_select_heads(ctypes.byref(prob), ctypes.byref(pg),
                                           _dev(q, "q", k_pool.dtype), _dev(k_pool, "k_pool"),
                                           int(token_budget), int(recent_window),
                                           ctypes.cast(heads, ctypes.c_void_p), len(voting_heads),
                                           _dev(token_idx, "token_idx", torch.int32, (B, n_out)),
                                           _dev(votes, "votes", torch.uint8, (B, T)), pws, nws,
                                           _stream(stream)), "ksa_paged_vote_select_heads")
    return (token_idx, votes) if votes is not None else token_idx


def ksa_paged_vote_select_per_head(q: torch.Tensor, k_pool: torch.Tensor,
                                   block_table: torch.Tensor, seq_lens: torch.Tensor,
                                   token_budget: int, recent_window: int,
                                   max_len: Optional[int] = None, token_idx=None, workspace=None,
                                   stream=None):
    """Per-head sets on a paged cache: token_idx [B, Hq, min(N, T_max)] int32
    (a sequence no longer than N: its T_b tokens, then -1), for
    ksa_paged_sparse_decode with KSA_SEL_HEAD_TOKENS."""
    lib = load_library()
    prob, pg = _paged_args(q, k_pool, block_table, seq_lens, max_len, 0.0)
    B, Hq = q.shape[0], q.shape[1]
    n_out = min(token_budget, prob.seq_len)
    if token_idx is None:
        token_idx = torch.empty((B, Hq, n_out), dtype=torch.int32, device=q.device)
    ws, pws, nws = _workspace(prob, KSA_OP_VOTE_SELECT, token_budget, q.device, workspace)
    _check(lib.ksa_paged_vote_select_per_head(ctypes.byref(prob), ctypes.byref(pg),
                                              _dev(q, "q", k_pool.dtype), _dev(k_pool, "k_pool"),
                                              int(token_budget), int(recent_window),
                                              _dev(token_idx, "token_idx", torch.int32,
                                                   (B, Hq, n_out)),
                                              pws, nws, _stream(stream)),
           "ksa_paged_vote_select_per_head")
    return token_idx


def ksa_paged_vote_layer_decode(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                                block_table: torch.Tensor, seq_lens: torch.Tensor,
                                token_budget: int, recent_window: int,
                                max_len: Optional[int] = None, out=None, lse=None,
                                want_lse: bool = True, token_idx=None, votes=None,
                                want_votes: bool = False, sm_scale: float = 0.0, workspace=None,
                                stream=None):
    """A token-selection layer on a paged cache: paged dense attention plus
    the paged vote-union set from the same logits.  Returns (out [B,Hq,D]
    fp32, lse [B,Hq] or None, token_idx [B,min(N,T_max)] int32 (-1 padded),
    votes [B,T_max] uint8 or None)."""
    lib = load_library()
    prob, pg = _paged_args(q, k_pool, block_table, seq_lens, max_len, sm_scale)
    B, Hq, D = q.shape
    T = prob.seq_len
    n_out = min(token_budget, T)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if token_idx is None:
        token_idx = torch.empty((B, n_out), dtype=torch.int32, device=q.device)
    if want_votes and votes is None:
        votes = torch.empty((B, T), dtype=torch.uint8, device=q.device)
    ws, pws, nws = _workspace(prob, KSA_OP_PAGED_VOTE_LAYER, token_budget, q.device, workspace)
    _check(lib.ksa_paged_vote_layer_decode(
        ctypes.byref(prob), ctypes.byref(pg), _dev(q, "q", k_pool.dtype), _dev(k_pool, "k_pool"),
        _dev(v_pool, "v_pool", k_pool.dtype, k_pool.shape), int(token_budget), int(recent_window),
        _dev(out, "out", torch.float32, (B, Hq, D)), _dev(lse, "lse", torch.float32, (B, Hq)),
        _dev(token_idx, "token_idx", torch.int32, (B, n_out)),
        _dev(votes, "votes", torch.uint8, (B, T)), pws, nws, _stream(stream)),
        "ksa_paged_vote_layer_decode")
    return out, lse, token_idx, votes


def ksa_paged_sparse_decode(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                            block_table: torch.Tensor, seq_lens: torch.Tensor, idx: torch.Tensor,
                            kind: int = KSA_SEL_TOKENS, max_len: Optional[int] = None, out=None,
                            lse=None, want_lse: bool = True, sm_scale: float = 0.0,
                            workspace=None, stream=None):
    """Attention over selected blocks ([B,Hkv,count]), a shared token list
    ([B,count]) or a list per query head ([B,Hq,count]) of a paged cache;
    negative entries are skipped."""
    lib = load_library()
    prob, pg = _paged_args(q, k_pool, block_table, seq_lens, max_len, sm_scale)
    B, Hq, D = q.shape
    count = idx.shape[-1]
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    ishape = {KSA_SEL_BLOCKS: (B, k_pool.shape[1], count), KSA_SEL_TOKENS: (B, count),
              KSA_SEL_HEAD_TOKENS: (B, Hq, count)}[kind]
    sel = Selection(int(kind), _dev(idx, "idx", torch.int32, ishape), int(count))
    op = {KSA_SEL_BLOCKS: KSA_OP_SPARSE_BLOCKS, KSA_SEL_TOKENS: KSA_OP_SPARSE_TOKENS,
          KSA_SEL_HEAD_TOKENS: KSA_OP_SPARSE_HEAD_TOKENS}[kind]
    ws, pws, nws = _workspace(prob, op, count, q.device, workspace)
    _check(lib.ksa_paged_sparse_decode(ctypes.byref(prob), ctypes.byref(pg),
                                       _dev(q, "q", k_pool.dtype), _dev(k_pool, "k_pool"),
                                       _dev(v_pool, "v_pool", k_pool.dtype, k_pool.shape),
                                       ctypes.byref(sel), _dev(out, "out", torch.float32, (B, Hq, D)),
                                       _dev(lse, "lse", torch.float32, (B, Hq)), pws, nws,
                                       _stream(stream)), "ksa_paged_sparse_decode")
    return out, lse
