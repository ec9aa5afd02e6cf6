"""fp64 CPU oracle for block top-k sparse decode attention and vote-union selection.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
library never loads it, and this package never imports the product package:
the two share nothing but the seeded input generators, which hold none of the
method's arithmetic.

The arithmetic lives in ``ksa_oracle.c`` (plain C, fp64, OpenMP over
independent rows); this module compiles it with gcc on first use and wraps it
for numpy arrays.  Every function states the page passage it follows:

* Kinetics explainer (news.43u.com.cn), section 五: history tokens are split into
  blocks, each block gets its mean representation, the K' most relevant blocks
  are selected and attended.
* Kinetics explainer, section 四: dense attention attends every history token.
* LessIsMore explainer (techwalker.com), section 二: equal votes per head, per-token
  vote totals, ranking by votes, and a 75 % / 25 % split of the token budget
  between voted history and the most recent tokens.
* LessIsMore explainer, section 五: the selection layer computes the full score
  matrix, each head picks, picks are aggregated and sorted, the most recent tokens
  are appended, and the set is shared by all heads.

bf16 tensors are passed as ``uint16`` arrays holding the raw bit patterns;
fp32 tensors as ``float32`` arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ksa_oracle.c")
_DEFAULT_LIB = os.path.join(_HERE, "libksa_oracle.so")
# KSA_ORACLE_LIB points the shim at another build of ksa_oracle.c (the mutant
# tests use it to check that the pins catch planted mistakes).
_LIB_PATH = os.environ.get("KSA_ORACLE_LIB", _DEFAULT_LIB)
_lock = threading.Lock()
_lib = None

F32, BF16 = 0, 1


def build(force: bool = True, src: str = _SRC, out: str = _DEFAULT_LIB) -> str:
    """Compile ksa_oracle.c into libksa_oracle.so (gcc, -O2, OpenMP, no fast-math)."""
    if _LIB_PATH != _DEFAULT_LIB and out == _DEFAULT_LIB:
        return _LIB_PATH  # an explicitly chosen build is used as is
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
           "-ffp-contract=off", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("Hq", ctypes.c_int64), ("Hkv", ctypes.c_int64),
                ("D", ctypes.c_int64), ("T", ctypes.c_int64), ("Tcap", ctypes.c_int64),
                ("Bs", ctypes.c_int64), ("dtype", ctypes.c_int32), ("sm_scale", ctypes.c_double)]


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            lib = ctypes.CDLL(_LIB_PATH)
            P = ctypes.c_void_p
            I = ctypes.c_int64
            S = ctypes.POINTER(Shape)
            lib.orc_block_summaries.argtypes = [S, P, I, I, P, P]
            lib.orc_group_scores.argtypes = [S, P, P, P, P]
            lib.orc_group_scores_max.argtypes = [S, P, P, P, P]
            lib.orc_topk.argtypes = [I, I, P, I, P]
            lib.orc_topk.restype = I
            lib.orc_attend_blocks.argtypes = [S, P, P, P, P, I, P, P]
            lib.orc_attend_tokens.argtypes = [S, P, P, P, P, I, P, P]
            lib.orc_attend_dense.argtypes = [S, P, P, P, P, P]
            lib.orc_head_logits.argtypes = [S, P, P, P]
            lib.orc_votes.argtypes = [I, I, I, P, I, I, P]
            lib.orc_set_from_votes.argtypes = [I, I, P, I, I, P]
            lib.orc_set_from_votes.restype = I
            _lib = lib
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    raise TypeError("oracle takes float32 arrays or uint16 bf16 bit patterns, got %s" % a.dtype)


def _shape(q, k, T, Bs=1, sm_scale=0.0):
    B, Hq, D = q.shape
    Bk, Hkv, Tcap, Dk = k.shape
    assert B == Bk and D == Dk and Hq % Hkv == 0 and 1 <= T <= Tcap
    return Shape(B, Hq, Hkv, D, T, Tcap, Bs, _dtype_code(k), float(sm_scale))


def nblocks(n: int, bs: int) -> int:
    return (n + bs - 1) // bs


def block_summaries(k: np.ndarray, T: int, Bs: int, first_block: int = 0, num_blocks: int | None = None,
                    out: np.ndarray | None = None, want_f64: bool = False):
    """Mean key of each block, stored rounded-to-nearest-even in the KV dtype
    (Kinetics explainer, section 五).  Returns summaries [B,Hkv,ceil(Tcap/Bs),D]
    (and the unrounded fp64 means when want_f64)."""
    lib = _load()
    B, Hkv, Tcap, D = k.shape
    if num_blocks is None:
        num_blocks = nblocks(T, Bs) - first_block
    s = Shape(B, Hkv, Hkv, D, T, Tcap, Bs, _dtype_code(k), 0.0)
    nbcap = nblocks(Tcap, Bs)
    if out is None:
        out = np.zeros((B, Hkv, nbcap, D), dtype=k.dtype)
    m64 = np.zeros((B, Hkv, nbcap, D), dtype=np.float64) if want_f64 else None
    lib.orc_block_summaries(ctypes.byref(s), _ptr(k), first_block, num_blocks, _ptr(out), _ptr(m64))
    return (out, m64) if want_f64 else out


def gather_pages(pool: np.ndarray, block_table: np.ndarray, b: int, T: int, Bs: int) -> np.ndarray:
    """Tokens [0, T) of sequence b of a paged cache, as a contiguous
    [1, Hkv, T, D] array (Kinetics explainer, section 五: the method works
    with a paged KV cache, its blocks being the pages).  Page
    block_table[b, j] of the pool [num_pages, Hkv, Bs, D] holds tokens
    [j*Bs, (j+1)*Bs) of the sequence for every KV head; the paged result is
    the contiguous definition applied to these tokens."""
    nb = nblocks(T, Bs)
    pages = pool[np.asarray(block_table)[b, :nb]]              # [nb, Hkv, Bs, D]
    seq = pages.transpose(1, 0, 2, 3).reshape(pool.shape[1], nb * Bs, pool.shape[3])
    return np.ascontiguousarray(seq[None, :, :T])


def group_scores(q: np.ndarray, summaries: np.ndarray, T: int, Bs: int, sm_scale: float = 0.0,
                 Tcap: int | None = None, aggregate: str = "sum"):
    """(raw, scaled) block relevance [B,Hkv,NB] from the stored summaries
    (Kinetics explainer, section 五).  raw = sum over the group's heads of
    q_h . summary (ranking key); scaled = sm_scale * raw / G.  aggregate="max"
    is the selection variant that ranks a block by its most interested head:
    raw = max over the group's heads of q_h . summary, scaled = sm_scale * raw."""
    lib = _load()
    B, Hq, D = q.shape
    Bs_, Hkv, nbcap, Ds = summaries.shape
    if Tcap is None:
        Tcap = nbcap * Bs
    assert nblocks(Tcap, Bs) == nbcap
    s = Shape(B, Hq, Hkv, D, T, Tcap, Bs, _dtype_code(summaries), float(sm_scale))
    nb = nblocks(T, Bs)
    raw = np.zeros((B, Hkv, nb), np.float64)
    scaled = np.zeros((B, Hkv, nb), np.float64)
    fn = lib.orc_group_scores_max if aggregate == "max" else lib.orc_group_scores
    fn(ctypes.byref(s), _ptr(q), _ptr(summaries), _ptr(raw), _ptr(scaled))
    return raw, scaled


def topk_with_block(scores: np.ndarray, k: int, forced: int) -> np.ndarray:
    """The forced-local-block selection variant: block `forced` (the one
    holding the newest token) is always kept, and the other min(k, n) - 1
    are the first ones of the remaining blocks by (score desc, index asc).
    Returned ascending, like topk."""
    rest = np.array(scores, dtype=np.float64, copy=True)
    rest[..., forced] = np.inf
    return topk(rest, k)


def topk(scores: np.ndarray, k: int) -> np.ndarray:
    """First min(k, n) indices per row in (score desc, index asc) order,
    returned ascending (Kinetics explainer, section 五)."""
    lib = _load()
    scores = np.ascontiguousarray(scores, dtype=np.float64)
    lead = scores.shape[:-1]
    n = scores.shape[-1]
    rows = int(np.prod(lead)) if lead else 1
    keff = min(k, n)
    out = np.zeros(lead + (keff,), np.int32)
    lib.orc_topk(rows, n, _ptr(scores), k, _ptr(out))
    return out


def attend_blocks(q, k, v, T: int, Bs: int, block_idx: np.ndarray, sm_scale: float = 0.0):
    """Exact softmax attention over the tokens of the selected blocks
    (Kinetics explainer, section 五).  block_idx [B,Hkv,count].  Returns
    (out [B,Hq,D] fp64, lse [B,Hq] fp64)."""
    lib = _load()
    s = _shape(q, k, T, Bs, sm_scale)
    block_idx = np.ascontiguousarray(block_idx, dtype=np.int32)
    count = block_idx.shape[-1]
    out = np.zeros(q.shape, np.float64)
    lse = np.zeros(q.shape[:2], np.float64)
    lib.orc_attend_blocks(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(block_idx), count,
                          _ptr(out), _ptr(lse))
    return out, lse


def attend_tokens(q, k, v, T: int, token_idx: np.ndarray, sm_scale: float = 0.0):
    """Exact softmax attention of every head of sequence b over token_idx[b]
    (LessIsMore explainer, section 五: one set shared by all heads)."""
    lib = _load()
    s = _shape(q, k, T, 1, sm_scale)
    token_idx = np.ascontiguousarray(token_idx, dtype=np.int32)
    count = token_idx.shape[-1]
    out = np.zeros(q.shape, np.float64)
    lse = np.zeros(q.shape[:2], np.float64)
    lib.orc_attend_tokens(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(token_idx), count,
                          _ptr(out), _ptr(lse))
    return out, lse


def attend_dense(q, k, v, T: int, sm_scale: float = 0.0):
    """Exact softmax attention over all T tokens (Kinetics explainer, section 四)."""
    lib = _load()
    s = _shape(q, k, T, 1, sm_scale)
    out = np.zeros(q.shape, np.float64)
    lse = np.zeros(q.shape[:2], np.float64)
    lib.orc_attend_dense(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse))
    return out, lse


def attention_recall(q, k, T: int, tokens_per_head, sm_scale: float = 0.0):
    """Attention recall (LessIsMore explainer, sections 四 and 五): for every
    query head, the sum of its dense softmax weights over the tokens a
    selection keeps.  tokens_per_head(b, h) -> iterable of token ids.
    Returns [B, Hq] fp64."""
    B, Hq, D = q.shape
    scale = sm_scale if sm_scale > 0 else 1.0 / np.sqrt(D)
    lg = head_logits(q, k, T) * scale                       # [B, Hq, T]
    m = lg.max(axis=-1, keepdims=True)
    p = np.exp(lg - m)
    p /= p.sum(axis=-1, keepdims=True)
    out = np.zeros((B, Hq), np.float64)
    for b in range(B):
        for h in range(Hq):
            out[b, h] = p[b, h, sorted(set(int(t) for t in tokens_per_head(b, h)))].sum()
    return out


def head_logits(q, k, T: int):
    """Full score matrix q_h . k_t for every head and every t < T
    (LessIsMore explainer, section 五).  [B,Hq,T] fp64, unscaled."""
    lib = _load()
    s = _shape(q, k, T)
    out = np.zeros((q.shape[0], q.shape[1], T), np.float64)
    lib.orc_head_logits(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(out))
    return out


def votes(logits: np.ndarray, N: int, W: int, heads=None) -> np.ndarray:
    """Per-token vote counts [B,T] int32 (LessIsMore explainer, section 二):
    every head picks its first N-W history tokens by (logit desc, t asc).
    `heads` (a list of head indices) restricts the vote to those heads: one
    head is the LessIsMore explainer's random-head ablation (section 五),
    where a single head's picks serve every head."""
    lib = _load()
    if heads is not None:
        logits = logits[:, list(heads)]
    logits = np.ascontiguousarray(logits, dtype=np.float64)
    B, Hq, T = logits.shape
    out = np.zeros((B, T), np.int32)
    lib.orc_votes(B, Hq, T, _ptr(logits), N, W, _ptr(out))
    return out


def set_from_votes(vote_counts: np.ndarray, N: int, W: int) -> np.ndarray:
    """Shared token set [B, min(N,T)] from vote counts (LessIsMore explainer,
    sections 二 and 五): top N-W history tokens by (votes desc, t asc), ascending,
    then the W most recent tokens."""
    lib = _load()
    vote_counts = np.ascontiguousarray(vote_counts, dtype=np.int32)
    B, T = vote_counts.shape
    out = np.zeros((B, min(N, T)), np.int32)
    lib.orc_set_from_votes(B, T, _ptr(vote_counts), N, W, _ptr(out))
    return out


def head_sets(logits: np.ndarray, N: int, W: int) -> np.ndarray:
    """The per-head-sets ablation (LessIsMore explainer, section 五: each
    head keeps its own set): for every head, its first N-W history tokens by
    (logit desc, t asc), ascending, then the W most recent tokens; all of
    [0, T) when T <= N.  logits [B,Hq,T] -> [B,Hq,min(N,T)] int32."""
    B, Hq, T = logits.shape
    if T <= N:
        return np.broadcast_to(np.arange(T, dtype=np.int32), (B, Hq, T)).copy()
    C, Kv = T - W, N - W
    out = np.zeros((B, Hq, N), np.int32)
    for b in range(B):
        for h in range(Hq):
            picks = topk(logits[b, h, :C][None], Kv)[0]
            out[b, h] = np.concatenate([picks, np.arange(C, T)])
    return out


def attend_head_tokens(q, k, v, T: int, token_idx: np.ndarray, sm_scale: float = 0.0):
    """Exact softmax attention of every query head over its own list
    token_idx[b, h] (the per-head-sets ablation): the shared-list attention
    of a one-head problem per (b, h).  Returns (out [B,Hq,D], lse [B,Hq])."""
    B, Hq, D = q.shape
    G = Hq // k.shape[1]
    out = np.zeros(q.shape, np.float64)
    lse = np.zeros((B, Hq), np.float64)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            o, l = attend_tokens(np.ascontiguousarray(q[b:b + 1, h:h + 1]),
                                 np.ascontiguousarray(k[b:b + 1, g:g + 1]),
                                 np.ascontiguousarray(v[b:b + 1, g:g + 1]), T,
                                 np.ascontiguousarray(token_idx[b:b + 1, h]), sm_scale)
            out[b, h], lse[b, h] = o[0, 0], l[0, 0]
    return out, lse


def vote_select(q, k, T: int, N: int, W: int, heads=None):
    """Whole vote-union selection: returns (token_idx [B,min(N,T)], votes [B,T]);
    `heads` as in votes."""
    if T > N:
        lg = head_logits(q, k, T)
    else:
        lg = np.zeros((q.shape[0], q.shape[1], T), np.float64)
    vc = votes(lg, N, W, heads)
    return set_from_votes(vc, N, W), vc
