"""ksa_sparse_decode_noalloc, the workspace-free variant of ksa_sparse_decode
for callers that cannot allocate: called through the C ABI with outputs the
test allocated beforehand, it must equal ksa_sparse_decode (the same kernels
and launch plan, with the library's own per-GPU scratch array in place of the
caller's workspace) bit for bit, on consecutive calls of decreasing size, for
every selection kind and for the default and a side stream."""
import ctypes

import pytest
import torch

import sparse_attention_decode_ksa_amd as ksa
from sparse_attention_decode_ksa_amd.inputs import small_workload
from test_gpu_parity import DEV, gpu_inputs

pytestmark = pytest.mark.gpu


def _case(B, Hq, Hkv, T, kind, count, seed):
    w = small_workload(B=B, Hq=Hq, Hkv=Hkv, D=128, T=T, Bs=16, dtype="bf16", top_k=count, seed=seed)
    q, k, v = gpu_inputs(w)
    if kind == ksa.KSA_SEL_BLOCKS:
        s = torch.zeros((B, Hkv, ksa.nblocks(w.cap, 16), 128), dtype=k.dtype, device=DEV)
        ksa.ksa_block_summaries(k, s, T, 16)
        idx = ksa.ksa_select_topk(q, s, T, 16, count, max_seq_len=w.cap)
        bs = 16
    elif kind == ksa.KSA_SEL_TOKENS:
        idx = ksa.ksa_vote_select(q, k, T, count, count // 4)
        bs = 1
    else:
        idx = ksa.ksa_vote_select_per_head(q, k, T, count, count // 4)
        bs = 1
    return w, q, k, v, idx, bs


def _noalloc(lib, w, q, k, v, idx, kind, bs, stream):
    """One call through the C ABI; out and lse are allocated before it."""
    prob = ksa.make_problem(q, k, w.T, bs)
    out = torch.full((w.B, w.Hq, 128), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((w.B, w.Hq), float("nan"), dtype=torch.float32, device=DEV)
    sel = ksa.Selection(kind, idx.data_ptr(), idx.shape[-1])
    V = lambda t: ctypes.c_void_p(t.data_ptr())
    st = lib.ksa_sparse_decode_noalloc(ctypes.byref(prob), V(q), V(k), V(v), ctypes.byref(sel),
                                       V(out), V(lse), ctypes.c_void_p(stream))
    assert st == ksa.KSA_OK, ksa.ksa_status_string(st)
    return prob, out, lse


@pytest.mark.parametrize("kind", [ksa.KSA_SEL_TOKENS, ksa.KSA_SEL_BLOCKS, ksa.KSA_SEL_HEAD_TOKENS],
                         ids=["tokens", "blocks", "head_tokens"])
@pytest.mark.parametrize("side_stream", [False, True], ids=["null_stream", "side_stream"])
def test_noalloc_equals_sparse_decode_on_consecutive_calls(kind, side_stream):
    lib = ksa.load_library()
    op = {ksa.KSA_SEL_BLOCKS: ksa.KSA_OP_SPARSE_BLOCKS, ksa.KSA_SEL_TOKENS: ksa.KSA_OP_SPARSE_TOKENS,
          ksa.KSA_SEL_HEAD_TOKENS: ksa.KSA_OP_SPARSE_HEAD_TOKENS}[kind]
    # a larger call, then a smaller one: the second finds the first's scratch
    big = _case(4, 16, 4, 12000, kind, 2048 if kind != ksa.KSA_SEL_BLOCKS else 96, seed=71)
    small = _case(1, 8, 2, 3000, kind, 512 if kind != ksa.KSA_SEL_BLOCKS else 40, seed=72)
    stream = torch.cuda.Stream(device=DEV) if side_stream else None
    for w, q, k, v, idx, bs in (big, small, big):
        prob = ksa.make_problem(q, k, w.T, bs)
        need = ksa.ksa_workspace_bytes(prob, op, idx.shape[-1])
        assert 0 < need <= ksa.NOALLOC_SCRATCH_BYTES  # rows are split: the scratch is used
        ref_out, ref_lse = ksa.ksa_sparse_decode(q, k, v, w.T, idx, kind, block_size=bs)
        torch.cuda.synchronize()
        if stream is None:
            _, out, lse = _noalloc(lib, w, q, k, v, idx, kind, bs, 0)
        else:
            with torch.cuda.stream(stream):
                _, out, lse = _noalloc(lib, w, q, k, v, idx, kind, bs, stream.cuda_stream)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)


def test_noalloc_rows_without_splits_and_the_binding():
    """A shape whose rows are not split needs no scratch; the binding's
    wrapper gives the same result as the C call."""
    w, q, k, v, idx, bs = _case(64, 16, 8, 4096, ksa.KSA_SEL_TOKENS, 1024, seed=73)
    prob = ksa.make_problem(q, k, w.T, bs)
    assert ksa.ksa_workspace_bytes(prob, ksa.KSA_OP_SPARSE_TOKENS, 1024) == 0
    ref = ksa.ksa_sparse_decode(q, k, v, w.T, idx, ksa.KSA_SEL_TOKENS)
    got = ksa.ksa_sparse_decode_noalloc(q, k, v, w.T, idx, ksa.KSA_SEL_TOKENS)
    torch.cuda.synchronize()
    assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])
