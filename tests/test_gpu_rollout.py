"""Decode loops: many consecutive steps over a growing cache, and the same
steps captured once in a HIP graph and replayed.

A decode step appends one token per sequence and refreshes only the newest
block's summary (Kinetics explainer, section 五: a block's mean key changes
only while the block is being filled).  Stepping token by token from a
prefill must therefore keep every summary exactly what a full rebuild over
the current length gives, across block boundaries, and each step's
selection and output must match the oracle on that step's own prefix.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_decode_ksa_amd as ksa
from sparse_attention_decode_ksa_amd.inputs import small_workload, to_paged
from parity import check_attention, check_block_selection, check_votes
from test_gpu_parity import DEV, gpu_inputs, np_bits

pytestmark = pytest.mark.gpu


def step_queries(n, B, Hq, D, dtype, seed):
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    return [torch.randn((B, Hq, D), generator=gen, device=DEV).to(dtype) for _ in range(n)]


@pytest.mark.parametrize("G,D,dtype,Bs", [(2, 128, "bf16", 16), (4, 128, "bf16", 16),
                                          (8, 128, "bf16", 32), (1, 64, "f32", 7)])
def test_contiguous_rollout_matches_rebuild_and_oracle(G, D, dtype, Bs):
    T0, S, Hkv, B, top_k = 990, 40, 2, 3, 12
    w = small_workload(B=B, Hq=G * Hkv, Hkv=Hkv, D=D, T=T0 + S, Tcap=T0 + S + Bs, Bs=Bs,
                       dtype=dtype, top_k=top_k, seed=41 + G)
    _, k, v = gpu_inputs(w)
    qs = step_queries(S, B, w.Hq, D, k.dtype, seed=7 + G)
    nbcap = ksa.nblocks(w.cap, Bs)
    s = torch.zeros((B, Hkv, nbcap, D), dtype=k.dtype, device=DEV)
    ksa.ksa_block_summaries(k, s, T0, Bs)  # prefill over T0 tokens
    kb_all, vb_all = np_bits(k), np_bits(v)
    for i, q in enumerate(qs):
        T = T0 + i + 1
        out, lse, idx = ksa.ksa_block_topk_decode(q, k, v, s, T, Bs, top_k, want_block_idx=True)
        if i % 9 == 0 or i == S - 1:  # check a few steps against the oracle in full
            torch.cuda.synchronize()
            nb = ksa.nblocks(T, Bs)
            ref_s = oracle.block_summaries(kb_all, T, Bs)
            np.testing.assert_array_equal(np_bits(s)[:, :, :nb], ref_s[:, :, :nb])
            qb = np_bits(q)
            raw, _ = oracle.group_scores(qb, ref_s, T, Bs, Tcap=w.cap)
            ib = idx.cpu().numpy()
            check_block_selection(ib.reshape(B * Hkv, -1), raw.reshape(B * Hkv, -1), top_k)
            ro, rl = oracle.attend_blocks(qb, kb_all, vb_all, T, Bs, ib)
            check_attention(out.cpu().numpy(), lse.cpu().numpy(), ro, rl)
    torch.cuda.synchronize()
    T = T0 + S
    full = torch.zeros_like(s)
    ksa.ksa_block_summaries(k, full, T, Bs)
    torch.cuda.synchronize()
    nb = ksa.nblocks(T, Bs)
    assert torch.equal(s[:, :, :nb], full[:, :, :nb])


def test_paged_rollout_with_ragged_lengths():
    """Sequences of different lengths each gain one token per step; the
    paged step refreshes each one's own newest block."""
    Bs, S, Hkv, G, D, top_k = 16, 35, 2, 4, 128, 10
    lens0 = [700, 31, 1000, 1]
    cap = (max(lens0) + S + Bs) // Bs * Bs
    w = small_workload(B=len(lens0), Hq=G * Hkv, Hkv=Hkv, D=D, T=cap, Tcap=cap, Bs=Bs,
                       dtype="bf16", top_k=top_k, seed=53)
    _, k, v = gpu_inputs(w)
    kp, vp, table = to_paged(k, v, Bs, seed=54, spare_pages=2)
    seq = torch.tensor(lens0, dtype=torch.int32, device=DEV)
    s = torch.zeros((w.B, Hkv, table.shape[1], D), dtype=k.dtype, device=DEV)
    ksa.ksa_paged_block_summaries(kp, s, table, seq, max_len=cap)  # prefill
    qs = step_queries(S, w.B, w.Hq, D, k.dtype, seed=55)
    kb_all, vb_all = np_bits(k), np_bits(v)
    for i, q in enumerate(qs):
        seq += 1
        out, lse, idx = ksa.ksa_paged_block_topk_decode(q, kp, vp, s, table, seq, top_k,
                                                        max_len=cap, want_block_idx=True)
        if i in (0, 17, S - 1):
            torch.cuda.synchronize()
            lens = seq.cpu().tolist()
            for b, T in enumerate(lens):
                sl = slice(b, b + 1)
                nb = ksa.nblocks(T, Bs)
                ref_s = oracle.block_summaries(kb_all[sl], T, Bs)
                np.testing.assert_array_equal(np_bits(s[sl])[:, :, :nb], ref_s[:, :, :nb])
                qb = np_bits(q[sl])
                raw, _ = oracle.group_scores(qb, ref_s, T, Bs, Tcap=cap)
                ib = idx[sl].cpu().numpy()
                keff = min(top_k, nb)
                assert np.all(ib[..., keff:] == -1)
                check_block_selection(ib[..., :keff].reshape(Hkv, -1), raw.reshape(Hkv, -1), top_k)
                ro, rl = oracle.attend_blocks(qb, kb_all[sl], vb_all[sl], T, Bs,
                                              np.ascontiguousarray(ib[..., :keff]))
                check_attention(out[sl].cpu().numpy(), lse[sl].cpu().numpy(), ro, rl)
    full = torch.zeros_like(s)
    ksa.ksa_paged_block_summaries(kp, full, table, seq, max_len=cap)
    torch.cuda.synchronize()
    assert torch.equal(s, full)


def test_paged_decode_loop_in_one_graph():
    """The paged step captured once and replayed as a decode loop: between
    replays the lengths grow by one on the device (no host sync inside the
    graph's work), and every replay matches an eager step on a copy."""
    Bs, Hkv, G, D, top_k = 16, 2, 4, 128, 8
    lens0 = [400, 129, 16]
    cap = 512
    w = small_workload(B=3, Hq=G * Hkv, Hkv=Hkv, D=D, T=cap, Tcap=cap, Bs=Bs, dtype="bf16",
                       top_k=top_k, seed=61)
    q, k, v = gpu_inputs(w)
    kp, vp, table = to_paged(k, v, Bs, seed=62)
    seq = torch.tensor(lens0, dtype=torch.int32, device=DEV)
    s = torch.zeros((w.B, Hkv, table.shape[1], D), dtype=k.dtype, device=DEV)
    ksa.ksa_paged_block_summaries(kp, s, table, seq, max_len=cap)
    idx = torch.empty((w.B, Hkv, top_k), dtype=torch.int32, device=DEV)
    out = torch.empty((w.B, w.Hq, D), dtype=torch.float32, device=DEV)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=DEV)
    qbuf = q.clone()
    stream = torch.cuda.Stream()

    def step():
        ksa.ksa_paged_block_topk_decode(qbuf, kp, vp, s, table, seq, top_k, max_len=cap,
                                        block_idx=idx, out=out, lse=lse, stream=stream)

    g = torch.cuda.CUDAGraph()
    s_save, seq_save = s.clone(), seq.clone()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        step()  # warm up outside capture
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        step()
    torch.cuda.synchronize()
    s.copy_(s_save)
    seq.copy_(seq_save)
    qs = step_queries(6, w.B, w.Hq, D, k.dtype, seed=63)
    s_e = s_save.clone()
    for rep, nq in enumerate(qs):
        seq.add_(1)
        qbuf.copy_(nq)
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        got = (idx.clone(), out.clone(), lse.clone(), s.clone())
        e_out, e_lse, e_idx = ksa.ksa_paged_block_topk_decode(nq, kp, vp, s_e, table, seq.clone(),
                                                              top_k, max_len=cap,
                                                              want_block_idx=True)
        torch.cuda.synchronize()
        assert torch.equal(got[0], e_idx), rep
        assert torch.equal(got[1], e_out) and torch.equal(got[2], e_lse), rep
        assert torch.equal(got[3], s_e), rep


def test_vote_path_and_selection_layer_graph_replay():
    """The vote select + shared-set attention, and the selection layer,
    captured in HIP graphs and replayed with new queries (eager work in
    between): every replay matches the eager calls bit for bit."""
    N, W = 256, 64
    w = small_workload(B=4, Hq=16, Hkv=4, D=128, T=3000, dtype="bf16", seed=71)
    q, k, v = gpu_inputs(w)
    n_out = min(N, w.T)
    idx = torch.empty((w.B, n_out), dtype=torch.int32, device=DEV)
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device=DEV)
    lse = torch.empty_like(out[..., 0])
    lidx = torch.empty_like(idx)
    lout, llse = torch.empty_like(out), torch.empty_like(lse)
    prob = ksa.make_problem(q, k, w.T)
    wv = ksa.new_workspace(ksa.ksa_workspace_bytes(prob, ksa.KSA_OP_VOTE_SELECT, N), DEV)
    wa = ksa.new_workspace(max(1, ksa.ksa_workspace_bytes(prob, ksa.KSA_OP_SPARSE_TOKENS, n_out)), DEV)
    wl = ksa.new_workspace(ksa.ksa_workspace_bytes(prob, ksa.KSA_OP_VOTE_LAYER, N), DEV)
    qbuf = q.clone()
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()

    def work():
        ksa.ksa_vote_select(qbuf, k, w.T, N, W, token_idx=idx, workspace=wv, stream=stream)
        ksa.ksa_sparse_decode(qbuf, k, v, w.T, idx, ksa.KSA_SEL_TOKENS, out=out, lse=lse,
                              workspace=wa, stream=stream)
        ksa.ksa_vote_layer_decode(qbuf, k, v, w.T, N, W, out=lout, lse=llse, token_idx=lidx,
                                  workspace=wl, stream=stream)

    with torch.cuda.stream(stream):
        work()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        work()
    torch.cuda.synchronize()
    for rep, nq in enumerate(step_queries(4, w.B, w.Hq, w.D, q.dtype, seed=72)):
        qbuf.copy_(nq)
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (idx, out, lse, lidx, lout, llse)]
        e_idx = ksa.ksa_vote_select(nq, k, w.T, N, W)
        e_out, e_lse = ksa.ksa_sparse_decode(nq, k, v, w.T, e_idx, ksa.KSA_SEL_TOKENS)
        l_out, l_lse, l_idx, _ = ksa.ksa_vote_layer_decode(nq, k, v, w.T, N, W)
        torch.cuda.synchronize()
        assert torch.equal(got[0], e_idx) and torch.equal(got[3], l_idx), rep
        assert torch.equal(got[1], e_out) and torch.equal(got[2], e_lse), rep
        assert torch.equal(got[4], l_out) and torch.equal(got[5], l_lse), rep
        assert torch.equal(l_idx, e_idx), rep
    # and the set is the oracle's rule on the logits of the last queries
    sl = slice(0, 1)
    lg = oracle.head_logits(np_bits(nq[sl]), np_bits(k[sl]), w.T)
    votes = ksa.ksa_vote_select(nq, k, w.T, N, W, want_votes=True)[1]
    check_votes(votes[sl].cpu().numpy(), got[0][sl].cpu().numpy(), lg, N, W)
