"""Parity of the HIP path (called through the C ABI) with the fp64 oracle.

Inputs come from the seeded generators; the oracle always receives a copy of
the exact bytes the GPU saw.  Small shapes are compared element by element
over whole tensors (several tiles, ragged tails, partial blocks); the five
workloads run at full size on the GPU, in the launch configuration the
benchmark uses, and are compared on sampled sequences.  Acceptance rules are
in tests/parity.py.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_decode_ksa_amd as ksa
from sparse_attention_decode_ksa_amd.inputs import (WORKLOADS, as_numpy_bits, integer_inputs,
                                                    make_inputs, small_workload)
from parity import check_attention, check_block_selection, check_votes, REL_TIE

pytestmark = pytest.mark.gpu

DEV = "cuda"


def gpu_inputs(w, integer=False, lo=-2, hi=2):
    if integer:
        x = integer_inputs(w, lo, hi, device=DEV)
    else:
        x = make_inputs(w, device=DEV) if w.B * w.Hkv * w.cap * w.D > 2 ** 22 else \
            {k_: t.to(DEV) for k_, t in make_inputs(w).items()}
    return x["q"], x["k"], x["v"]


def np_bits(t):
    return as_numpy_bits(t)


def run_summaries(k, w):
    nbcap = ksa.nblocks(w.cap, w.Bs)
    s = torch.full((w.B, w.Hkv, nbcap, w.D), 7, dtype=k.dtype, device=DEV)
    ksa.ksa_block_summaries(k, s, w.T, w.Bs)
    return s


# ----------------------------------------------------------------------------- summaries
SUMMARY_CASES = [
    dict(dtype="f32", D=64, Bs=16, T=1024, Tcap=1024),
    dict(dtype="bf16", D=128, Bs=16, T=1000, Tcap=1040),
    dict(dtype="bf16", D=64, Bs=5, T=333, Tcap=340),
    dict(dtype="f32", D=128, Bs=32, T=77, Tcap=96),
    dict(dtype="bf16", D=128, Bs=1, T=50, Tcap=50),
]


@pytest.mark.parametrize("case", SUMMARY_CASES, ids=lambda c: "%s-D%d-Bs%d-T%d" % (c["dtype"], c["D"], c["Bs"], c["T"]))
def test_summaries_bit_exact(case):
    w = small_workload(B=3, Hq=4, Hkv=2, seed=case["T"], **case)
    q, k, v = gpu_inputs(w)
    s = run_summaries(k, w)
    ref = oracle.block_summaries(np_bits(k), w.T, w.Bs)
    got = np_bits(s)
    nb = w.NB
    np.testing.assert_array_equal(got[:, :, :nb], ref[:, :, :nb])
    # blocks past NB(T) are untouched
    assert np.all(s[:, :, nb:].float().cpu().numpy() == 7)


def test_summary_refresh_of_the_last_block_only():
    w = small_workload(B=2, Hq=4, Hkv=2, D=128, T=100, Tcap=128, Bs=16, dtype="bf16", seed=3)
    q, k, v = gpu_inputs(w)
    s = run_summaries(k, w)
    before = s.clone()
    # append a token: T -> 101 changes block 6 only
    k[:, :, 100] = torch.randn(2, 2, 128, device=DEV).to(k.dtype)
    ksa.ksa_block_summaries(k, s, 101, 16, first_block=100 // 16, num_blocks=1)
    ref = oracle.block_summaries(np_bits(k), 101, 16)
    got = np_bits(s)
    np.testing.assert_array_equal(got[:, :, :7], ref[:, :, :7])
    assert torch.equal(s[:, :, :6], before[:, :, :6])


# ----------------------------------------------------------------------------- selection
SELECT_CASES = [
    dict(B=2, Hq=4, Hkv=2, D=64, T=1024, Bs=16, dtype="f32", top_k=8),
    dict(B=3, Hq=8, Hkv=1, D=128, T=3000, Bs=16, dtype="bf16", top_k=64),
    dict(B=2, Hq=16, Hkv=2, D=128, T=4099, Bs=32, dtype="bf16", top_k=20),
    dict(B=2, Hq=2, Hkv=2, D=64, T=517, Bs=7, dtype="bf16", top_k=30),
    dict(B=1, Hq=4, Hkv=4, D=128, T=200, Bs=1, dtype="f32", top_k=17),
    dict(B=2, Hq=4, Hkv=2, D=64, T=64, Bs=16, dtype="bf16", top_k=9),   # k > NB
]


def sel_id(c):
    return "%s-G%d-D%d-T%d-Bs%d-k%d" % (c["dtype"], c["Hq"] // c["Hkv"], c["D"], c["T"], c["Bs"], c["top_k"])


@pytest.mark.parametrize("case", SELECT_CASES, ids=sel_id)
def test_select_topk_matches_oracle(case):
    w = small_workload(seed=case["T"] + 1, **case)
    q, k, v = gpu_inputs(w)
    s = run_summaries(k, w)
    idx, scores = ksa.ksa_select_topk(q, s, w.T, w.Bs, w.top_k, max_seq_len=w.cap, want_scores=True)
    torch.cuda.synchronize()
    raw, scaled = oracle.group_scores(np_bits(q), np_bits(s), w.T, w.Bs, Tcap=w.cap)
    rows = w.B * w.Hkv
    check_block_selection(idx.cpu().numpy().reshape(rows, -1), raw.reshape(rows, -1), w.top_k)
    sc = scores.cpu().numpy().astype(np.float64)
    tol = REL_TIE * np.abs(scaled).max(axis=-1, keepdims=True)
    assert np.all(np.abs(sc - scaled) <= tol)


@pytest.mark.parametrize("G,Bs,dtype", [(1, 16, "bf16"), (2, 16, "bf16"), (4, 32, "bf16"),
                                        (8, 16, "bf16"), (2, 16, "f32")])
def test_select_integer_ties_are_bit_exact(G, Bs, dtype):
    """Small-integer q and K: every summary mean of a power-of-two block and every
    score is exact on both sides, so the tie rule (lowest block id) must agree
    exactly -- there are many exact ties."""
    w = small_workload(B=3, Hq=2 * G, Hkv=2, D=64, T=64 * Bs, Bs=Bs, dtype=dtype, top_k=13, seed=G)
    q, k, v = gpu_inputs(w, integer=True, lo=-1, hi=1)
    # blocks 32..63 repeat blocks 0..31: every score occurs at least twice
    k[:, :, 32 * Bs:] = k[:, :, :32 * Bs]
    s = run_summaries(k, w)
    idx = ksa.ksa_select_topk(q, s, w.T, w.Bs, w.top_k)
    raw, _ = oracle.group_scores(np_bits(q), np_bits(s), w.T, w.Bs)
    ref = oracle.topk(raw, w.top_k)
    assert np.array_equal(raw[..., :32], raw[..., 32:])
    np.testing.assert_array_equal(idx.cpu().numpy(), ref)


# ----------------------------------------------------------------------------- attention
ATTN_CASES = [
    dict(B=2, Hq=4, Hkv=2, D=64, T=1024, Bs=16, dtype="f32", top_k=8),
    dict(B=2, Hq=2, Hkv=2, D=128, T=1000, Tcap=1024, Bs=16, dtype="bf16", top_k=63),
    dict(B=1, Hq=16, Hkv=4, D=128, T=5000, Bs=32, dtype="bf16", top_k=40),
    dict(B=2, Hq=16, Hkv=2, D=128, T=2050, Bs=16, dtype="bf16", top_k=129),
    dict(B=3, Hq=2, Hkv=1, D=64, T=300, Bs=6, dtype="bf16", top_k=11),
    dict(B=1, Hq=8, Hkv=8, D=128, T=900, Bs=1, dtype="f32", top_k=100),
    dict(B=1, Hq=4, Hkv=1, D=128, T=1, Bs=16, dtype="bf16", top_k=4),
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=sel_id)
def test_block_sparse_decode_matches_oracle(case):
    w = small_workload(seed=case["T"] + 7, **case)
    q, k, v = gpu_inputs(w)
    s = run_summaries(k, w)
    idx = ksa.ksa_select_topk(q, s, w.T, w.Bs, w.top_k, max_seq_len=w.cap)
    out, lse = ksa.ksa_sparse_decode(q, k, v, w.T, idx, ksa.KSA_SEL_BLOCKS, block_size=w.Bs)
    ref_out, ref_lse = oracle.attend_blocks(np_bits(q), np_bits(k), np_bits(v), w.T, w.Bs,
                                            idx.cpu().numpy())
    check_attention(out.cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse)


def test_block_sparse_decode_with_given_blocks_and_partial_tail():
    w = small_workload(B=2, Hq=8, Hkv=2, D=128, T=1000, Tcap=1008, Bs=16, dtype="bf16", seed=5)
    q, k, v = gpu_inputs(w)
    rng = np.random.default_rng(1)
    # 19 random full blocks plus the partial last block (8 of its 16 tokens are below T)
    idx = np.stack([np.stack([np.sort(np.append(rng.choice(w.NB - 1, 19, replace=False), w.NB - 1))
                              for _ in range(2)]) for _ in range(2)]).astype(np.int32)
    it = torch.from_numpy(idx).to(DEV)
    out, lse = ksa.ksa_sparse_decode(q, k, v, w.T, it, ksa.KSA_SEL_BLOCKS, block_size=16)
    ref_out, ref_lse = oracle.attend_blocks(np_bits(q), np_bits(k), np_bits(v), w.T, 16, idx)
    check_attention(out.cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse)


@pytest.mark.parametrize("G,D,dtype,count", [(4, 128, "bf16", 2048), (2, 64, "f32", 37),
                                             (8, 128, "bf16", 513), (1, 128, "bf16", 1)])
def test_token_sparse_decode_matches_oracle(G, D, dtype, count):
    w = small_workload(B=3, Hq=2 * G, Hkv=2, D=D, T=5000, dtype=dtype, seed=count)
    q, k, v = gpu_inputs(w)
    rng = np.random.default_rng(count)
    idx = np.stack([np.sort(rng.choice(w.T, count, replace=False)) for _ in range(3)]).astype(np.int32)
    out, lse = ksa.ksa_sparse_decode(q, k, v, w.T, torch.from_numpy(idx).to(DEV), ksa.KSA_SEL_TOKENS)
    ref_out, ref_lse = oracle.attend_tokens(np_bits(q), np_bits(k), np_bits(v), w.T, idx)
    check_attention(out.cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse)


@pytest.mark.parametrize("G,D,dtype,T", [(2, 64, "f32", 1024), (4, 128, "bf16", 7777),
                                         (8, 128, "bf16", 3000), (1, 64, "bf16", 1),
                                         (2, 128, "bf16", 33000)])
def test_dense_decode_matches_oracle(G, D, dtype, T):
    w = small_workload(B=2, Hq=2 * G, Hkv=2, D=D, T=T, Tcap=T + 5, dtype=dtype, seed=T)
    q, k, v = gpu_inputs(w)
    out, lse = ksa.ksa_dense_decode(q, k, v, w.T)
    ref_out, ref_lse = oracle.attend_dense(np_bits(q), np_bits(k), np_bits(v), w.T)
    check_attention(out.cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse)


def test_dense_decode_explicit_scale():
    w = small_workload(B=1, Hq=4, Hkv=2, D=64, T=500, dtype="bf16", seed=2)
    q, k, v = gpu_inputs(w)
    out, lse = ksa.ksa_dense_decode(q, k, v, w.T, sm_scale=0.05)
    ref_out, ref_lse = oracle.attend_dense(np_bits(q), np_bits(k), np_bits(v), w.T, sm_scale=0.05)
    check_attention(out.cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse)


def test_all_blocks_selected_equals_dense():
    w = small_workload(B=2, Hq=8, Hkv=2, D=128, T=777, Bs=16, dtype="bf16", top_k=10 ** 6, seed=4)
    q, k, v = gpu_inputs(w)
    s = run_summaries(k, w)
    idx = ksa.ksa_select_topk(q, s, w.T, w.Bs, w.top_k)
    assert idx.shape[-1] == w.NB
    o1, l1 = ksa.ksa_sparse_decode(q, k, v, w.T, idx, ksa.KSA_SEL_BLOCKS, block_size=16)
    o2, l2 = ksa.ksa_dense_decode(q, k, v, w.T)
    assert float((o1 - o2).abs().max()) <= 1e-6
    assert float((l1 - l2).abs().max()) <= 1e-6


def test_results_are_bitwise_repeatable_and_split_invariant():
    w = small_workload(B=8, Hq=16, Hkv=8, D=128, T=16384, Bs=16, dtype="bf16", top_k=64, seed=9)
    q, k, v = gpu_inputs(w)
    s = run_summaries(k, w)
    idx = ksa.ksa_select_topk(q, s, w.T, w.Bs, w.top_k)
    idx2 = ksa.ksa_select_topk(q, s, w.T, w.Bs, w.top_k)
    assert torch.equal(idx, idx2)
    o1, l1 = ksa.ksa_sparse_decode(q, k, v, w.T, idx, ksa.KSA_SEL_BLOCKS, block_size=16)
    o2, l2 = ksa.ksa_sparse_decode(q, k, v, w.T, idx, ksa.KSA_SEL_BLOCKS, block_size=16)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    d1, _ = ksa.ksa_dense_decode(q, k, v, w.T)
    d2, _ = ksa.ksa_dense_decode(q, k, v, w.T)
    assert torch.equal(d1, d2)
    # the first sequence alone gets a different launch split; results agree
    o3, l3 = ksa.ksa_sparse_decode(q[:1].contiguous(), k[:1].contiguous(), v[:1].contiguous(), w.T,
                                   idx[:1].contiguous(), ksa.KSA_SEL_BLOCKS, block_size=16)
    assert float((o3 - o1[:1]).abs().max()) <= 1e-6
    d3, _ = ksa.ksa_dense_decode(q[:1].contiguous(), k[:1].contiguous(), v[:1].contiguous(), w.T)
    assert float((d3 - d1[:1]).abs().max()) <= 1e-6


def test_split_rows_on_a_reused_workspace():
    """Rows split over many workgroups, merged by the last one to arrive:
    one workspace serves a long run of calls on two alternating inputs
    (and starts filled with random bytes), and every call equals the same
    call on a fresh workspace bit for bit, so no call reads another's
    partial states or arrival counts."""
    ws = torch.randint(0, 256, (1 << 24,), dtype=torch.uint8, device=DEV)
    cases = []
    for seed in (21, 22):
        w = small_workload(B=2, Hq=8, Hkv=2, D=128, T=8192, dtype="bf16", seed=seed)
        q, k, v = gpu_inputs(w)
        tok = ksa.ksa_vote_select(q, k, w.T, 2048, 512)
        p = ksa.make_problem(q, k, w.T)
        assert ksa.ksa_workspace_bytes(p, ksa.KSA_OP_SPARSE_TOKENS, 2048) > 0  # rows are split
        ref_s = ksa.ksa_sparse_decode(q, k, v, w.T, tok, ksa.KSA_SEL_TOKENS)
        ref_d = ksa.ksa_dense_decode(q, k, v, w.T)
        cases.append((w, q, k, v, tok, ref_s, ref_d))
    for i in range(40):
        w, q, k, v, tok, ref_s, ref_d = cases[i % 2]
        o, l = ksa.ksa_sparse_decode(q, k, v, w.T, tok, ksa.KSA_SEL_TOKENS, workspace=ws)
        assert torch.equal(o, ref_s[0]) and torch.equal(l, ref_s[1]), i
        o, l = ksa.ksa_dense_decode(q, k, v, w.T, workspace=ws)
        assert torch.equal(o, ref_d[0]) and torch.equal(l, ref_d[1]), i


# ----------------------------------------------------------------------------- votes
VOTE_CASES = [
    dict(B=2, Hq=4, Hkv=2, D=64, T=300, N=64, W=16, dtype="bf16"),
    dict(B=2, Hq=32, Hkv=8, D=128, T=4000, N=512, W=128, dtype="bf16"),
    dict(B=1, Hq=8, Hkv=1, D=128, T=2100, N=2048, W=0, dtype="f32"),
    dict(B=2, Hq=4, Hkv=4, D=64, T=1000, N=100, W=100, dtype="bf16"),
    dict(B=2, Hq=4, Hkv=2, D=64, T=90, N=100, W=25, dtype="bf16"),
    dict(B=3, Hq=1, Hkv=1, D=128, T=777, N=65, W=1, dtype="bf16"),
]


@pytest.mark.parametrize("case", VOTE_CASES, ids=lambda c: "H%d-T%d-N%d-W%d" % (c["Hq"], c["T"], c["N"], c["W"]))
def test_vote_select_matches_oracle(case):
    c = dict(case)
    N, W = c.pop("N"), c.pop("W")
    w = small_workload(seed=c["T"] + N, **c)
    q, k, v = gpu_inputs(w)
    idx, votes = ksa.ksa_vote_select(q, k, w.T, N, W, want_votes=True)
    torch.cuda.synchronize()
    lg = oracle.head_logits(np_bits(q), np_bits(k), w.T)
    check_votes(votes.cpu().numpy(), idx.cpu().numpy(), lg, N, W)
    ii = idx.cpu().numpy()
    assert ii.shape == (w.B, min(N, w.T)) and np.all(np.diff(ii, axis=1) > 0)
    if w.T > N:
        assert np.all(ii[:, N - W:] == np.arange(w.T - W, w.T))


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (32, 8), (8, 8)])
def test_vote_integer_inputs_are_bit_exact(Hq, Hkv):
    w = small_workload(B=2, Hq=Hq, Hkv=Hkv, D=64, T=1500, dtype="bf16", seed=Hq)
    q, k, v = gpu_inputs(w, integer=True, lo=-1, hi=1)
    idx, votes = ksa.ksa_vote_select(q, k, w.T, 256, 64, want_votes=True)
    sel, ref_votes = oracle.vote_select(np_bits(q), np_bits(k), w.T, 256, 64)
    np.testing.assert_array_equal(votes.cpu().numpy().astype(np.int32), ref_votes)
    np.testing.assert_array_equal(idx.cpu().numpy(), sel)


# ----------------------------------------------------------------------------- full workloads
def block_step(w, q, k, v):
    s = torch.zeros((w.B, w.Hkv, ksa.nblocks(w.cap, w.Bs), w.D), dtype=k.dtype, device=DEV)
    ksa.ksa_block_summaries(k, s, w.T, w.Bs)
    idx = ksa.ksa_select_topk(q, s, w.T, w.Bs, w.top_k)
    out, lse = ksa.ksa_sparse_decode(q, k, v, w.T, idx, ksa.KSA_SEL_BLOCKS, block_size=w.Bs)
    dout, dlse = ksa.ksa_dense_decode(q, k, v, w.T)
    torch.cuda.synchronize()
    return s, idx, out, lse, dout, dlse


def check_block_workload(w, seqs):
    q, k, v = gpu_inputs(w)
    s, idx, out, lse, dout, dlse = block_step(w, q, k, v)
    swaps = 0
    for b in seqs:
        sl = slice(b, b + 1)
        qb, kb, vb = np_bits(q[sl]), np_bits(k[sl]), np_bits(v[sl])
        sb = oracle.block_summaries(kb, w.T, w.Bs)
        np.testing.assert_array_equal(np_bits(s[sl])[:, :, :w.NB], sb[:, :, :w.NB])
        raw, _ = oracle.group_scores(qb, sb, w.T, w.Bs, Tcap=w.cap)
        ib = idx[sl].cpu().numpy()
        swaps += check_block_selection(ib.reshape(w.Hkv, -1), raw.reshape(w.Hkv, -1), w.top_k)
        ro, rl = oracle.attend_blocks(qb, kb, vb, w.T, w.Bs, ib)
        check_attention(out[sl].cpu().numpy(), lse[sl].cpu().numpy(), ro, rl)
        do, dl = oracle.attend_dense(qb, kb, vb, w.T)
        check_attention(dout[sl].cpu().numpy(), dlse[sl].cpu().numpy(), do, dl)
    return swaps


def test_workload_c1_full():
    w = WORKLOADS["c1"]
    check_block_workload(w, range(w.B))


def test_workload_c2_sampled():
    w = WORKLOADS["c2"]
    check_block_workload(w, [0, 37, 63])


def test_workload_c3_sampled():
    w = WORKLOADS["c3"]
    check_block_workload(w, [0, 31])


def test_workload_c5_sampled():
    w = WORKLOADS["c5"]
    check_block_workload(w, [0, 255])
    torch.cuda.empty_cache()


def test_workload_c4_sampled():
    w = WORKLOADS["c4"]
    N, W = w.token_budget, w.recent_window
    q, k, v = gpu_inputs(w)
    idx, votes = ksa.ksa_vote_select(q, k, w.T, N, W, want_votes=True)
    out, lse = ksa.ksa_sparse_decode(q, k, v, w.T, idx, ksa.KSA_SEL_TOKENS)
    torch.cuda.synchronize()
    for b in [0, 15]:
        sl = slice(b, b + 1)
        qb, kb, vb = np_bits(q[sl]), np_bits(k[sl]), np_bits(v[sl])
        lg = oracle.head_logits(qb, kb, w.T)
        check_votes(votes[sl].cpu().numpy(), idx[sl].cpu().numpy(), lg, N, W)
        ro, rl = oracle.attend_tokens(qb, kb, vb, w.T, idx[sl].cpu().numpy())
        check_attention(out[sl].cpu().numpy(), lse[sl].cpu().numpy(), ro, rl)


def test_hip_graph_replay_matches_eager_calls():
    """The block top-k step captured in a HIP graph (the C calls launched on the
    capturing stream) and replayed several times, with new queries copied in
    and eager work in between, matches eager calls every time.  The selection
    workspace's counters are zero-filled once and must stay consistent."""
    w = small_workload(B=8, Hq=16, Hkv=8, D=128, T=4000, Bs=16, dtype="bf16", top_k=32, seed=21)
    q, k, v = gpu_inputs(w)
    s = run_summaries(k, w)
    idx = torch.empty((w.B, w.Hkv, w.top_k), dtype=torch.int32, device=DEV)
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device=DEV)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=DEV)
    prob = ksa.make_problem(q, k, w.T, w.Bs)
    wsel = ksa.new_workspace(ksa.ksa_workspace_bytes(prob, ksa.KSA_OP_SELECT_TOPK, w.top_k), DEV)
    wat = ksa.new_workspace(ksa.ksa_workspace_bytes(prob, ksa.KSA_OP_SPARSE_BLOCKS, w.top_k), DEV)
    stream = torch.cuda.Stream()
    qbuf = q.clone()

    def step():
        ksa.ksa_block_summaries(k, s, w.T, w.Bs, first_block=(w.T - 1) // w.Bs, num_blocks=1,
                                stream=stream)
        ksa.ksa_select_topk(qbuf, s, w.T, w.Bs, w.top_k, block_idx=idx, workspace=wsel, stream=stream)
        ksa.ksa_sparse_decode(qbuf, k, v, w.T, idx, ksa.KSA_SEL_BLOCKS, block_size=w.Bs, out=out,
                              lse=lse, workspace=wat, stream=stream)

    with torch.cuda.stream(stream):
        step()                      # warm up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    torch.cuda.synchronize()
    gen = torch.Generator(device=DEV)
    gen.manual_seed(5)
    for rep in range(4):
        newq = torch.randn(q.shape, generator=gen, device=DEV).to(q.dtype)
        qbuf.copy_(newq)
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        got = (idx.clone(), out.clone(), lse.clone())
        # eager reference on the same inputs, with fresh buffers
        e_idx = ksa.ksa_select_topk(newq, s, w.T, w.Bs, w.top_k)
        e_out, e_lse = ksa.ksa_sparse_decode(newq, k, v, w.T, e_idx, ksa.KSA_SEL_BLOCKS, block_size=w.Bs)
        torch.cuda.synchronize()
        assert torch.equal(got[0], e_idx), rep
        assert torch.equal(got[1], e_out) and torch.equal(got[2], e_lse), rep
    # the last replay also agrees with the oracle
    ro, rl = oracle.attend_blocks(np_bits(qbuf), np_bits(k), np_bits(v), w.T, w.Bs, idx.cpu().numpy())
    check_attention(out.cpu().numpy(), lse.cpu().numpy(), ro, rl)


@pytest.mark.parametrize("T,Bs,k", [(4000, 1, 300), (15360, 1, 1000), (9000, 2, 77)])
def test_select_topk_large_block_counts(T, Bs, k):
    """Rows of 4000, 15360 (the supported maximum) and 4500 blocks exercise the
    top-k kernel's larger register tiles."""
    w = small_workload(B=2, Hq=4, Hkv=2, D=64, T=T, Bs=Bs, dtype="bf16", top_k=k, seed=T)
    q, k_, v = gpu_inputs(w)
    s = run_summaries(k_, w)
    idx = ksa.ksa_select_topk(q, s, w.T, w.Bs, w.top_k)
    raw, _ = oracle.group_scores(np_bits(q), np_bits(s), w.T, w.Bs)
    check_block_selection(idx.cpu().numpy().reshape(4, -1), raw.reshape(4, -1), w.top_k)


@pytest.mark.parametrize("T,W,Hq,Hkv,D,integer", [
    (4003, 128, 32, 8, 128, False),   # MFMA scoring, history not a multiple of 4 (ragged key tail)
    (12000, 500, 8, 2, 128, False),   # 16 keys per thread in registers, MFMA G = 4
    (24000, 600, 16, 2, 128, False),  # 24 keys per thread, MFMA G = 8
    (30000, 100, 4, 2, 64, True),     # 32 keys per thread, integer logits: exact ties everywhere
    (35000, 1000, 4, 2, 64, False),   # 34000 history tokens: keys in LDS, vote set over 2 words a thread
])
def test_vote_select_selection_paths(T, W, Hq, Hkv, D, integer):
    """Each way the per-head selection can run (keys in registers at 8..32
    per thread, in LDS, or streamed) and both vote-set layouts agree with
    the oracle's rule on the GPU's own logits (integer inputs: bit for bit)."""
    w = small_workload(B=1, Hq=Hq, Hkv=Hkv, D=D, T=T, dtype="bf16", seed=T + W)
    if integer:
        q, k, v = gpu_inputs(w, integer=True, lo=-1, hi=1)
    else:
        q, k, v = gpu_inputs(w)
    N = 2048
    idx, votes = ksa.ksa_vote_select(q, k, w.T, N, W, want_votes=True)
    torch.cuda.synchronize()
    if integer:
        sel, ref_votes = oracle.vote_select(np_bits(q), np_bits(k), w.T, N, W)
        np.testing.assert_array_equal(votes.cpu().numpy().astype(np.int32), ref_votes)
        np.testing.assert_array_equal(idx.cpu().numpy(), sel)
    else:
        lg = oracle.head_logits(np_bits(q), np_bits(k), w.T)
        check_votes(votes.cpu().numpy(), idx.cpu().numpy(), lg, N, W)


def test_vote_select_history_longer_than_lds():
    """More than 36864 history tokens: the per-head selection streams its keys
    from the workspace instead of holding them in LDS."""
    w = small_workload(B=1, Hq=8, Hkv=2, D=64, T=40000, dtype="bf16", seed=40)
    q, k, v = gpu_inputs(w)
    idx, votes = ksa.ksa_vote_select(q, k, w.T, 4096, 1024, want_votes=True)
    torch.cuda.synchronize()
    lg = oracle.head_logits(np_bits(q), np_bits(k), w.T)
    check_votes(votes.cpu().numpy(), idx.cpu().numpy(), lg, 4096, 1024)
