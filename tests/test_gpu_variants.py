"""GPU parity of the selection variants and the attention-recall diagnostic.

* ksa_select_topk_ex: MAX group aggregation and the forced local block,
  against the oracle's max-aggregated relevance and its forced-block rule
  (near-tie rules of tests/parity.py).
* ksa_vote_select_heads: votes of a subset of heads (one head: the
  random-head ablation) against the oracle's vote of those heads.
* ksa_attention_recall: exp(lse_selected - lse_dense) on the GPU against the
  oracle's sum of dense softmax weights over the GPU's own selection.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_decode_ksa_amd as ksa
from sparse_attention_decode_ksa_amd.inputs import WORKLOADS, small_workload
from parity import check_attention, check_block_selection, check_votes
from test_gpu_parity import DEV, gpu_inputs, np_bits, run_summaries

pytestmark = pytest.mark.gpu

SEL_CASES = [
    dict(B=2, Hq=4, Hkv=2, D=64, T=1000, Bs=16, dtype="f32", top_k=8),
    dict(B=2, Hq=16, Hkv=2, D=128, T=3001, Bs=16, dtype="bf16", top_k=40),
    dict(B=3, Hq=8, Hkv=2, D=128, T=777, Bs=7, dtype="bf16", top_k=20),
    dict(B=1, Hq=2, Hkv=2, D=64, T=50, Bs=16, dtype="bf16", top_k=9),     # k > NB
]


def sel_id(c):
    return "%s-G%d-D%d-T%d-Bs%d-k%d" % (c["dtype"], c["Hq"] // c["Hkv"], c["D"], c["T"], c["Bs"],
                                        c["top_k"])


@pytest.mark.parametrize("case", SEL_CASES, ids=sel_id)
def test_max_aggregation_matches_oracle(case):
    w = small_workload(seed=case["T"] + 1, **case)
    q, k, v = gpu_inputs(w)
    s = run_summaries(k, w)
    idx, sc = ksa.ksa_select_topk_ex(q, s, w.T, w.Bs, w.top_k, aggregate=ksa.KSA_AGG_MAX,
                                     want_scores=True)
    torch.cuda.synchronize()
    raw, scaled = oracle.group_scores(np_bits(q), np_bits(s), w.T, w.Bs, Tcap=w.cap,
                                      aggregate="max")
    check_block_selection(idx.cpu().numpy().reshape(w.B * w.Hkv, -1),
                          raw.reshape(w.B * w.Hkv, -1), w.top_k)
    np.testing.assert_allclose(sc.cpu().numpy(), scaled, rtol=0,
                               atol=1e-5 * max(1.0, float(np.abs(scaled).max())))


@pytest.mark.parametrize("agg", [ksa.KSA_AGG_SUM, ksa.KSA_AGG_MAX])
@pytest.mark.parametrize("case", SEL_CASES, ids=sel_id)
def test_forced_last_block(case, agg):
    w = small_workload(seed=case["T"] + 2, **case)
    q, k, v = gpu_inputs(w)
    s = run_summaries(k, w)
    idx = ksa.ksa_select_topk_ex(q, s, w.T, w.Bs, w.top_k, aggregate=agg, force_last_block=True)
    torch.cuda.synchronize()
    raw, _ = oracle.group_scores(np_bits(q), np_bits(s), w.T, w.Bs, Tcap=w.cap,
                                 aggregate="max" if agg == ksa.KSA_AGG_MAX else "sum")
    raw = raw.reshape(w.B * w.Hkv, -1)
    forced = (w.T - 1) // w.Bs
    ids = idx.cpu().numpy().reshape(w.B * w.Hkv, -1)
    keff = ids.shape[1]
    assert np.all(ids == np.sort(ids, axis=1)) and np.all(np.any(ids == forced, axis=1))
    if keff == raw.shape[1]:
        return
    # the other k_eff - 1 blocks: the top of the rest (forced block pushed below everything)
    rest = raw.copy()
    rest[:, forced] = raw.min() - 1.0
    others = np.array([[j for j in row if j != forced] for row in ids])
    check_block_selection(others, rest, keff - 1)
    # exact rule where nothing is near a tie
    ref = oracle.topk_with_block(raw, w.top_k, forced)
    assert (ref == ids).mean() > 0.9


@pytest.mark.parametrize("heads", [[0], [5], [1, 6, 7], list(range(8))])
def test_vote_of_chosen_heads_matches_oracle(heads):
    w = small_workload(B=2, Hq=8, Hkv=2, D=128, T=3000, dtype="bf16", seed=len(heads))
    q, k, v = gpu_inputs(w)
    N, W = 512, 128
    idx, votes = ksa.ksa_vote_select_heads(q, k, w.T, N, W, heads, want_votes=True)
    torch.cuda.synchronize()
    lg = oracle.head_logits(np_bits(q), np_bits(k), w.T)[:, heads]
    check_votes(votes.cpu().numpy(), idx.cpu().numpy(), lg, N, W)
    assert votes.max().item() <= len(heads)


def test_vote_of_chosen_heads_integer_bit_exact():
    w = small_workload(B=2, Hq=8, Hkv=4, D=64, T=1500, dtype="bf16", seed=3)
    q, k, v = gpu_inputs(w, integer=True, lo=-1, hi=1)
    for heads in ([2], [0, 3, 4]):
        idx, votes = ksa.ksa_vote_select_heads(q, k, w.T, 256, 64, heads, want_votes=True)
        sel, ref_votes = oracle.vote_select(np_bits(q), np_bits(k), w.T, 256, 64, heads=heads)
        np.testing.assert_array_equal(votes.cpu().numpy().astype(np.int32), ref_votes)
        np.testing.assert_array_equal(idx.cpu().numpy(), sel)


def test_vote_heads_validation():
    w = small_workload(B=1, Hq=4, Hkv=2, D=64, T=300, dtype="bf16", seed=1)
    q, k, v = gpu_inputs(w)
    for bad in ([], [4], [-1], [1, 1]):
        with pytest.raises(ksa.KsaError):
            ksa.ksa_vote_select_heads(q, k, w.T, 64, 16, bad)


def test_recall_of_the_fused_step_matches_oracle():
    w = small_workload(B=2, Hq=8, Hkv=2, D=128, T=3000, Bs=16, dtype="bf16", top_k=32, seed=12)
    q, k, v = gpu_inputs(w)
    s = run_summaries(k, w)
    out, lse, idx = ksa.ksa_block_topk_decode(q, k, v, s, w.T, w.Bs, w.top_k, want_block_idx=True)
    dout, dlse = ksa.ksa_dense_decode(q, k, v, w.T)
    rec = ksa.ksa_attention_recall(lse, dlse)
    torch.cuda.synchronize()
    ids = idx.cpu().numpy()
    G = w.G
    ref = oracle.attention_recall(np_bits(q), np_bits(k), w.T, lambda b, h: [
        t for j in ids[b, h // G] for t in range(j * w.Bs, min((j + 1) * w.Bs, w.T))])
    np.testing.assert_allclose(rec.cpu().numpy(), ref, rtol=0, atol=1e-4)
    assert np.all(rec.cpu().numpy() <= 1.0 + 1e-5)


def test_recall_of_every_block_is_one():
    w = small_workload(B=2, Hq=4, Hkv=2, D=64, T=400, Bs=16, dtype="f32", top_k=25, seed=4)
    q, k, v = gpu_inputs(w)
    s = run_summaries(k, w)
    out, lse, _ = ksa.ksa_block_topk_decode(q, k, v, s, w.T, w.Bs, w.top_k)
    _, dlse = ksa.ksa_dense_decode(q, k, v, w.T)
    rec = ksa.ksa_attention_recall(lse, dlse)
    torch.cuda.synchronize()
    np.testing.assert_allclose(rec.cpu().numpy(), 1.0, atol=2e-5)


def test_recall_on_the_c2_workload_is_high():
    """The recall the pages judge selections by, on the planted c2 caches
    (first 8 sequences): between 0 and 1, and for most heads above the 1/16
    share of tokens the 64 of 1024 blocks hold (the selection beats a
    uniform one)."""
    w = WORKLOADS["c2"].with_(B=8)
    q, k, v = gpu_inputs(w)
    s = run_summaries(k, w)
    out, lse, _ = ksa.ksa_block_topk_decode(q, k, v, s, w.T, w.Bs, w.top_k)
    _, dlse = ksa.ksa_dense_decode(q, k, v, w.T)
    rec = ksa.ksa_attention_recall(lse, dlse).cpu().numpy()
    assert rec.min() > 0.0 and rec.max() <= 1.0 + 1e-5
    print("c2 recall: median %.3f, min %.3f" % (float(np.median(rec)), float(rec.min())))
    assert float(np.median(rec)) > 64 / 1024


# ----------------------------------------------------------------------------- selection layer
@pytest.mark.parametrize("Hq,Hkv,D,dtype,T,N,W", [
    (32, 8, 128, "bf16", 5000, 1024, 256),    # G = 4, MFMA: one K read
    (16, 2, 128, "bf16", 3001, 512, 128),     # G = 8, MFMA, ragged key tail
    (8, 4, 128, "bf16", 4000, 512, 128),      # G = 2: dense and the vote's scoring apart
    (4, 2, 64, "f32", 1500, 256, 64),
    (8, 2, 128, "bf16", 300, 512, 128),       # T <= N: every token, no vote
])
def test_vote_layer_equals_dense_plus_vote(Hq, Hkv, D, dtype, T, N, W):
    """The selection layer's output is ksa_dense_decode's and its set and
    votes are ksa_vote_select's, bit for bit; the set also passes the
    oracle's vote rule."""
    w = small_workload(B=2, Hq=Hq, Hkv=Hkv, D=D, T=T, dtype=dtype, seed=T + N)
    q, k, v = gpu_inputs(w)
    out, lse, idx, votes = ksa.ksa_vote_layer_decode(q, k, v, w.T, N, W, want_votes=True)
    dout, dlse = ksa.ksa_dense_decode(q, k, v, w.T)
    ridx, rvotes = ksa.ksa_vote_select(q, k, w.T, N, W, want_votes=True)
    torch.cuda.synchronize()
    assert torch.equal(out, dout) and torch.equal(lse, dlse)
    assert torch.equal(idx, ridx) and torch.equal(votes, rvotes)
    if T > N:
        lg = oracle.head_logits(np_bits(q), np_bits(k), w.T)
        check_votes(votes.cpu().numpy(), idx.cpu().numpy(), lg, N, W)


@pytest.mark.parametrize("seqs", [[0, 15]])
def test_vote_layer_on_c4(seqs):
    """The selection layer at the full c4 shape: bitwise the dense call plus
    the vote call, and on sampled sequences the fp64 oracle's dense attention
    (out, lse) and vote rule (votes up to per-head near ties, the set exactly
    the rule on the GPU's votes)."""
    w = WORKLOADS["c4"]
    q, k, v = gpu_inputs(w)
    N, W = w.token_budget, w.recent_window
    out, lse, idx, votes = ksa.ksa_vote_layer_decode(q, k, v, w.T, N, W, want_votes=True)
    dout, dlse = ksa.ksa_dense_decode(q, k, v, w.T)
    ridx, rvotes = ksa.ksa_vote_select(q, k, w.T, N, W, want_votes=True)
    torch.cuda.synchronize()
    assert torch.equal(out, dout) and torch.equal(lse, dlse)
    assert torch.equal(idx, ridx) and torch.equal(votes, rvotes)
    for b in seqs:
        sl = slice(b, b + 1)
        qb, kb, vb = np_bits(q[sl]), np_bits(k[sl]), np_bits(v[sl])
        ro, rl = oracle.attend_dense(qb, kb, vb, w.T)
        check_attention(out[sl].cpu().numpy(), lse[sl].cpu().numpy(), ro, rl)
        lg = oracle.head_logits(qb, kb, w.T)
        check_votes(votes[sl].cpu().numpy(), idx[sl].cpu().numpy(), lg, N, W)
    del q, k, v
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------- per-head sets
def check_head_sets(gpu, lg, N, W):
    """Every head's set is the oracle's except at near-ties of that head's
    threshold (relative gap < 1e-5 of its max |logit|)."""
    from parity import REL_TIE
    ref = oracle.head_sets(lg, N, W)
    B, Hq, T = lg.shape
    assert gpu.shape == ref.shape
    for b in range(B):
        for h in range(Hq):
            g_, r_ = set(gpu[b, h].tolist()), set(ref[b, h].tolist())
            assert np.all(np.diff(gpu[b, h]) > 0)
            if g_ == r_:
                continue
            C = T - W
            thr = np.sort(lg[b, h, :C])[::-1][N - W - 1]
            tol = REL_TIE * np.abs(lg[b, h, :C]).max()
            for t in g_ ^ r_:
                assert t < C and abs(lg[b, h, t] - thr) <= tol, (b, h, t)


@pytest.mark.parametrize("Hq,Hkv,D,dtype,T,N,W", [
    (32, 8, 128, "bf16", 4000, 512, 128),
    (8, 2, 64, "f32", 2100, 300, 60),
    (4, 4, 128, "bf16", 1000, 100, 0),
    (8, 2, 128, "bf16", 300, 512, 128),   # T <= N
])
def test_per_head_sets_and_their_attention(Hq, Hkv, D, dtype, T, N, W):
    w = small_workload(B=2, Hq=Hq, Hkv=Hkv, D=D, T=T, dtype=dtype, seed=T + Hq)
    q, k, v = gpu_inputs(w)
    idx = ksa.ksa_vote_select_per_head(q, k, w.T, N, W)
    out, lse = ksa.ksa_sparse_decode(q, k, v, w.T, idx, ksa.KSA_SEL_HEAD_TOKENS)
    torch.cuda.synchronize()
    lg = oracle.head_logits(np_bits(q), np_bits(k), w.T)
    ids = idx.cpu().numpy()
    check_head_sets(ids, lg, N, W)
    ro, rl = oracle.attend_head_tokens(np_bits(q), np_bits(k), np_bits(v), w.T, ids)
    from parity import check_attention
    check_attention(out.cpu().numpy(), lse.cpu().numpy(), ro, rl)


def test_per_head_sets_integer_bit_exact():
    w = small_workload(B=2, Hq=8, Hkv=2, D=64, T=1500, dtype="bf16", seed=8)
    q, k, v = gpu_inputs(w, integer=True, lo=-1, hi=1)
    idx = ksa.ksa_vote_select_per_head(q, k, w.T, 256, 64)
    torch.cuda.synchronize()
    lg = oracle.head_logits(np_bits(q), np_bits(k), w.T)
    np.testing.assert_array_equal(idx.cpu().numpy(), oracle.head_sets(lg, 256, 64))


def test_head_token_attention_with_one_list_per_head_equals_shared_list():
    """Giving every head the same list reproduces the shared-list attention
    (to fp32 merge order: the two read K/V in different row groupings)."""
    w = small_workload(B=2, Hq=8, Hkv=2, D=128, T=3000, dtype="bf16", seed=13)
    q, k, v = gpu_inputs(w)
    shared = ksa.ksa_vote_select(q, k, w.T, 512, 128)
    per_head = shared[:, None, :].expand(w.B, w.Hq, shared.shape[1]).contiguous()
    o1, l1 = ksa.ksa_sparse_decode(q, k, v, w.T, shared, ksa.KSA_SEL_TOKENS)
    o2, l2 = ksa.ksa_sparse_decode(q, k, v, w.T, per_head, ksa.KSA_SEL_HEAD_TOKENS)
    torch.cuda.synchronize()
    assert float((o1 - o2).abs().max()) <= 1e-5 and float((l1 - l2).abs().max()) <= 1e-5
