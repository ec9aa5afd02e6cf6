"""Parity on seeded random shapes: every call of the path against the oracle on
configurations drawn from the whole supported range at once (dtype, D, G, Hkv,
Bs, T, k, N, W, per-sequence lengths) rather than from hand-picked cases.

Each case draws its configuration from its own seed, so a failure names a
reproducible shape.  The acceptance rules are those of tests/parity.py.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_decode_ksa_amd as ksa
from sparse_attention_decode_ksa_amd.inputs import small_workload
from parity import check_attention, check_block_selection, check_votes
from test_gpu_parity import DEV, gpu_inputs, np_bits
from test_gpu_fused_step import check_against_oracle, fused_vs_separate
from test_gpu_paged import gathered, paged_inputs
from test_gpu_variants import check_head_sets

pytestmark = pytest.mark.gpu

NCASES = 64


def draw(seed):
    """One configuration inside the library's documented limits: a quarter of
    the cases short (1..200 tokens), the rest 200..12000; N a random fraction
    of T (so some rows have T <= N), W anywhere in [0, N]."""
    r = np.random.default_rng(9000 + seed)
    G = int(r.choice([1, 2, 4, 8]))
    Hkv = int(r.choice([1, 2, 4, 8]))
    Bs = int(r.choice([1, 3, 7, 8, 16, 16, 16, 32, 32, 64]))
    lo, hi = (1, 200) if r.random() < 0.25 else (200, 12000)
    T = int(np.exp(r.uniform(np.log(lo), np.log(hi))))
    T = max(1, min(T, 4095 * Bs))                       # NB + 1 spare page <= 4096
    B = int(r.integers(1, 5))
    nb = -(-T // Bs)
    lens = sorted(set([T] + [int(r.integers(1, T + 1)) for _ in range(B - 1)]), reverse=True)
    N = max(1, int(T * r.uniform(0.02, 1.2)))
    return dict(B=B, Hq=G * Hkv, Hkv=Hkv, D=int(r.choice([64, 128])),
                dtype=str(r.choice(["bf16", "f32"])), Bs=Bs, T=T,
                Tcap=T + int(r.integers(0, 3)) * Bs,
                top_k=int(r.integers(1, min(2048, nb + 3))),
                N=N, W=int(r.integers(0, N + 1)), lens=lens)


def cid(i):
    c = draw(i)
    return "s%d-%s-G%d-Hkv%d-D%d-Bs%d-T%d-k%d-N%d-W%d" % (
        i, c["dtype"], c["Hq"] // c["Hkv"], c["Hkv"], c["D"], c["Bs"], c["T"], c["top_k"], c["N"],
        c["W"])


CASES = list(range(NCASES))


@pytest.mark.parametrize("i", CASES, ids=cid)
def test_random_block_step(i):
    """The fused step (stale newest block refreshed) equals the separate calls
    and matches the oracle on every sequence; the paged step matches the
    oracle on each sequence's own length."""
    c = draw(i)
    w = small_workload(B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], D=c["D"], dtype=c["dtype"], Bs=c["Bs"],
                       T=c["T"], Tcap=c["Tcap"], top_k=c["top_k"], seed=100 + i)
    q, k, v = gpu_inputs(w)
    s, idx, out, lse = fused_vs_separate(w, q, k, v, refresh=True, seed=i)
    check_against_oracle(w, q, k, v, s, idx, out, lse, range(w.B))

    lens, Bs, top_k = c["lens"], c["Bs"], c["top_k"]
    w, q, k, v, kp, vp, table, seq = paged_inputs(lens, Bs, seed=200 + i, Hq=c["Hq"],
                                                  Hkv=c["Hkv"], D=c["D"], dtype=c["dtype"])
    s = torch.zeros((w.B, w.Hkv, table.shape[1], w.D), dtype=k.dtype, device=DEV)
    ksa.ksa_paged_block_summaries(kp, s, table, seq)
    for b, T in enumerate(lens):
        s[b, :, (T - 1) // Bs] = (torch.randn(s[b, :, 0].shape, device=DEV) * 3).to(s.dtype)
    out, lse, ids = ksa.ksa_paged_block_topk_decode(q, kp, vp, s, table, seq, top_k,
                                                    want_block_idx=True)
    torch.cuda.synchronize()
    got_s, ids = np_bits(s), ids.cpu().numpy()
    for b, T in enumerate(lens):
        nb = ksa.nblocks(T, Bs)
        keff = min(top_k, nb)
        kb, vb = gathered(kp, table, b, T, Bs), gathered(vp, table, b, T, Bs)
        qb = np_bits(q[b:b + 1])
        sb = oracle.block_summaries(kb, T, Bs)
        np.testing.assert_array_equal(got_s[b:b + 1, :, :nb], sb[:, :, :nb])
        assert np.all(ids[b, :, keff:] == -1)
        raw, _ = oracle.group_scores(qb, sb, T, Bs)
        ib = ids[b:b + 1, :, :keff]
        check_block_selection(ib.reshape(w.Hkv, -1), raw.reshape(w.Hkv, -1), top_k)
        ro, rl = oracle.attend_blocks(qb, kb, vb, T, Bs, ib)
        check_attention(out[b:b + 1].cpu().numpy(), lse[b:b + 1].cpu().numpy(), ro, rl)


@pytest.mark.parametrize("i", CASES, ids=cid)
def test_random_block_step_varlen(i):
    """The fused step with one length per sequence on a contiguous cache
    matches the oracle on each sequence's own length."""
    from test_gpu_fused_step import varlen_inputs
    c = draw(i)
    lens, Bs, top_k = c["lens"], c["Bs"], c["top_k"]
    w, q, k, v, s, seq = varlen_inputs(lens, Bs, seed=900 + i, Hq=c["Hq"], Hkv=c["Hkv"],
                                       D=c["D"], dtype=c["dtype"])
    out, lse, idx = ksa.ksa_block_topk_decode_varlen(q, k, v, s, seq, Bs, top_k, max_len=w.T,
                                                     want_block_idx=True)
    torch.cuda.synchronize()
    got_s, ids = np_bits(s), idx.cpu().numpy()
    for b, T in enumerate(lens):
        nb = ksa.nblocks(T, Bs)
        keff = min(top_k, nb)
        qb, kb, vb = np_bits(q[b:b + 1]), np_bits(k[b:b + 1]), np_bits(v[b:b + 1])
        sb = oracle.block_summaries(kb, T, Bs)
        np.testing.assert_array_equal(got_s[b:b + 1, :, :nb], sb[:, :, :nb])
        assert np.all(ids[b, :, keff:] == -1)
        raw, _ = oracle.group_scores(qb, sb, T, Bs, Tcap=w.cap)
        ib = np.ascontiguousarray(ids[b:b + 1, :, :keff])
        check_block_selection(ib.reshape(w.Hkv, -1), raw.reshape(w.Hkv, -1), top_k)
        ro, rl = oracle.attend_blocks(qb, kb, vb, T, Bs, ib)
        check_attention(out[b:b + 1].cpu().numpy(), lse[b:b + 1].cpu().numpy(), ro, rl)


@pytest.mark.parametrize("i", CASES, ids=cid)
def test_random_vote_paths(i):
    """The shared vote-union set, its token attention and the per-head sets
    match the oracle on a contiguous cache; the paged vote and its attention
    match it on each sequence's own length."""
    c = draw(i)
    N, W = c["N"], c["W"]
    w = small_workload(B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], D=c["D"], dtype=c["dtype"], T=c["T"],
                       seed=300 + i)
    q, k, v = gpu_inputs(w)
    idx, votes = ksa.ksa_vote_select(q, k, w.T, N, W, want_votes=True)
    out, lse = ksa.ksa_sparse_decode(q, k, v, w.T, idx, ksa.KSA_SEL_TOKENS)
    hidx = ksa.ksa_vote_select_per_head(q, k, w.T, N, W)
    hout, hlse = ksa.ksa_sparse_decode(q, k, v, w.T, hidx, ksa.KSA_SEL_HEAD_TOKENS)
    torch.cuda.synchronize()
    qn, kn, vn = np_bits(q), np_bits(k), np_bits(v)
    ids, hids = idx.cpu().numpy(), hidx.cpu().numpy()
    lg = oracle.head_logits(qn, kn, w.T)
    if w.T <= N:
        assert np.array_equal(ids, np.broadcast_to(np.arange(w.T), ids.shape))
        assert int(votes.sum()) == 0
    else:
        check_votes(votes.cpu().numpy(), ids, lg, N, W)
    check_head_sets(hids, lg, N, W)
    ro, rl = oracle.attend_tokens(qn, kn, vn, w.T, ids)
    check_attention(out.cpu().numpy(), lse.cpu().numpy(), ro, rl)
    ro, rl = oracle.attend_head_tokens(qn, kn, vn, w.T, hids)
    check_attention(hout.cpu().numpy(), hlse.cpu().numpy(), ro, rl)

    lens, Bs = c["lens"], c["Bs"]
    w, q, k, v, kp, vp, table, seq = paged_inputs(lens, Bs, seed=400 + i, Hq=c["Hq"],
                                                  Hkv=c["Hkv"], D=c["D"], dtype=c["dtype"])
    pidx, pvotes = ksa.ksa_paged_vote_select(q, kp, table, seq, N, W, want_votes=True)
    pout, plse = ksa.ksa_paged_sparse_decode(q, kp, vp, table, seq, pidx, ksa.KSA_SEL_TOKENS)
    phidx = ksa.ksa_paged_vote_select_per_head(q, kp, table, seq, N, W)
    phout, phlse = ksa.ksa_paged_sparse_decode(q, kp, vp, table, seq, phidx,
                                               ksa.KSA_SEL_HEAD_TOKENS)
    torch.cuda.synchronize()
    pids, pvts, phids = pidx.cpu().numpy(), pvotes.cpu().numpy(), phidx.cpu().numpy()
    for b, T in enumerate(lens):
        kb, vb = gathered(kp, table, b, T, Bs), gathered(vp, table, b, T, Bs)
        qb = np_bits(q[b:b + 1])
        row = pids[b][pids[b] >= 0]
        assert np.all(pids[b][row.shape[0]:] == -1)
        n_b = min(N, T)
        assert np.all(phids[b, :, n_b:] == -1)
        hrow = phids[b:b + 1, :, :n_b]
        lg = oracle.head_logits(qb, kb, T)
        if T <= N:
            assert row.tolist() == list(range(T)) and np.all(pvts[b] == 0)
        else:
            assert row.shape[0] == N
            check_votes(pvts[b:b + 1, :T], row[None], lg, N, W)
        check_head_sets(hrow, lg, N, W)
        ro, rl = oracle.attend_tokens(qb, kb, vb, T, row[None].astype(np.int32))
        check_attention(pout[b:b + 1].cpu().numpy(), plse[b:b + 1].cpu().numpy(), ro, rl)
        ro, rl = oracle.attend_head_tokens(qb, kb, vb, T, np.ascontiguousarray(hrow))
        check_attention(phout[b:b + 1].cpu().numpy(), phlse[b:b + 1].cpu().numpy(), ro, rl)


@pytest.mark.parametrize("i", CASES, ids=cid)
def test_random_dense_and_selection_layers(i):
    """Dense decode matches the oracle; the selection layers (contiguous and
    paged) give the dense outputs and the vote calls' sets bit for bit."""
    c = draw(i)
    N, W = c["N"], c["W"]
    w = small_workload(B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], D=c["D"], dtype=c["dtype"], T=c["T"],
                       seed=500 + i)
    q, k, v = gpu_inputs(w)
    dout, dlse = ksa.ksa_dense_decode(q, k, v, w.T)
    out, lse, idx, votes = ksa.ksa_vote_layer_decode(q, k, v, w.T, N, W, want_votes=True)
    ridx, rvotes = ksa.ksa_vote_select(q, k, w.T, N, W, want_votes=True)
    torch.cuda.synchronize()
    ro, rl = oracle.attend_dense(np_bits(q), np_bits(k), np_bits(v), w.T)
    check_attention(dout.cpu().numpy(), dlse.cpu().numpy(), ro, rl)
    assert torch.equal(out, dout) and torch.equal(lse, dlse)
    assert torch.equal(idx, ridx) and torch.equal(votes, rvotes)

    lens, Bs = c["lens"], c["Bs"]
    w, q, k, v, kp, vp, table, seq = paged_inputs(lens, Bs, seed=600 + i, Hq=c["Hq"],
                                                  Hkv=c["Hkv"], D=c["D"], dtype=c["dtype"])
    pout, plse, pidx, pvotes = ksa.ksa_paged_vote_layer_decode(q, kp, vp, table, seq, N, W,
                                                               want_votes=True)
    do, dl = ksa.ksa_paged_dense_decode(q, kp, vp, table, seq)
    vi, vv = ksa.ksa_paged_vote_select(q, kp, table, seq, N, W, want_votes=True)
    torch.cuda.synchronize()
    assert torch.equal(pout, do) and torch.equal(plse, dl)
    assert torch.equal(pidx, vi) and torch.equal(pvotes, vv)
    for b, T in enumerate(lens):
        ro, rl = oracle.attend_dense(np_bits(q[b:b + 1]), gathered(kp, table, b, T, Bs),
                                     gathered(vp, table, b, T, Bs), T)
        check_attention(do[b:b + 1].cpu().numpy(), dl[b:b + 1].cpu().numpy(), ro, rl)


def forced_rule_ok(ids, raw, keff, forced):
    """ids [rows, keff] keep block `forced` of each row and, apart from it,
    the top keff - 1 of the rest (near-tie rules)."""
    assert np.all(np.diff(ids, axis=1) > 0)
    assert np.all(np.any(ids == forced[:, None], axis=1))
    if keff < 2 or keff == raw.shape[1]:
        return
    rest = raw.copy()
    rest[np.arange(raw.shape[0]), forced] = raw.min() - 1.0
    others = np.array([[j for j in row if j != f] for row, f in zip(ids, forced)])
    check_block_selection(others, rest, keff - 1)


@pytest.mark.parametrize("i", CASES, ids=cid)
def test_random_selection_variants(i):
    """MAX aggregation and the forced newest block (contiguous and paged) and
    the vote of a random subset of heads (contiguous and paged) against the
    oracle's rules."""
    c = draw(i)
    r = np.random.default_rng(7000 + i)
    N, W, Bs, top_k = c["N"], c["W"], c["Bs"], c["top_k"]
    w = small_workload(B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], D=c["D"], dtype=c["dtype"], Bs=Bs,
                       T=c["T"], Tcap=c["Tcap"], top_k=top_k, seed=700 + i)
    q, k, v = gpu_inputs(w)
    s = torch.zeros((w.B, w.Hkv, ksa.nblocks(w.cap, Bs), w.D), dtype=k.dtype, device=DEV)
    ksa.ksa_block_summaries(k, s, w.T, Bs)
    heads = sorted(r.choice(w.Hq, size=int(r.integers(1, w.Hq + 1)), replace=False).tolist())
    mx, sc = ksa.ksa_select_topk_ex(q, s, w.T, Bs, top_k, aggregate=ksa.KSA_AGG_MAX,
                                    want_scores=True)
    fs = ksa.ksa_select_topk_ex(q, s, w.T, Bs, top_k, force_last_block=True)
    fm = ksa.ksa_select_topk_ex(q, s, w.T, Bs, top_k, aggregate=ksa.KSA_AGG_MAX,
                                force_last_block=True)
    hidx, hv = ksa.ksa_vote_select_heads(q, k, w.T, N, W, heads, want_votes=True)
    torch.cuda.synchronize()
    rows = w.B * w.Hkv
    qn, sn = np_bits(q), np_bits(s)
    raw_max, scaled = oracle.group_scores(qn, sn, w.T, Bs, Tcap=w.cap, aggregate="max")
    raw_sum, _ = oracle.group_scores(qn, sn, w.T, Bs, Tcap=w.cap)
    raw_max, raw_sum = raw_max.reshape(rows, -1), raw_sum.reshape(rows, -1)
    check_block_selection(mx.cpu().numpy().reshape(rows, -1), raw_max, top_k)
    np.testing.assert_allclose(sc.cpu().numpy(), scaled, rtol=0,
                               atol=1e-5 * max(1.0, float(np.abs(scaled).max())))
    keff = min(top_k, w.NB)
    last = np.full(rows, w.NB - 1)
    forced_rule_ok(fs.cpu().numpy().reshape(rows, -1), raw_sum, keff, last)
    forced_rule_ok(fm.cpu().numpy().reshape(rows, -1), raw_max, keff, last)
    if w.T <= N:
        assert np.array_equal(hidx.cpu().numpy(), np.broadcast_to(np.arange(w.T), hidx.shape))
    else:
        lg = oracle.head_logits(qn, np_bits(k), w.T)[:, heads]
        check_votes(hv.cpu().numpy(), hidx.cpu().numpy(), lg, N, W)

    lens = c["lens"]
    w, q, k, v, kp, vp, table, seq = paged_inputs(lens, Bs, seed=800 + i, Hq=c["Hq"],
                                                  Hkv=c["Hkv"], D=c["D"], dtype=c["dtype"])
    s = torch.zeros((w.B, w.Hkv, table.shape[1], w.D), dtype=k.dtype, device=DEV)
    ksa.ksa_paged_block_summaries(kp, s, table, seq)
    pm = ksa.ksa_paged_select_topk_ex(q, s, table, seq, Bs, top_k, aggregate=ksa.KSA_AGG_MAX)
    pf = ksa.ksa_paged_select_topk_ex(q, s, table, seq, Bs, top_k, force_last_block=True)
    pidx, pv = ksa.ksa_paged_vote_select_heads(q, kp, table, seq, N, W, heads, want_votes=True)
    torch.cuda.synchronize()
    sn = np_bits(s)
    pm, pf, pids, pvts = pm.cpu().numpy(), pf.cpu().numpy(), pidx.cpu().numpy(), pv.cpu().numpy()
    for b, T in enumerate(lens):
        nb = ksa.nblocks(T, Bs)
        keff = min(top_k, nb)
        qb = np_bits(q[b:b + 1])
        rm, _ = oracle.group_scores(qb, sn[b:b + 1], T, Bs, Tcap=table.shape[1] * Bs,
                                    aggregate="max")
        rs, _ = oracle.group_scores(qb, sn[b:b + 1], T, Bs, Tcap=table.shape[1] * Bs)
        rm, rs = rm.reshape(w.Hkv, -1), rs.reshape(w.Hkv, -1)
        assert np.all(pm[b][:, keff:] == -1) and np.all(pf[b][:, keff:] == -1)
        check_block_selection(np.ascontiguousarray(pm[b][:, :keff]), rm, top_k)
        forced_rule_ok(np.ascontiguousarray(pf[b][:, :keff]), rs, keff, np.full(w.Hkv, nb - 1))
        row = pids[b][pids[b] >= 0]
        if T <= N:
            assert row.tolist() == list(range(T))
        else:
            assert row.shape[0] == N
            lg = oracle.head_logits(qb, gathered(kp, table, b, T, Bs), T)[:, heads]
            check_votes(pvts[b:b + 1, :T], row[None], lg, N, W)
