"""GPU parity of the paged-cache calls: ksa_paged_block_summaries,
ksa_paged_block_topk_decode, ksa_paged_dense_decode, ksa_paged_vote_select,
ksa_paged_sparse_decode, ksa_paged_vote_layer_decode and
ksa_paged_select_topk_ex.

Pools come from the seeded contiguous inputs through to_paged (a random page
order plus spare pages of noise); every sequence has its own length.  Each
sequence is checked against the oracle on its own tokens, gathered from the
pool by oracle.gather_pages, under the acceptance rules of tests/parity.py.
With one length for the whole batch the paged calls must reproduce the
contiguous calls bit for bit (the same arithmetic on the same tokens).
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_decode_ksa_amd as ksa
from sparse_attention_decode_ksa_amd.inputs import small_workload, to_paged
from parity import check_attention, check_block_selection
from test_gpu_parity import DEV, gpu_inputs, np_bits

pytestmark = pytest.mark.gpu


def paged_inputs(lens, Bs, seed, **kw):
    nbmax = max(ksa.nblocks(t, Bs) for t in lens) + 1
    w = small_workload(B=len(lens), T=max(lens), Tcap=nbmax * Bs, Bs=Bs, seed=seed, **kw)
    q, k, v = gpu_inputs(w)
    kp, vp, table = to_paged(k, v, Bs, seed=seed + 1, spare_pages=3)
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    return w, q, k, v, kp, vp, table, seq


def gathered(pool, table, b, T, Bs):
    return oracle.gather_pages(np_bits(pool), table.cpu().numpy(), b, T, Bs)


PAGED_CASES = [
    dict(lens=[1000, 17, 1, 512], Bs=16, Hq=4, Hkv=2, D=64, dtype="bf16", top_k=8),
    dict(lens=[3000, 2048, 777], Bs=16, Hq=8, Hkv=1, D=128, dtype="bf16", top_k=64),   # MFMA G = 8
    dict(lens=[4099, 64, 2000], Bs=32, Hq=16, Hkv=4, D=128, dtype="bf16", top_k=20),   # MFMA G = 4
    dict(lens=[517, 200, 7], Bs=7, Hq=2, Hkv=2, D=64, dtype="bf16", top_k=30),         # Bs not 2^n
    dict(lens=[1025, 1024, 33], Bs=16, Hq=4, Hkv=2, D=128, dtype="f32", top_k=12),     # T-1 opens a block
    dict(lens=[200, 150], Bs=1, Hq=4, Hkv=4, D=128, dtype="f32", top_k=17),            # one-token pages
]


def case_id(c):
    return "%s-G%d-D%d-Bs%d-k%d-%s" % (c["dtype"], c["Hq"] // c["Hkv"], c["D"], c["Bs"], c["top_k"],
                                       "_".join(map(str, c["lens"])))


@pytest.mark.parametrize("case", PAGED_CASES, ids=case_id)
def test_paged_summaries_match_oracle_per_sequence(case):
    c = dict(case)
    lens, Bs = c.pop("lens"), c.pop("Bs")
    c.pop("top_k")
    w, q, k, v, kp, vp, table, seq = paged_inputs(lens, Bs, seed=lens[0], **c)
    s = torch.full((w.B, w.Hkv, table.shape[1], w.D), 7, dtype=k.dtype, device=DEV)
    ksa.ksa_paged_block_summaries(kp, s, table, seq)
    got = np_bits(s)
    for b, T in enumerate(lens):
        nb = ksa.nblocks(T, Bs)
        ref = oracle.block_summaries(gathered(kp, table, b, T, Bs), T, Bs)
        np.testing.assert_array_equal(got[b:b + 1, :, :nb], ref[:, :, :nb])
        assert np.all(s[b, :, nb:].float().cpu().numpy() == 7)  # past the sequence: untouched


@pytest.mark.parametrize("case", PAGED_CASES, ids=case_id)
def test_paged_step_matches_oracle_per_sequence(case):
    c = dict(case)
    lens, Bs, top_k = c.pop("lens"), c.pop("Bs"), c.pop("top_k")
    w, q, k, v, kp, vp, table, seq = paged_inputs(lens, Bs, seed=lens[-1] + 11, **c)
    s = torch.zeros((w.B, w.Hkv, table.shape[1], w.D), dtype=k.dtype, device=DEV)
    ksa.ksa_paged_block_summaries(kp, s, table, seq)
    # the newest block of every sequence holds stale values until the refresh
    for b, T in enumerate(lens):
        s[b, :, (T - 1) // Bs] = (torch.randn(s[b, :, 0].shape, device=DEV) * 3).to(s.dtype)
    out, lse, idx = ksa.ksa_paged_block_topk_decode(q, kp, vp, s, table, seq, top_k,
                                                    want_block_idx=True)
    torch.cuda.synchronize()
    got_s, ids = np_bits(s), idx.cpu().numpy()
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


@pytest.mark.parametrize("case", PAGED_CASES[:3] + PAGED_CASES[4:5], ids=case_id)
def test_paged_dense_matches_oracle_per_sequence(case):
    c = dict(case)
    lens, Bs = c.pop("lens"), c.pop("Bs")
    c.pop("top_k")
    w, q, k, v, kp, vp, table, seq = paged_inputs(lens, Bs, seed=lens[1] + 5, **c)
    out, lse = ksa.ksa_paged_dense_decode(q, kp, vp, table, seq)
    torch.cuda.synchronize()
    for b, T in enumerate(lens):
        ro, rl = oracle.attend_dense(np_bits(q[b:b + 1]), gathered(kp, table, b, T, Bs),
                                     gathered(vp, table, b, T, Bs), T)
        check_attention(out[b:b + 1].cpu().numpy(), lse[b:b + 1].cpu().numpy(), ro, rl)


@pytest.mark.parametrize("G,D,dtype,Bs,T", [(2, 128, "bf16", 16, 5000), (4, 128, "bf16", 32, 4097),
                                             (8, 128, "bf16", 16, 3001), (1, 64, "f32", 16, 999)])
def test_paged_step_equals_contiguous_step_bitwise(G, D, dtype, Bs, T):
    """One length for the whole batch: summaries, ids, out and lse of the paged
    step are bitwise those of the contiguous step on the same tokens, and the
    paged dense call agrees with the contiguous one to fp32 merge order."""
    w, q, k, v, kp, vp, table, seq = paged_inputs([T] * 6, Bs, seed=T, Hq=2 * G, Hkv=2, D=D,
                                                  dtype=dtype)
    nbc = table.shape[1]
    s_c = torch.zeros((w.B, w.Hkv, nbc, w.D), dtype=k.dtype, device=DEV)
    ksa.ksa_block_summaries(k, s_c, T - 1, Bs) if T > 1 else None
    s_c[:, :, (T - 1) // Bs] = 0
    s_p = s_c.clone()
    oc, lc, ic = ksa.ksa_block_topk_decode(q, k, v, s_c, T, Bs, 24, want_block_idx=True)
    op, lp, ip = ksa.ksa_paged_block_topk_decode(q, kp, vp, s_p, table, seq, 24, max_len=T,
                                                 want_block_idx=True)
    torch.cuda.synchronize()
    assert torch.equal(s_c, s_p)
    assert torch.equal(ic, ip[:, :, :ic.shape[2]])
    assert torch.equal(oc, op) and torch.equal(lc, lp)
    dc, dlc = ksa.ksa_dense_decode(q, k, v, T)
    dp, dlp = ksa.ksa_paged_dense_decode(q, kp, vp, table, seq, max_len=T)
    torch.cuda.synchronize()
    assert float((dc - dp).abs().max()) <= 1e-5 and float((dlc - dlp).abs().max()) <= 1e-5


def test_paged_step_without_refresh_keeps_summaries():
    w, q, k, v, kp, vp, table, seq = paged_inputs([700, 300, 90], 16, seed=70, Hq=4, Hkv=2, D=64,
                                                  dtype="bf16")
    s = torch.zeros((w.B, w.Hkv, table.shape[1], w.D), dtype=k.dtype, device=DEV)
    ksa.ksa_paged_block_summaries(kp, s, table, seq)
    before = s.clone()
    out, lse, idx = ksa.ksa_paged_block_topk_decode(q, kp, vp, s, table, seq, 10,
                                                    refresh_last_block=False, want_block_idx=True)
    torch.cuda.synchronize()
    assert torch.equal(s, before)
    for b, T in enumerate([700, 300, 90]):
        kb = gathered(kp, table, b, T, 16)
        sb = oracle.block_summaries(kb, T, 16)
        raw, _ = oracle.group_scores(np_bits(q[b:b + 1]), sb, T, 16)
        keff = min(10, ksa.nblocks(T, 16))
        ib = idx[b].cpu().numpy()
        assert np.all(ib[:, keff:] == -1)
        check_block_selection(ib[:, :keff], raw.reshape(w.Hkv, -1), 10)


def test_paged_newest_block_refresh_only():
    """first_block = -1 rewrites each sequence's own newest block and nothing else."""
    lens = [100, 33, 64]
    w, q, k, v, kp, vp, table, seq = paged_inputs(lens, 16, seed=9, Hq=4, Hkv=2, D=128, dtype="bf16")
    s = torch.full((w.B, w.Hkv, table.shape[1], w.D), 3, dtype=k.dtype, device=DEV)
    ksa.ksa_paged_block_summaries(kp, s, table, seq, newest_only=True)
    got = np_bits(s)
    for b, T in enumerate(lens):
        j = (T - 1) // 16
        ref = oracle.block_summaries(gathered(kp, table, b, T, 16), T, 16)
        np.testing.assert_array_equal(got[b, :, j], ref[0, :, j])
        others = [i for i in range(table.shape[1]) if i != j]
        assert np.all(s[b, :, others].float().cpu().numpy() == 3)


# ----------------------------------------------------------------------------- the vote path
VOTE_PAGED = [
    dict(lens=[5000, 3000, 900, 1], Bs=16, Hq=32, Hkv=8, D=128, dtype="bf16", N=1024, W=256),  # MFMA
    dict(lens=[2100, 700, 1500], Bs=7, Hq=8, Hkv=2, D=64, dtype="f32", N=512, W=128),
    dict(lens=[400, 300], Bs=16, Hq=4, Hkv=2, D=64, dtype="bf16", N=512, W=64),    # all T_b <= N
    # histories past 32768 tokens: the two-kernel tally and set, per-sequence lengths
    dict(lens=[40000, 34000, 2000, 600], Bs=16, Hq=8, Hkv=2, D=128, dtype="bf16", N=1024, W=256),
]


@pytest.mark.parametrize("case", VOTE_PAGED, ids=lambda c: "G%d-Bs%d-%s" % (
    c["Hq"] // c["Hkv"], c["Bs"], "_".join(map(str, c["lens"]))))
def test_paged_vote_and_token_attention_match_oracle_per_sequence(case):
    c = dict(case)
    lens, Bs, N, W = c.pop("lens"), c.pop("Bs"), c.pop("N"), c.pop("W")
    w, q, k, v, kp, vp, table, seq = paged_inputs(lens, Bs, seed=sum(lens) % 997, **c)
    idx, votes = ksa.ksa_paged_vote_select(q, kp, table, seq, N, W, want_votes=True)
    out, lse = ksa.ksa_paged_sparse_decode(q, kp, vp, table, seq, idx, ksa.KSA_SEL_TOKENS)
    torch.cuda.synchronize()
    ids, vts = idx.cpu().numpy(), votes.cpu().numpy()
    from parity import check_votes
    for b, T in enumerate(lens):
        kb, vb = gathered(kp, table, b, T, Bs), gathered(vp, table, b, T, Bs)
        qb = np_bits(q[b:b + 1])
        row = ids[b][ids[b] >= 0]
        if T <= N:
            assert row.tolist() == list(range(T)) and np.all(vts[b] == 0)
        else:
            lg = oracle.head_logits(qb, kb, T)
            assert row.shape[0] == N and np.all(ids[b] >= 0)
            check_votes(vts[b:b + 1, :T], row[None], lg, N, W)
            assert np.all(vts[b, T - W:] == 0)
        ro, rl = oracle.attend_tokens(qb, kb, vb, T, row[None].astype(np.int32))
        check_attention(out[b:b + 1].cpu().numpy(), lse[b:b + 1].cpu().numpy(), ro, rl)


def test_paged_vote_equals_contiguous_vote_bitwise():
    T, Bs, N, W = 4000, 16, 512, 128
    w, q, k, v, kp, vp, table, seq = paged_inputs([T] * 3, Bs, seed=77, Hq=32, Hkv=8, D=128,
                                                  dtype="bf16")
    pi, pv = ksa.ksa_paged_vote_select(q, kp, table, seq, N, W, want_votes=True)
    ci, cv = ksa.ksa_vote_select(q, k, T, N, W, want_votes=True)
    torch.cuda.synchronize()
    assert torch.equal(pi, ci) and torch.equal(pv[:, :T], cv)
    po, pl = ksa.ksa_paged_sparse_decode(q, kp, vp, table, seq, pi, ksa.KSA_SEL_TOKENS)
    co, cl = ksa.ksa_sparse_decode(q, k, v, T, ci, ksa.KSA_SEL_TOKENS)
    torch.cuda.synchronize()
    assert torch.equal(po, co) and torch.equal(pl, cl)


def test_paged_vote_equals_contiguous_vote_bitwise_long_history():
    """Histories past 32768 tokens take the two-kernel tally; at one length
    the paged and contiguous calls still agree bit for bit."""
    T, Bs, N, W = 36000, 16, 2048, 512
    w, q, k, v, kp, vp, table, seq = paged_inputs([T] * 2, Bs, seed=78, Hq=8, Hkv=2, D=128,
                                                  dtype="bf16")
    pi, pv = ksa.ksa_paged_vote_select(q, kp, table, seq, N, W, want_votes=True)
    ci, cv = ksa.ksa_vote_select(q, k, T, N, W, want_votes=True)
    torch.cuda.synchronize()
    assert torch.equal(pi, ci) and torch.equal(pv[:, :T], cv)


LAYER_PAGED = [
    dict(lens=[5000, 3000, 900, 1], Bs=16, Hq=32, Hkv=8, D=128, dtype="bf16", N=1024, W=256),  # G 4
    dict(lens=[2500, 1200, 2047], Bs=32, Hq=16, Hkv=2, D=128, dtype="bf16", N=512, W=128),     # G 8
    dict(lens=[1500, 400, 999], Bs=7, Hq=8, Hkv=4, D=64, dtype="f32", N=256, W=64),            # two passes
    dict(lens=[300, 200], Bs=16, Hq=8, Hkv=2, D=128, dtype="bf16", N=512, W=128),              # no vote
    dict(lens=[34000, 2000], Bs=16, Hq=8, Hkv=2, D=128, dtype="bf16", N=1024, W=256),          # long
]


@pytest.mark.parametrize("case", LAYER_PAGED, ids=lambda c: "G%d-%s-%s" % (
    c["Hq"] // c["Hkv"], c["dtype"], "_".join(map(str, c["lens"]))))
def test_paged_selection_layer_equals_dense_plus_vote(case):
    """The paged selection layer gives ksa_paged_dense_decode's outputs and
    ksa_paged_vote_select's set and votes, bit for bit (on MFMA shapes the
    vote's keys come from the dense walk's own logits)."""
    c = dict(case)
    lens, Bs, N, W = c.pop("lens"), c.pop("Bs"), c.pop("N"), c.pop("W")
    w, q, k, v, kp, vp, table, seq = paged_inputs(lens, Bs, seed=sum(lens) % 991, **c)
    out, lse, idx, votes = ksa.ksa_paged_vote_layer_decode(q, kp, vp, table, seq, N, W,
                                                           want_votes=True)
    do, dl = ksa.ksa_paged_dense_decode(q, kp, vp, table, seq)
    vi, vv = ksa.ksa_paged_vote_select(q, kp, table, seq, N, W, want_votes=True)
    torch.cuda.synchronize()
    assert torch.equal(out, do) and torch.equal(lse, dl)
    assert torch.equal(idx, vi) and torch.equal(votes, vv)
    # and the layer's set is the oracle's rule on the layer's own votes
    from parity import check_votes
    ids, vts = idx.cpu().numpy(), votes.cpu().numpy()
    for b, T in enumerate(lens):
        if T <= N:
            assert ids[b][ids[b] >= 0].tolist() == list(range(T))
            continue
        if T > 6000:  # the oracle's logits of the long row are covered by the paged vote tests
            continue
        kb = gathered(kp, table, b, T, Bs)
        lg = oracle.head_logits(np_bits(q[b:b + 1]), kb, T)
        check_votes(vts[b:b + 1, :T], ids[b][None], lg, N, W)


def test_paged_sparse_decode_of_the_steps_blocks_equals_the_step():
    """Attending the paged step's own ids (padding included) with the
    separate paged call gives the step's outputs (to fp32 merge order)."""
    lens = [3000, 700, 40]
    w, q, k, v, kp, vp, table, seq = paged_inputs(lens, 16, seed=31, Hq=8, Hkv=2, D=128,
                                                  dtype="bf16")
    s = torch.zeros((w.B, w.Hkv, table.shape[1], w.D), dtype=k.dtype, device=DEV)
    ksa.ksa_paged_block_summaries(kp, s, table, seq)
    out, lse, idx = ksa.ksa_paged_block_topk_decode(q, kp, vp, s, table, seq, 32,
                                                    want_block_idx=True)
    o2, l2 = ksa.ksa_paged_sparse_decode(q, kp, vp, table, seq, idx, ksa.KSA_SEL_BLOCKS)
    torch.cuda.synchronize()
    assert float((out - o2).abs().max()) <= 1e-5 and float((lse - l2).abs().max()) <= 1e-5


# ----------------------------------------------------------------------------- selection variants
SELECT_PAGED = [
    dict(lens=[3000, 700, 16, 1], Bs=16, Hq=8, Hkv=2, D=128, dtype="bf16", top_k=20),
    dict(lens=[1200, 999, 65], Bs=32, Hq=16, Hkv=2, D=128, dtype="bf16", top_k=8),
    dict(lens=[500, 333], Bs=7, Hq=4, Hkv=4, D=64, dtype="f32", top_k=30),
]


@pytest.mark.parametrize("case", SELECT_PAGED, ids=case_id)
def test_paged_select_ex_sum_equals_the_paged_steps_selection(case):
    """With the method's own ranking the separate paged selection picks the
    paged step's blocks, bit for bit (the same scores and the same search)."""
    c = dict(case)
    lens, Bs, top_k = c.pop("lens"), c.pop("Bs"), c.pop("top_k")
    w, q, k, v, kp, vp, table, seq = paged_inputs(lens, Bs, seed=sum(lens) % 313, **c)
    s = torch.zeros((w.B, w.Hkv, table.shape[1], w.D), dtype=k.dtype, device=DEV)
    ksa.ksa_paged_block_summaries(kp, s, table, seq)
    idx = ksa.ksa_paged_select_topk_ex(q, s, table, seq, Bs, top_k)
    _, _, sidx = ksa.ksa_paged_block_topk_decode(q, kp, vp, s.clone(), table, seq, top_k,
                                                 refresh_last_block=False, want_block_idx=True)
    torch.cuda.synchronize()
    assert torch.equal(idx, sidx)


@pytest.mark.parametrize("agg", [ksa.KSA_AGG_SUM, ksa.KSA_AGG_MAX])
@pytest.mark.parametrize("case", SELECT_PAGED, ids=case_id)
def test_paged_select_ex_variants_match_oracle_per_sequence(case, agg):
    """MAX aggregation and the forced newest block on a paged cache: each row
    ranks its own blocks by the oracle's relevance of that aggregation, keeps
    its own newest block, and pads with -1."""
    c = dict(case)
    lens, Bs, top_k = c.pop("lens"), c.pop("Bs"), c.pop("top_k")
    w, q, k, v, kp, vp, table, seq = paged_inputs(lens, Bs, seed=sum(lens) % 317 + agg, **c)
    s = torch.zeros((w.B, w.Hkv, table.shape[1], w.D), dtype=k.dtype, device=DEV)
    ksa.ksa_paged_block_summaries(kp, s, table, seq)
    name = "max" if agg == ksa.KSA_AGG_MAX else "sum"
    plain, sc = ksa.ksa_paged_select_topk_ex(q, s, table, seq, Bs, top_k, aggregate=agg,
                                             want_scores=True)
    forced = ksa.ksa_paged_select_topk_ex(q, s, table, seq, Bs, top_k, aggregate=agg,
                                          force_last_block=True)
    torch.cuda.synchronize()
    sb_all = np_bits(s)
    for b, T in enumerate(lens):
        nb = ksa.nblocks(T, Bs)
        keff = min(top_k, nb)
        qb = np_bits(q[b:b + 1])
        raw, scaled = oracle.group_scores(qb, sb_all[b:b + 1], T, Bs, Tcap=table.shape[1] * Bs,
                                          aggregate=name)
        raw = raw.reshape(w.Hkv, -1)
        ids = plain[b].cpu().numpy()
        assert np.all(ids[:, keff:] == -1)
        check_block_selection(np.ascontiguousarray(ids[:, :keff]), raw, top_k)
        np.testing.assert_allclose(sc[b, :, :nb].cpu().numpy(), scaled[0], rtol=0,
                                   atol=1e-5 * max(1.0, float(np.abs(scaled).max())))
        fid = forced[b].cpu().numpy()
        assert np.all(fid[:, keff:] == -1)
        fid = fid[:, :keff]
        assert np.all(np.any(fid == nb - 1, axis=1))
        if keff < nb:
            rest = raw.copy()
            rest[:, nb - 1] = raw.min() - 1.0
            others = np.array([[j for j in row if j != nb - 1] for row in fid])
            check_block_selection(others, rest, keff - 1)


@pytest.mark.parametrize("heads", [[0], [3, 9], list(range(16))])
def test_paged_vote_of_chosen_heads(heads):
    """Only the listed heads vote on a paged cache: at one length it is the
    contiguous call bit for bit; with ragged lengths each sequence's votes
    are the listed heads' picks over its own history (oracle rule)."""
    N, W, Bs = 512, 128, 16
    w, q, k, v, kp, vp, table, seq = paged_inputs([3000] * 2, Bs, seed=81 + len(heads), Hq=16,
                                                  Hkv=4, D=128, dtype="bf16")
    pi, pv = ksa.ksa_paged_vote_select_heads(q, kp, table, seq, N, W, heads, want_votes=True)
    ci, cv = ksa.ksa_vote_select_heads(q, k, 3000, N, W, heads, want_votes=True)
    torch.cuda.synchronize()
    assert torch.equal(pi, ci) and torch.equal(pv[:, :3000], cv)
    from parity import check_votes
    lens = [2500, 400, 1800]
    w, q, k, v, kp, vp, table, seq = paged_inputs(lens, Bs, seed=91 + len(heads), Hq=16, Hkv=4,
                                                  D=128, dtype="bf16")
    idx, votes = ksa.ksa_paged_vote_select_heads(q, kp, table, seq, N, W, heads, want_votes=True)
    torch.cuda.synchronize()
    ids, vts = idx.cpu().numpy(), votes.cpu().numpy()
    for b, T in enumerate(lens):
        row = ids[b][ids[b] >= 0]
        if T <= N:
            assert row.tolist() == list(range(T))
            continue
        kb = gathered(kp, table, b, T, Bs)
        lg = oracle.head_logits(np_bits(q[b:b + 1]), kb, T)[:, heads]
        check_votes(vts[b:b + 1, :T], row[None], lg, N, W)


PER_HEAD_PAGED = [
    dict(lens=[4000, 900, 300, 1], Hq=16, Hkv=4, D=128, dtype="bf16", N=512, W=128),
    dict(lens=[2100, 1500], Hq=8, Hkv=2, D=64, dtype="f32", N=300, W=60),
]


@pytest.mark.parametrize("case", PER_HEAD_PAGED, ids=lambda c: "G%d-%s-%s" % (
    c["Hq"] // c["Hkv"], c["dtype"], "_".join(map(str, c["lens"]))))
def test_paged_per_head_sets_and_their_attention(case):
    """Per-head sets on a paged cache: every head's own picks over its
    sequence's history (oracle rule per sequence; a sequence no longer than
    N keeps all its tokens, then -1), and attention over one list per query
    head through the block table against the oracle."""
    from test_gpu_variants import check_head_sets
    c = dict(case)
    lens, N, W, Bs = c.pop("lens"), c.pop("N"), c.pop("W"), 16
    w, q, k, v, kp, vp, table, seq = paged_inputs(lens, Bs, seed=sum(lens) % 331, **c)
    idx = ksa.ksa_paged_vote_select_per_head(q, kp, table, seq, N, W)
    out, lse = ksa.ksa_paged_sparse_decode(q, kp, vp, table, seq, idx, ksa.KSA_SEL_HEAD_TOKENS)
    torch.cuda.synchronize()
    ids = idx.cpu().numpy()
    for b, T in enumerate(lens):
        kb, vb = gathered(kp, table, b, T, Bs), gathered(vp, table, b, T, Bs)
        qb = np_bits(q[b:b + 1])
        if T <= N:
            row = ids[b][:, :T]
            assert np.all(ids[b][:, T:] == -1)
            assert np.all(row == np.arange(T)[None])
        else:
            row = ids[b]
            check_head_sets(row[None], oracle.head_logits(qb, kb, T), N, W)
        ro, rl = oracle.attend_head_tokens(qb, kb, vb, T, np.ascontiguousarray(row[None]))
        check_attention(out[b:b + 1].cpu().numpy(), lse[b:b + 1].cpu().numpy(), ro, rl)


def test_paged_per_head_sets_equal_contiguous_bitwise():
    T, Bs, N, W = 3000, 16, 512, 128
    w, q, k, v, kp, vp, table, seq = paged_inputs([T] * 2, Bs, seed=97, Hq=16, Hkv=4, D=128,
                                                  dtype="bf16")
    pi = ksa.ksa_paged_vote_select_per_head(q, kp, table, seq, N, W)
    ci = ksa.ksa_vote_select_per_head(q, k, T, N, W)
    torch.cuda.synchronize()
    assert torch.equal(pi, ci)
    po, pl = ksa.ksa_paged_sparse_decode(q, kp, vp, table, seq, pi, ksa.KSA_SEL_HEAD_TOKENS)
    co, cl = ksa.ksa_sparse_decode(q, k, v, T, ci, ksa.KSA_SEL_HEAD_TOKENS)
    torch.cuda.synchronize()
    assert torch.equal(po, co) and torch.equal(pl, cl)


def _canary(shape, dtype, fill, extra=4096):
    """A buffer of `shape` followed by `extra` elements of `fill`; returns
    (view of the front, the whole buffer)."""
    n = int(np.prod(shape))
    buf = torch.full((n + extra,), fill, dtype=dtype, device=DEV)
    return buf[:n].view(*shape), buf


def _ws(prob, op, param):
    need = max(16, ksa.ksa_workspace_bytes(prob, op, param))
    front, buf = _canary((need,), torch.uint8, 0x5A, extra=1 << 16)
    return front, buf, need


@pytest.mark.parametrize("G,D,dtype", [(4, 128, "bf16"), (2, 64, "f32")], ids=["mfma", "valu"])
def test_paged_lengths_past_seq_len_are_clamped(G, D, dtype):
    """A length above the call's seq_len T acts as T in every paged call: the
    outputs equal those of the same call with the lengths clamped, and no
    write lands past the buffers sized from T (votes [B,T], token_idx,
    block_idx, block_scores, workspaces)."""
    Bs, T, N, W, top_k = 16, 800, 256, 64, 12
    lens = [700, 1100, 300]
    w, q, k, v, kp, vp, table, seq = paged_inputs(lens, Bs, seed=91, Hq=G * 2, Hkv=2, D=D,
                                                  dtype=dtype)
    seq_c = torch.tensor([min(t, T) for t in lens], dtype=torch.int32, device=DEV)
    B, Hkv, mb = w.B, w.Hkv, table.shape[1]
    prob, _ = ksa._paged_args(q, kp, table, seq, T, 0.0)
    NB = ksa.nblocks(T, Bs)

    def run(lengths):
        r = {}
        s = torch.zeros((B, Hkv, mb, D), dtype=kp.dtype, device=DEV)
        ksa.ksa_paged_block_summaries(kp, s, table, lengths, max_len=T)
        r["summ"] = s.clone()
        idx, ib = _canary((B, Hkv, top_k), torch.int32, -7)
        r["step"] = ksa.ksa_paged_block_topk_decode(q, kp, vp, s, table, lengths, top_k, max_len=T,
                                                    block_idx=idx)
        r["idx_pad"] = ib[idx.numel():]
        ws, wb, need = _ws(prob, ksa.KSA_OP_PAGED_DENSE, 0)
        r["dense"] = ksa.ksa_paged_dense_decode(q, kp, vp, table, lengths, max_len=T, workspace=ws)
        r["dense_ws_pad"] = wb[need:]
        sc, sb = _canary((B, Hkv, NB), torch.float32, -3.0)
        ws, wb, need = _ws(prob, ksa.KSA_OP_SELECT_TOPK, top_k)
        ids2, ib2 = _canary((B, Hkv, top_k), torch.int32, -7)
        ksa.ksa_paged_select_topk_ex(q, r["summ"], table, lengths, Bs, top_k, max_len=T,
                                     block_idx=ids2, block_scores=sc, workspace=ws)
        r["sel_ex"], r["scores"] = ids2.clone(), sc.clone()
        r["sel_pads"] = (sb[sc.numel():], ib2[ids2.numel():], wb[need:])
        tok, tb = _canary((B, min(N, T)), torch.int32, -9)
        votes, vb = _canary((B, T), torch.uint8, 0xAB)
        ws, wb, need = _ws(prob, ksa.KSA_OP_VOTE_SELECT, N)
        ksa.ksa_paged_vote_select(q, kp, table, lengths, N, W, max_len=T, token_idx=tok,
                                  votes=votes, workspace=ws)
        r["vote"] = (tok.clone(), votes.clone())
        r["vote_pads"] = (tb[tok.numel():], vb[votes.numel():], wb[need:])
        ws, wb, need = _ws(prob, ksa.KSA_OP_SPARSE_TOKENS, tok.shape[1])
        r["tok_attn"] = ksa.ksa_paged_sparse_decode(q, kp, vp, table, lengths, tok, max_len=T,
                                                    workspace=ws)
        r["tok_ws_pad"] = wb[need:]
        tok2, tb2 = _canary((B, min(N, T)), torch.int32, -9)
        votes2, vb2 = _canary((B, T), torch.uint8, 0xAB)
        ws, wb, need = _ws(prob, ksa.KSA_OP_PAGED_VOTE_LAYER, N)
        r["layer"] = ksa.ksa_paged_vote_layer_decode(q, kp, vp, table, lengths, N, W, max_len=T,
                                                     token_idx=tok2, votes=votes2, workspace=ws)
        r["layer_pads"] = (tb2[tok2.numel():], vb2[votes2.numel():], wb[need:])
        torch.cuda.synchronize()
        return r

    got, ref = run(seq), run(seq_c)
    assert torch.equal(got["summ"], ref["summ"])
    for a, b in zip(got["step"], ref["step"]):
        assert torch.equal(a, b)
    for a, b in zip(got["dense"], ref["dense"]):
        assert torch.equal(a, b)
    assert torch.equal(got["sel_ex"], ref["sel_ex"]) and torch.equal(got["scores"], ref["scores"])
    for a, b in zip(got["vote"], ref["vote"]):
        assert torch.equal(a, b)
    for a, b in zip(got["tok_attn"], ref["tok_attn"]):
        assert torch.equal(a, b)
    for a, b in zip(got["layer"], ref["layer"]):
        assert torch.equal(a, b)
    # nothing written past the T-sized buffers
    assert torch.all(got["idx_pad"] == -7)
    assert torch.all(got["dense_ws_pad"] == 0x5A)
    sp, ip, wp = got["sel_pads"]
    assert torch.all(sp == -3.0) and torch.all(ip == -7) and torch.all(wp == 0x5A)
    for pad, fill in zip(got["vote_pads"], (-9, 0xAB, 0x5A)):
        assert torch.all(pad == fill)
    assert torch.all(got["tok_ws_pad"] == 0x5A)
    for pad, fill in zip(got["layer_pads"], (-9, 0xAB, 0x5A)):
        assert torch.all(pad == fill)
