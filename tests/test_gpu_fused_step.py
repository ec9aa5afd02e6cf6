"""GPU parity of ksa_block_topk_decode, the one-launch decode step.

Every case starts from summaries built before the newest token was appended
(so the refresh has real work), runs the fused step, and checks it against
(a) the three separate calls on the same inputs -- summaries and block ids
bitwise, outputs bitwise where the separate attention runs one split of 8
waves per row and within 1e-5 otherwise -- and (b) the fp64 oracle, under the
acceptance rules of tests/parity.py.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_decode_ksa_amd as ksa
from sparse_attention_decode_ksa_amd.inputs import WORKLOADS, small_workload
from parity import check_attention, check_block_selection
from test_gpu_parity import DEV, gpu_inputs, np_bits

pytestmark = pytest.mark.gpu


def stale_summaries(k, w, seed=0):
    """Summaries as they stood before token T-1 was appended: the newest block
    holds its mean over one token fewer, or garbage when T-1 opens it."""
    s = torch.zeros((w.B, w.Hkv, ksa.nblocks(w.cap, w.Bs), w.D), dtype=k.dtype, device=DEV)
    jref = (w.T - 1) // w.Bs
    if w.T > 1:
        ksa.ksa_block_summaries(k, s, w.T - 1, w.Bs)
    if (w.T - 1) % w.Bs == 0:
        g = torch.Generator(device=DEV)
        g.manual_seed(seed)
        s[:, :, jref] = (torch.randn(s[:, :, jref].shape, generator=g, device=DEV) * 3).to(k.dtype)
    return s


def separate_step(w, q, k, v, s, refresh=True):
    if refresh:
        ksa.ksa_block_summaries(k, s, w.T, w.Bs, first_block=(w.T - 1) // w.Bs, num_blocks=1)
    idx = ksa.ksa_select_topk(q, s, w.T, w.Bs, w.top_k, max_seq_len=w.cap)
    out, lse = ksa.ksa_sparse_decode(q, k, v, w.T, idx, ksa.KSA_SEL_BLOCKS, block_size=w.Bs)
    return idx, out, lse


def fused_vs_separate(w, q, k, v, refresh=True, bitwise_out=False, seed=0):
    s0 = stale_summaries(k, w, seed) if refresh else None
    if s0 is None:
        s0 = torch.zeros((w.B, w.Hkv, ksa.nblocks(w.cap, w.Bs), w.D), dtype=k.dtype, device=DEV)
        ksa.ksa_block_summaries(k, s0, w.T, w.Bs)
    s_sep, s_f = s0.clone(), s0.clone()
    idx_sep, out_sep, lse_sep = separate_step(w, q, k, v, s_sep, refresh)
    out_f, lse_f, idx_f = ksa.ksa_block_topk_decode(q, k, v, s_f, w.T, w.Bs, w.top_k,
                                                    refresh_last_block=refresh, want_block_idx=True)
    torch.cuda.synchronize()
    assert torch.equal(s_f, s_sep)
    assert torch.equal(idx_f, idx_sep)
    if bitwise_out:
        assert torch.equal(out_f, out_sep) and torch.equal(lse_f, lse_sep)
    else:
        assert float((out_f - out_sep).abs().max()) <= 1e-5
        assert float((lse_f - lse_sep).abs().max()) <= 1e-5
    return s_f, idx_f, out_f, lse_f


def check_against_oracle(w, q, k, v, s, idx, out, lse, seqs):
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
    return swaps


STEP_CASES = [
    dict(B=2, Hq=4, Hkv=2, D=64, T=1024, Bs=16, dtype="f32", top_k=8),
    dict(B=3, Hq=8, Hkv=1, D=128, T=3000, Bs=16, dtype="bf16", top_k=64),     # MFMA, G = 8
    dict(B=2, Hq=16, Hkv=4, D=128, T=4099, Bs=32, dtype="bf16", top_k=20),    # MFMA, G = 4
    dict(B=2, Hq=2, Hkv=2, D=64, T=517, Bs=7, dtype="bf16", top_k=30),        # Bs not 2^n
    dict(B=1, Hq=4, Hkv=4, D=128, T=200, Bs=1, dtype="f32", top_k=17),        # one-token blocks
    dict(B=2, Hq=4, Hkv=2, D=64, T=64, Bs=16, dtype="bf16", top_k=9),         # k > NB
    dict(B=2, Hq=4, Hkv=2, D=128, T=1025, Bs=16, dtype="bf16", top_k=12),     # T-1 opens a block
    dict(B=1, Hq=16, Hkv=2, D=128, T=1000, Bs=64, dtype="f32", top_k=5),      # largest refreshed Bs
    dict(B=1, Hq=4, Hkv=1, D=128, T=1, Bs=16, dtype="bf16", top_k=4),         # a single token
    dict(B=1, Hq=2, Hkv=1, D=128, T=65536, Bs=16, dtype="bf16", top_k=2048),  # NB and k_eff limits
    dict(B=8, Hq=16, Hkv=8, D=128, T=16384, Bs=16, dtype="bf16", top_k=64),
]


def step_id(c):
    return "%s-G%d-D%d-T%d-Bs%d-k%d" % (c["dtype"], c["Hq"] // c["Hkv"], c["D"], c["T"], c["Bs"],
                                        c["top_k"])


@pytest.mark.parametrize("case", STEP_CASES, ids=step_id)
def test_fused_step_matches_separate_calls_and_oracle(case):
    w = small_workload(seed=case["T"] + 3, **case)
    q, k, v = gpu_inputs(w)
    s, idx, out, lse = fused_vs_separate(w, q, k, v, refresh=True, seed=case["T"])
    check_against_oracle(w, q, k, v, s, idx, out, lse, range(min(w.B, 2)))


@pytest.mark.parametrize("case", STEP_CASES[:4], ids=step_id)
def test_fused_step_without_refresh(case):
    w = small_workload(seed=case["T"] + 4, **case)
    q, k, v = gpu_inputs(w)
    s, idx, out, lse = fused_vs_separate(w, q, k, v, refresh=False)
    check_against_oracle(w, q, k, v, s, idx, out, lse, [0])


@pytest.mark.parametrize("G,Bs,dtype", [(1, 16, "bf16"), (2, 16, "bf16"), (4, 32, "bf16"),
                                        (8, 16, "bf16"), (2, 16, "f32")])
def test_fused_step_integer_ties_are_bit_exact(G, Bs, dtype):
    """Integer q and K with blocks 32..63 repeating blocks 0..31: every score
    occurs twice, exactly, so the lowest-id tie rule decides and must agree
    with the oracle bit for bit."""
    w = small_workload(B=3, Hq=2 * G, Hkv=2, D=64, T=64 * Bs, Bs=Bs, dtype=dtype, top_k=13, seed=G)
    q, k, v = gpu_inputs(w, integer=True, lo=-1, hi=1)
    k[:, :, 32 * Bs:] = k[:, :, :32 * Bs]
    s = stale_summaries(k, w)
    out, lse, idx = ksa.ksa_block_topk_decode(q, k, v, s, w.T, w.Bs, w.top_k, want_block_idx=True)
    sb = oracle.block_summaries(np_bits(k), w.T, w.Bs)
    np.testing.assert_array_equal(np_bits(s)[:, :, :w.NB], sb[:, :, :w.NB])
    raw, _ = oracle.group_scores(np_bits(q), sb, w.T, w.Bs)
    assert np.array_equal(raw[..., :32], raw[..., 32:])
    np.testing.assert_array_equal(idx.cpu().numpy(), oracle.topk(raw, w.top_k))
    ro, rl = oracle.attend_blocks(np_bits(q), np_bits(k), np_bits(v), w.T, w.Bs, idx.cpu().numpy())
    check_attention(out.cpu().numpy(), lse.cpu().numpy(), ro, rl)


VARLEN_CASES = [
    dict(lens=[1000, 17, 1, 512], Bs=16, Hq=4, Hkv=2, D=64, dtype="bf16", top_k=8),
    dict(lens=[3000, 2048, 777], Bs=16, Hq=8, Hkv=1, D=128, dtype="bf16", top_k=64),   # MFMA G = 8
    dict(lens=[4099, 64, 2000], Bs=32, Hq=16, Hkv=4, D=128, dtype="bf16", top_k=20),   # MFMA G = 4
    dict(lens=[517, 200, 7], Bs=7, Hq=2, Hkv=2, D=64, dtype="bf16", top_k=30),         # Bs not 2^n
    dict(lens=[1025, 1024, 33], Bs=16, Hq=4, Hkv=2, D=128, dtype="f32", top_k=12),     # T-1 opens a block
    dict(lens=[200, 150], Bs=1, Hq=4, Hkv=4, D=128, dtype="f32", top_k=17),            # one-token blocks
]


def varlen_inputs(lens, Bs, seed, **kw):
    """A contiguous cache holding sequences of the given lengths, and summaries
    as they stood before each sequence's newest token (its newest block holds
    noise, so the refresh does real work)."""
    T = max(lens)
    w = small_workload(B=len(lens), T=T, Tcap=T + 2 * Bs, Bs=Bs, seed=seed, **kw)
    q, k, v = gpu_inputs(w)
    s = torch.zeros((w.B, w.Hkv, ksa.nblocks(w.cap, Bs), w.D), dtype=k.dtype, device=DEV)
    for b, Tb in enumerate(lens):
        ksa.ksa_block_summaries(k[b:b + 1], s[b:b + 1], Tb, Bs)
        s[b, :, (Tb - 1) // Bs] = (torch.randn(s[b, :, 0].shape, device=DEV) * 3).to(s.dtype)
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    return w, q, k, v, s, seq


@pytest.mark.parametrize("case", VARLEN_CASES, ids=lambda c: "%s-G%d-D%d-Bs%d-k%d-%s" % (
    c["dtype"], c["Hq"] // c["Hkv"], c["D"], c["Bs"], c["top_k"], "_".join(map(str, c["lens"]))))
def test_fused_step_varlen_matches_oracle_per_sequence(case):
    """One length per sequence on a contiguous cache: every sequence's newest
    block is refreshed, its own blocks ranked and its own tokens attended
    (oracle per sequence on its own length); ids past a row's k_eff are -1."""
    c = dict(case)
    lens, Bs, top_k = c.pop("lens"), c.pop("Bs"), c.pop("top_k")
    w, q, k, v, s, seq = varlen_inputs(lens, Bs, seed=sum(lens) % 499, **c)
    out, lse, idx = ksa.ksa_block_topk_decode_varlen(q, k, v, s, seq, Bs, top_k, max_len=w.T,
                                                     want_block_idx=True)
    torch.cuda.synchronize()
    got_s, ids = np_bits(s), idx.cpu().numpy()
    assert ids.shape[2] == min(top_k, ksa.nblocks(w.T, Bs))
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


@pytest.mark.parametrize("G,Bs,dtype,T", [(2, 16, "bf16", 5000), (4, 32, "bf16", 4097),
                                           (8, 16, "bf16", 3001), (1, 16, "f32", 999)])
def test_fused_step_varlen_at_one_length_equals_the_step_bitwise(G, Bs, dtype, T):
    """Every length equal to T: the varlen call is the plain step bit for bit."""
    w = small_workload(B=5, Hq=2 * G, Hkv=2, D=128 if dtype == "bf16" else 64, T=T, Bs=Bs,
                       dtype=dtype, top_k=24, seed=T)
    q, k, v = gpu_inputs(w)
    s1 = stale_summaries(k, w)
    s2 = s1.clone()
    o1, l1, i1 = ksa.ksa_block_topk_decode(q, k, v, s1, w.T, w.Bs, w.top_k, want_block_idx=True)
    seq = torch.full((w.B,), T, dtype=torch.int32, device=DEV)
    o2, l2, i2 = ksa.ksa_block_topk_decode_varlen(q, k, v, s2, seq, w.Bs, w.top_k, max_len=T,
                                                  want_block_idx=True)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2) and torch.equal(i1, i2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fused_step_optional_outputs():
    """block_idx and lse are optional; leaving them out changes nothing else."""
    w = small_workload(B=4, Hq=8, Hkv=4, D=128, T=5000, Bs=16, dtype="bf16", top_k=40, seed=8)
    q, k, v = gpu_inputs(w)
    s1, s2 = stale_summaries(k, w), stale_summaries(k, w)
    o1, l1, i1 = ksa.ksa_block_topk_decode(q, k, v, s1, w.T, w.Bs, w.top_k, want_block_idx=True)
    o2, l2, i2 = ksa.ksa_block_topk_decode(q, k, v, s2, w.T, w.Bs, w.top_k, want_lse=False)
    torch.cuda.synchronize()
    assert l2 is None and i2 is None
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@pytest.mark.parametrize("name,seqs,bitwise", [("c2", [0, 37, 63], True), ("c3", [0, 31], True),
                                               ("c5", [0, 255], False)])
def test_fused_step_full_workloads(name, seqs, bitwise):
    """The full-size block top-k workloads.  c2 and c3 run one 8-wave
    workgroup per row on both paths, so the fused step equals the separate
    calls bit for bit; c5 has more rows than the chip holds 8-wave
    workgroups, so the fused step uses 4-wave workgroups and agrees to fp32
    merge-order rounding."""
    w = WORKLOADS[name]
    q, k, v = gpu_inputs(w)
    s, idx, out, lse = fused_vs_separate(w, q, k, v, refresh=True, bitwise_out=bitwise)
    check_against_oracle(w, q, k, v, s, idx, out, lse, seqs)
    del q, k, v
    torch.cuda.empty_cache()


def test_fused_step_graph_replay_matches_eager():
    """The fused step captured in a HIP graph and replayed with new queries
    (eager work in between) matches eager calls every time."""
    w = small_workload(B=8, Hq=16, Hkv=8, D=128, T=4000, Bs=16, dtype="bf16", top_k=32, seed=22)
    q, k, v = gpu_inputs(w)
    s = stale_summaries(k, w)
    s_ref = s.clone()
    idx = torch.empty((w.B, w.Hkv, w.top_k), dtype=torch.int32, device=DEV)
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device=DEV)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=DEV)
    stream = torch.cuda.Stream()
    qbuf = q.clone()

    def step():
        ksa.ksa_block_topk_decode(qbuf, k, v, s, w.T, w.Bs, w.top_k, block_idx=idx, out=out,
                                  lse=lse, stream=stream)

    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    torch.cuda.synchronize()
    gen = torch.Generator(device=DEV)
    gen.manual_seed(6)
    for rep in range(4):
        newq = torch.randn(q.shape, generator=gen, device=DEV).to(q.dtype)
        qbuf.copy_(newq)
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        got = (idx.clone(), out.clone(), lse.clone())
        s_e = s_ref.clone()
        e_out, e_lse, e_idx = ksa.ksa_block_topk_decode(newq, k, v, s_e, w.T, w.Bs, w.top_k,
                                                        want_block_idx=True)
        torch.cuda.synchronize()
        assert torch.equal(got[0], e_idx), rep
        assert torch.equal(got[1], e_out) and torch.equal(got[2], e_lse), rep
        assert torch.equal(s, s_e), rep
