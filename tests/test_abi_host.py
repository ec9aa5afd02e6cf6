"""Host-side checks of the C ABI (no GPU): the library loads, exports every
entry point include/ksa.h declares, sizes workspaces as a pure function, and
rejects invalid arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

import sparse_attention_decode_ksa_amd as ksa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ksa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ksa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_five_operations():
    names = declared_functions()
    for n in ("ksa_block_summaries", "ksa_select_topk", "ksa_sparse_decode", "ksa_vote_select",
              "ksa_dense_decode", "ksa_block_topk_decode", "ksa_workspace_bytes",
              "ksa_status_string", "ksa_version"):
        assert n in names
    assert set(names) == set(ksa.EXPORTED)


def test_library_loads_and_exports_every_declared_symbol():
    lib = ksa.load_library()
    raw = ctypes.CDLL(ksa.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name
    assert re.fullmatch(r"\d+\.\d+\.\d+", ksa.ksa_version())
    assert lib is ksa.load_library()


def test_status_strings():
    for s in range(5):
        assert ksa.ksa_status_string(s).startswith("KSA_")
    assert "unknown" in ksa.ksa_status_string(99)


def P(B=2, Hq=4, Hkv=2, D=64, T=1024, Tcap=1024, Bs=16, dtype=ksa.KSA_F32, scale=0.0):
    return ksa.Problem(B, Hq, Hkv, D, T, Tcap, Bs, dtype, scale)


def test_workspace_sizing_is_pure_and_validates():
    lib = ksa.load_library()
    p = P()
    a = ksa.ksa_workspace_bytes(p, ksa.KSA_OP_DENSE, 0)
    assert a == ksa.ksa_workspace_bytes(p, ksa.KSA_OP_DENSE, 0)
    # selection keeps one uint32 key per block
    assert ksa.ksa_workspace_bytes(p, ksa.KSA_OP_SELECT_TOPK, 8) == 2 * 2 * 64 * 4
    # the vote workspace holds fp32-sized keys for every (b, h, history token) plus bitmasks
    p4 = P(B=16, Hq=32, Hkv=8, D=128, T=20000, Tcap=20000, dtype=ksa.KSA_BF16)
    assert ksa.ksa_workspace_bytes(p4, ksa.KSA_OP_VOTE_SELECT, 2048) >= 16 * 32 * 20000 * 4
    # T <= N needs no workspace
    assert ksa.ksa_workspace_bytes(P(T=100, Tcap=100), ksa.KSA_OP_VOTE_SELECT, 2048) == 0
    bad = [P(Hq=3, Hkv=2), P(T=0), P(Tcap=10, T=20), P(Bs=0), P(B=0), P(B=16385, Hq=1, Hkv=1)]
    for b in bad:
        n = lib.ksa_workspace_bytes(ctypes.byref(b), ksa.KSA_OP_SPARSE_BLOCKS, 4)
        assert n == ksa.SIZE_MAX
    assert lib.ksa_workspace_bytes(ctypes.byref(p), 17, 1) == ksa.SIZE_MAX
    assert lib.ksa_workspace_bytes(None, ksa.KSA_OP_DENSE, 0) == ksa.SIZE_MAX


FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: validation fails first


def test_invalid_arguments_are_rejected_before_launch():
    lib = ksa.load_library()
    null = None
    p = P()
    E = ksa.KSA_ERR_INVALID_ARGUMENT
    U = ksa.KSA_ERR_UNSUPPORTED
    W = ksa.KSA_ERR_WORKSPACE_TOO_SMALL
    # summaries: block range outside [0, NB)
    assert lib.ksa_block_summaries(ctypes.byref(p), FAKE, FAKE, 60, 5, null) == E
    assert lib.ksa_block_summaries(ctypes.byref(p), FAKE, FAKE, -1, 1, null) == E
    assert lib.ksa_block_summaries(ctypes.byref(p), FAKE, FAKE, 0, 0, null) == E
    assert lib.ksa_block_summaries(ctypes.byref(p), null, FAKE, 0, 1, null) == E
    assert lib.ksa_block_summaries(ctypes.byref(p), ctypes.c_void_p(0x10002), FAKE, 0, 1, null) == E
    assert lib.ksa_block_summaries(None, FAKE, FAKE, 0, 1, null) == E
    # select: k <= 0, Hq not a multiple of Hkv, unsupported D / G
    assert lib.ksa_select_topk(ctypes.byref(p), FAKE, FAKE, 0, FAKE, null, null, 0, null) == E
    assert lib.ksa_select_topk(ctypes.byref(P(Hq=3)), FAKE, FAKE, 4, FAKE, null, null, 0, null) == E
    assert lib.ksa_select_topk(ctypes.byref(P(D=96)), FAKE, FAKE, 4, FAKE, null, null, 0, null) == U
    assert lib.ksa_select_topk(ctypes.byref(P(Hq=6, Hkv=2)), FAKE, FAKE, 4, FAKE, null, null, 0, null) == U
    assert lib.ksa_select_topk(ctypes.byref(P(T=20000, Tcap=20000, Bs=1)), FAKE, FAKE, 4, FAKE,
                               null, null, 0, null) == U
    # sparse: bad kind, count out of range, workspace too small
    sel = ksa.Selection(7, FAKE, 4)
    assert lib.ksa_sparse_decode(ctypes.byref(p), FAKE, FAKE, FAKE, ctypes.byref(sel), FAKE, null,
                                 null, 0, null) == E
    sel = ksa.Selection(ksa.KSA_SEL_BLOCKS, FAKE, 65)  # NB = 64
    assert lib.ksa_sparse_decode(ctypes.byref(p), FAKE, FAKE, FAKE, ctypes.byref(sel), FAKE, null,
                                 null, 0, null) == E
    sel = ksa.Selection(ksa.KSA_SEL_TOKENS, FAKE, 0)
    assert lib.ksa_sparse_decode(ctypes.byref(p), FAKE, FAKE, FAKE, ctypes.byref(sel), FAKE, null,
                                 null, 0, null) == E
    big = P(B=1, Hq=8, Hkv=1, D=128, T=65536, Tcap=65536, dtype=ksa.KSA_BF16)
    need = ksa.ksa_workspace_bytes(big, ksa.KSA_OP_DENSE, 0)
    assert need > 0
    assert lib.ksa_dense_decode(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, null, FAKE, need - 1,
                                null) == W
    # vote: W > N, N < 1, too many heads
    p4 = P(B=1, Hq=4, Hkv=2, D=64, T=100, Tcap=100)
    assert lib.ksa_vote_select(ctypes.byref(p4), FAKE, FAKE, 10, 11, FAKE, null, null, 0, null) == E
    assert lib.ksa_vote_select(ctypes.byref(p4), FAKE, FAKE, 0, 0, FAKE, null, null, 0, null) == E
    assert lib.ksa_vote_select(ctypes.byref(p4), FAKE, FAKE, 10, -1, FAKE, null, null, 0, null) == E
    p5 = P(B=1, Hq=256, Hkv=256, D=64, T=100, Tcap=100)
    assert lib.ksa_vote_select(ctypes.byref(p5), FAKE, FAKE, 10, 2, FAKE, null, null, 0, null) == U
    need = ksa.ksa_workspace_bytes(p4, ksa.KSA_OP_VOTE_SELECT, 10)
    assert lib.ksa_vote_select(ctypes.byref(p4), FAKE, FAKE, 10, 2, FAKE, null, FAKE, need - 1,
                               null) == W


def test_fused_step_validation():
    lib = ksa.load_library()
    null = None
    E = ksa.KSA_ERR_INVALID_ARGUMENT
    U = ksa.KSA_ERR_UNSUPPORTED

    def call(p, top_k=4, refresh=1, q=FAKE, summ=FAKE, out=FAKE, idx=null, lse=null):
        return lib.ksa_block_topk_decode(ctypes.byref(p) if p is not None else None, q, FAKE, FAKE,
                                         summ, top_k, refresh, idx, out, lse, null)

    p = P()
    assert call(None) == E
    assert call(p, top_k=0) == E
    assert call(p, q=null) == E
    assert call(p, summ=null) == E
    assert call(p, out=null) == E
    assert call(p, summ=ctypes.c_void_p(0x10008)) == E   # summaries must be 16-byte aligned
    assert call(p, idx=ctypes.c_void_p(0x10002)) == E    # block_idx must be 4-byte aligned
    assert call(P(Bs=0)) == E
    assert call(P(D=96)) == U
    # more blocks than the step keeps in LDS (4096), or more selected ids than it stages (2048)
    assert call(P(T=4097 * 16, Tcap=4097 * 16)) == U
    assert call(P(T=4096 * 2, Tcap=4096 * 2, Bs=2), top_k=2049) == U
    # the newest block is refreshed only for Bs <= 64; without refresh any Bs is fine
    assert call(P(Bs=65), refresh=1) == U


def test_fused_step_varlen_validation():
    """ksa_block_topk_decode_varlen: a lengths pointer is required and 4-byte
    aligned; everything else is checked as for ksa_block_topk_decode."""
    lib = ksa.load_library()
    null = None
    E = ksa.KSA_ERR_INVALID_ARGUMENT
    U = ksa.KSA_ERR_UNSUPPORTED

    def call(p, lens=FAKE, top_k=4, refresh=1, q=FAKE, out=FAKE):
        return lib.ksa_block_topk_decode_varlen(ctypes.byref(p) if p is not None else None, lens,
                                                q, FAKE, FAKE, FAKE, top_k, refresh, null, out,
                                                null, null)

    p = P()
    assert call(None) == E
    assert call(p, lens=null) == E
    assert call(p, lens=ctypes.c_void_p(0x10002)) == E   # seq_lens must be 4-byte aligned
    assert call(p, top_k=0) == E
    assert call(p, q=null) == E
    assert call(p, out=null) == E
    assert call(P(D=96)) == U
    assert call(P(T=4097 * 16, Tcap=4097 * 16)) == U
    assert call(P(Bs=65), refresh=1) == U


def test_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 2, 64)
    k = torch.zeros(1, 1, 16, 64)
    with pytest.raises(ValueError):
        ksa.ksa_dense_decode(q, k, k, 16)


def test_paged_validation():
    """The paged calls check the cache description on the host: table and
    lengths present and aligned, max_seq_len == max_blocks * Bs, a pool whose
    rows fit int32 offsets; the step keeps the fused step's limits."""
    lib = ksa.load_library()
    null = None
    E = ksa.KSA_ERR_INVALID_ARGUMENT
    U = ksa.KSA_ERR_UNSUPPORTED
    FA = ctypes.c_void_p(0x10000)

    def pg(max_blocks=64, num_pages=200, table=FA, lens=FA):
        return ksa.PagedKv(table, lens, max_blocks, num_pages)

    def step(p, g, top_k=4, refresh=1):
        return lib.ksa_paged_block_topk_decode(ctypes.byref(p), ctypes.byref(g) if g else None,
                                               FAKE, FAKE, FAKE, FAKE, top_k, refresh, null,
                                               FAKE, null, null)

    def summ(p, g, first=0, num=1):
        return lib.ksa_paged_block_summaries(ctypes.byref(p), ctypes.byref(g), FAKE, FAKE, first,
                                             num, null)

    def dense(p, g, nws=0):
        return lib.ksa_paged_dense_decode(ctypes.byref(p), ctypes.byref(g), FAKE, FAKE, FAKE, FAKE,
                                          null, null, nws, null)

    p = P()  # Tcap 1024 = 64 blocks of 16
    assert step(p, None) == E
    assert step(p, pg(table=null)) == E
    assert step(p, pg(lens=ctypes.c_void_p(0x10002))) == E
    assert step(p, pg(max_blocks=63)) == E              # max_seq_len must be max_blocks * Bs
    assert step(p, pg(num_pages=0)) == E
    assert step(p, pg(), top_k=0) == E
    assert step(P(Bs=65, T=65 * 64, Tcap=65 * 64), pg()) == U          # refresh needs Bs <= 64
    assert step(P(T=4097 * 16, Tcap=4097 * 16), pg(max_blocks=4097)) == U
    assert step(P(Hkv=2), pg(num_pages=1 << 26)) == U   # pool rows beyond int32
    assert summ(p, pg(), first=-1, num=2) == E           # -1 selects the newest block only
    assert summ(p, pg(), first=60, num=5) == E
    assert summ(p, pg(), first=-2) == E
    # paged dense needs a workspace when it splits rows
    need = ksa.ksa_workspace_bytes(P(B=1, Hkv=1, Hq=1, T=1 << 15, Tcap=1 << 15),
                                   ksa.KSA_OP_PAGED_DENSE, 0)
    assert need > 0
    assert dense(P(B=1, Hkv=1, Hq=1, T=1 << 15, Tcap=1 << 15), pg(max_blocks=2048)) == \
        ksa.KSA_ERR_WORKSPACE_TOO_SMALL


def test_variant_and_layer_validation():
    """Host-side checks of the variant, selection-layer and paged-vote calls."""
    lib = ksa.load_library()
    null = None
    E = ksa.KSA_ERR_INVALID_ARGUMENT
    U = ksa.KSA_ERR_UNSUPPORTED
    W_ = ksa.KSA_ERR_WORKSPACE_TOO_SMALL
    p = P(B=2, Hq=8, Hkv=2, D=128, T=4096, Tcap=4096, dtype=ksa.KSA_BF16)
    pp = ctypes.byref(p)
    # select options: bad aggregate, no options, k < 1
    bad = ksa.SelectOptions(4, 7, 0)
    assert lib.ksa_select_topk_ex(pp, FAKE, FAKE, ctypes.byref(bad), FAKE, null, FAKE, 1 << 30,
                                  null) == E
    assert lib.ksa_select_topk_ex(pp, FAKE, FAKE, null, FAKE, null, FAKE, 1 << 30, null) == E
    zero = ksa.SelectOptions(0, 0, 0)
    assert lib.ksa_select_topk_ex(pp, FAKE, FAKE, ctypes.byref(zero), FAKE, null, FAKE, 1 << 30,
                                  null) == E
    # voting heads: empty, out of range, repeated
    for heads in ([], [8], [-1], [2, 2]):
        arr = (ctypes.c_int32 * max(1, len(heads)))(*(heads or [0]))
        st = lib.ksa_vote_select_heads(pp, FAKE, FAKE, 512, 128, ctypes.cast(arr, ctypes.c_void_p),
                                       len(heads), FAKE, null, FAKE, 1 << 30, null)
        assert st == E, heads
    # selection layer: W > N, and a workspace smaller than asked
    assert lib.ksa_vote_layer_decode(pp, FAKE, FAKE, FAKE, 100, 200, FAKE, null, FAKE, null, FAKE,
                                     1 << 30, null) == E
    need = ksa.ksa_workspace_bytes(p, ksa.KSA_OP_VOTE_LAYER, 512)
    assert need > ksa.ksa_workspace_bytes(p, ksa.KSA_OP_VOTE_SELECT, 512)
    assert lib.ksa_vote_layer_decode(pp, FAKE, FAKE, FAKE, 512, 128, FAKE, null, FAKE, null, FAKE,
                                     0, null) == W_
    # paged vote: histories longer than the one-kernel vote set are supported,
    # so only the workspace check stops this call
    pl = P(B=1, Hq=8, Hkv=2, D=128, T=40000, Tcap=40000, dtype=ksa.KSA_BF16)
    g = ksa.PagedKv(FAKE, FAKE, 2500, 3000)
    assert lib.ksa_paged_vote_select(ctypes.byref(pl), ctypes.byref(g), FAKE, FAKE, 512, 128, FAKE,
                                     null, FAKE, 0, null) == W_
    # paged selection layer: W > N, no paged description, a workspace smaller
    # than asked (the asked size covers the vote and the paged dense partials)
    pgv = ctypes.byref(pl)
    assert lib.ksa_paged_vote_layer_decode(pgv, ctypes.byref(g), FAKE, FAKE, FAKE, 100, 200, FAKE,
                                           null, FAKE, null, FAKE, 1 << 34, null) == E
    assert lib.ksa_paged_vote_layer_decode(pgv, null, FAKE, FAKE, FAKE, 512, 128, FAKE, null, FAKE,
                                           null, FAKE, 1 << 34, null) == E
    lneed = ksa.ksa_workspace_bytes(pl, ksa.KSA_OP_PAGED_VOTE_LAYER, 512)
    assert lneed >= ksa.ksa_workspace_bytes(pl, ksa.KSA_OP_VOTE_SELECT, 512)
    assert lib.ksa_paged_vote_layer_decode(pgv, ctypes.byref(g), FAKE, FAKE, FAKE, 512, 128, FAKE,
                                           null, FAKE, null, FAKE, 0, null) == W_
    # paged voting heads: empty, out of range, repeated
    for heads in ([], [8], [-1], [2, 2]):
        arr = (ctypes.c_int32 * max(1, len(heads)))(*(heads or [0]))
        st = lib.ksa_paged_vote_select_heads(pgv, ctypes.byref(g), FAKE, FAKE, 512, 128,
                                             ctypes.cast(arr, ctypes.c_void_p), len(heads), FAKE,
                                             null, FAKE, 1 << 34, null)
        assert st == E, heads
    # paged selection variants: no options, a bad aggregate, k < 1
    assert lib.ksa_paged_select_topk_ex(pgv, ctypes.byref(g), FAKE, FAKE, null, FAKE, null, FAKE,
                                        1 << 34, null) == E
    assert lib.ksa_paged_select_topk_ex(pgv, ctypes.byref(g), FAKE, FAKE, ctypes.byref(bad), FAKE,
                                        null, FAKE, 1 << 34, null) == E
    assert lib.ksa_paged_select_topk_ex(pgv, ctypes.byref(g), FAKE, FAKE, ctypes.byref(zero), FAKE,
                                        null, FAKE, 1 << 34, null) == E
    # more query heads than a uint8 vote total counts
    ph = P(B=1, Hq=256, Hkv=32, D=128, T=4000, Tcap=40000, dtype=ksa.KSA_BF16)
    assert lib.ksa_paged_vote_select(ctypes.byref(ph), ctypes.byref(g), FAKE, FAKE, 512, 128, FAKE,
                                     null, FAKE, 1 << 34, null) == U
    # paged sparse decode: an unknown selection kind; more blocks than the table holds
    sel = ksa.Selection(7, FAKE.value, 4)
    g2 = ksa.PagedKv(FAKE, FAKE, 256, 1000)
    assert lib.ksa_paged_sparse_decode(pp, ctypes.byref(g2), FAKE, FAKE, FAKE, ctypes.byref(sel),
                                       FAKE, null, FAKE, 1 << 30, null) == E
    sel = ksa.Selection(ksa.KSA_SEL_BLOCKS, FAKE.value, 257)
    assert lib.ksa_paged_sparse_decode(pp, ctypes.byref(g2), FAKE, FAKE, FAKE, ctypes.byref(sel),
                                       FAKE, null, FAKE, 1 << 30, null) == E
    # recall: count < 1
    assert lib.ksa_attention_recall(FAKE, FAKE, FAKE, 0, null) == E


def test_paged_vote_history_limit():
    """ksa_paged_vote_select keeps the vote's history limit (T - W <= 2^21)
    like every other vote entry point: a longer history is unsupported and
    nothing is launched."""
    lib = ksa.load_library()
    U = ksa.KSA_ERR_UNSUPPORTED
    FA = ctypes.c_void_p(0x10000)
    T = (1 << 21) + 2048
    p = P(B=1, Hq=4, Hkv=1, D=128, T=T, Tcap=T, Bs=16, dtype=ksa.KSA_BF16)
    g = ksa.PagedKv(FA, FA, T // 16, T // 16)

    def vote(N, W):
        return lib.ksa_paged_vote_select(ctypes.byref(p), ctypes.byref(g), FAKE, FAKE, N, W, FAKE,
                                         None, FAKE, 1 << 40, None)

    assert vote(1024, 0) == U
    assert vote(4096, 2047) == U          # T - W = 2^21 + 1
    assert lib.ksa_vote_select(ctypes.byref(p), FAKE, FAKE, 1024, 0, FAKE, None, FAKE, 1 << 40,
                               None) == U


def test_workspace_sizing_ignores_the_environment(monkeypatch):
    """Workspace sizes (and the launch plans behind them) are a function of
    the arguments alone: no environment variable changes them."""
    shapes = [P(B=16, Hq=32, Hkv=8, D=128, T=20000, Tcap=20000, Bs=1, dtype=ksa.KSA_BF16),
              P(B=1, Hkv=1, Hq=1, T=1 << 15, Tcap=1 << 15), P()]
    ops = [(ksa.KSA_OP_SPARSE_TOKENS, 2048), (ksa.KSA_OP_DENSE, 0), (ksa.KSA_OP_SPARSE_BLOCKS, 8)]
    before = [ksa.ksa_workspace_bytes(p, op, prm) for p in shapes for op, prm in ops]
    monkeypatch.setenv("KSA_ATTN_PLAN", "1,32")
    after = [ksa.ksa_workspace_bytes(p, op, prm) for p in shapes for op, prm in ops]
    assert before == after


def test_noalloc_scratch_size_and_limit():
    """The binding's copy of KSA_NOALLOC_SCRATCH_BYTES is the header's; every
    call whose rows are split only to fill the chip (fewer than 256 rows,
    lists of at most 2048 entries) fits in it; a call needing more is
    refused with KSA_ERR_UNSUPPORTED on the host, before any device call."""
    lib = ksa.load_library()
    text = open(HEADER).read()
    m = re.search(r"#define KSA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == ksa.NOALLOC_SCRATCH_BYTES
    worst = 0
    for rows in (1, 2, 3, 5, 16, 100, 128, 255):
        for G in (1, 2, 4, 8):
            p = P(B=rows, Hq=G, Hkv=1, D=128, T=1 << 15, Tcap=1 << 15, Bs=16, dtype=ksa.KSA_BF16)
            for op, prm in ((ksa.KSA_OP_SPARSE_TOKENS, 2048), (ksa.KSA_OP_SPARSE_BLOCKS, 128)):
                worst = max(worst, ksa.ksa_workspace_bytes(p, op, prm))
    assert 0 < worst <= ksa.NOALLOC_SCRATCH_BYTES
    # 255 rows of 8 heads over a 32768-token list: 16 splits a row, 17 MB
    p = P(B=255, Hq=8, Hkv=1, D=128, T=1 << 15, Tcap=1 << 15, Bs=16, dtype=ksa.KSA_BF16)
    assert ksa.ksa_workspace_bytes(p, ksa.KSA_OP_SPARSE_TOKENS, 1 << 15) > ksa.NOALLOC_SCRATCH_BYTES
    sel = ksa.Selection(ksa.KSA_SEL_TOKENS, 0x10000, 1 << 15)
    st = lib.ksa_sparse_decode_noalloc(ctypes.byref(p), FAKE, FAKE, FAKE, ctypes.byref(sel), FAKE,
                                       FAKE, None)
    assert st == ksa.KSA_ERR_UNSUPPORTED


def test_read_probe_is_separate_and_validates():
    """The measurement-only read probe lives in its own library: libksa.so
    does not export it, and it refuses bad launch arguments on the host
    (status 1, nothing launched)."""
    path = os.path.join(os.path.dirname(ksa.LIB_PATH), "libksa_probe.so")
    if not os.path.exists(path):
        pytest.skip("libksa_probe.so is not built")
    assert not hasattr(ctypes.CDLL(ksa.LIB_PATH), "ksa_probe_read")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.ksa_probe_read.argtypes = [P, P, ctypes.c_longlong, ctypes.c_int, P, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, P, P]
    fake = 1 << 20  # never dereferenced: every call below is refused first

    def call(**kw):
        a = dict(k=fake, v=fake, stride=16 * 256, cap=16, lists=fake, rpl=1, rows=4, ntok=64,
                 splits=1, waves=4, inflight=1, sink=fake)
        a.update(kw)
        return lib.ksa_probe_read(a["k"], a["v"], a["stride"], a["cap"], a["lists"], a["rpl"],
                                  a["rows"], a["ntok"], a["splits"], a["waves"], a["inflight"],
                                  a["sink"], None)

    assert call(k=None) == 1
    assert call(lists=None) == 1
    assert call(waves=9) == 1
    assert call(waves=0) == 1
    assert call(inflight=3) == 1
    assert call(stride=100) == 1                # not a multiple of 16
    assert call(stride=16 * 256, cap=17) == 1  # rows shorter than their capacity
    assert call(ntok=4096, splits=1) == 1      # a workgroup's slice must fit its LDS stage
    assert call(rows=0) == 1
