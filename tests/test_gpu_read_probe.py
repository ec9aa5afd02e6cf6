"""The measurement-only read probe (libksa_probe.so) reads exactly the rows its
lists name: the XOR of every 32-bit word it loads (the XOR of its per-thread
folds) equals the XOR of the listed K and V rows computed on the host, for
per-row lists, lists shared by several rows, K alone, ragged list lengths and
every launch shape the benchmark uses.  The probe's rates bound the decode
kernels' bandwidth, so its addressing is checked like the kernels'."""
import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

PROBE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                     "sparse_attention_decode_ksa_amd", "libksa_probe.so")
ROW_B = 256


def _lib():
    assert os.path.exists(PROBE), "libksa_probe.so is not built: run __graft_entry__.build()"
    lib = ctypes.CDLL(PROBE)
    P = ctypes.c_void_p
    lib.ksa_probe_read.argtypes = [P, P, ctypes.c_longlong, ctypes.c_int, P, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, P, P]
    return lib


def _host_xor(buf, rows, cap, lists, rpl):
    words = buf.view(np.uint32).reshape(rows, cap, ROW_B // 4)
    acc = np.uint32(0)
    for r in range(rows):
        sel = words[r, lists[r // rpl]]
        acc ^= np.bitwise_xor.reduce(sel.reshape(-1))
    return int(acc)


# list lengths are whole chunks of 16, as every pattern the benchmark reads
# (a partial last chunk re-reads its last entry)
@pytest.mark.parametrize("rows,cap,ntok,rpl,two,shape", [
    (6, 96, 48, 1, True, (8, 1, 1)),      # a list per row, K and V
    (6, 96, 48, 3, True, (4, 2, 2)),      # lists shared by 3 rows, split rows
    (5, 80, 48, 1, False, (8, 1, 4)),     # K alone, fewer chunks than in flight
    (4, 64, 64, 4, True, (2, 3, 2)),      # one list for every row, an empty split
    (3, 4096, 2048, 1, True, (4, 1, 4)),  # a full 2048-entry stage, 4 chunks in flight
    (3, 4096, 2048, 1, False, (8, 1, 2)),
])
def test_probe_reads_exactly_the_listed_rows(rows, cap, ntok, rpl, two, shape):
    lib = _lib()
    waves, splits, inflight = shape
    rng = np.random.default_rng(rows * 1000 + ntok)
    kh = rng.integers(0, 2**32, size=rows * cap * ROW_B // 4, dtype=np.uint32)
    vh = rng.integers(0, 2**32, size=rows * cap * ROW_B // 4, dtype=np.uint32)
    nl = (rows + rpl - 1) // rpl
    lists = np.stack([np.sort(rng.choice(cap, size=ntok, replace=False)) for _ in range(nl)])
    lists = lists.astype(np.int32)
    dev = torch.device("cuda:0")
    k = torch.from_numpy(kh.view(np.int32)).to(dev)
    v = torch.from_numpy(vh.view(np.int32)).to(dev)
    lt = torch.from_numpy(lists).to(dev)
    sink = torch.zeros(rows * splits * waves * 64, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    st = lib.ksa_probe_read(k.data_ptr(), v.data_ptr() if two else None, cap * ROW_B, cap,
                            lt.data_ptr(), rpl, rows, ntok, splits, waves, inflight,
                            sink.data_ptr(), None)
    assert st == 0
    torch.cuda.synchronize()
    got = int(np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)))
    want = _host_xor(kh, rows, cap, lists, rpl)
    if two:
        want ^= _host_xor(vh, rows, cap, lists, rpl)
    assert got == want
