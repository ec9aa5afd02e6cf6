"""Resource use of the built kernels, read from the library's own gfx950 code
objects (no GPU needed).

The one-launch decode step runs 4-wave workgroups when the rows outnumber the
8-wave workgroups the chip holds (the Qwen3-32B-shaped c5 layer: 2048 rows);
its speed rests on two of them being resident per CU, so that one row's top-k
is covered by the other's streaming.  An LDS or register increase that drops
that to one costs about a third of the step (measured: 532 -> 704 us on the
paged c5 step), with every parity test still green, so it is checked here.
"""
import os
import re
import subprocess

import pytest

from sparse_attention_decode_ksa_amd import LIB_PATH

LLVM = "/opt/rocm/llvm/bin"
LDS_PER_CU = 160 * 1024       # gfx950
VGPRS_PER_SIMD_LANE = 512     # unified architected + accumulation registers, wave64
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _kernels(tmp_path):
    """{kernel symbol: {lds, vgprs, threads}} over every translation unit."""
    if not os.path.exists(LIB_PATH):
        pytest.skip("libksa.so is not built")
    for tool in ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf"):
        if not os.path.exists(os.path.join(LLVM, tool)):
            pytest.skip("%s not available" % tool)
    fat = tmp_path / "fatbin.bin"
    subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section=.hip_fatbin=%s" % fat,
                    LIB_PATH, str(tmp_path / "stripped.so")], check=True, capture_output=True)
    blob = fat.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), blob)] + [len(blob)]
    out = {}
    for n in range(len(starts) - 1):
        part, co = tmp_path / ("b%d.bin" % n), tmp_path / ("co%d.o" % n)
        part.write_bytes(blob[starts[n]:starts[n + 1]])
        subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o",
                        "--input=%s" % part, "--targets=hipv4-amdgcn-amd-amdhsa--gfx950",
                        "--output=%s" % co], check=True, capture_output=True)
        notes = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", str(co)],
                               check=True, capture_output=True, text=True).stdout
        # one map per kernel, keys in sorted order, each map opening at .agpr_count
        for block in re.split(r"\n\s+- \.agpr_count:", notes)[1:]:
            name = re.search(r"\.name:\s+(\S+)", block)
            lds = re.search(r"\.group_segment_fixed_size:\s+(\d+)", block)
            vgpr = re.search(r"\.vgpr_count:\s+(\d+)", block)
            thr = re.search(r"\.max_flat_workgroup_size:\s+(\d+)", block)
            if name and lds and vgpr and thr:
                out[name.group(1)] = {"lds": int(lds.group(1)), "vgprs": int(vgpr.group(1)),
                                      "threads": int(thr.group(1))}
    return out


def _resident_per_cu(k):
    waves = k["threads"] // 64
    per_simd = -(-waves // 4)
    by_vgpr = (VGPRS_PER_SIMD_LANE // max(k["vgprs"], 1)) // per_simd
    by_lds = LDS_PER_CU // max(k["lds"], 1)
    return min(by_vgpr, by_lds)


def test_four_wave_step_kernels_fit_two_per_cu(tmp_path):
    ks = _kernels(tmp_path)
    assert ks, "no kernel metadata found in the library"
    # block_topk_decode_kernel<T = uint16_t (bf16), D = 128, G, NW = 4, PAGED>
    pat = re.compile(r"block_topk_decode_kernelItLi128ELi(\d+)ELi4ELb(\d)E")
    seen = []
    for name, k in ks.items():
        m = pat.search(name)
        if not m or int(m.group(1)) not in (4, 8):
            continue
        seen.append((int(m.group(1)), int(m.group(2))))
        assert _resident_per_cu(k) >= 2, (
            "G=%s paged=%s: %d B LDS, %d VGPRs -> %d workgroups per CU"
            % (m.group(1), m.group(2), k["lds"], k["vgprs"], _resident_per_cu(k)))
    assert sorted(seen) == [(4, 0), (4, 1), (8, 0), (8, 1)], seen


def test_every_kernel_fits_the_cu(tmp_path):
    # a workgroup that asks for more LDS than a CU has would fail at launch
    for name, k in _kernels(tmp_path).items():
        assert k["lds"] <= LDS_PER_CU, (name, k)
        assert k["threads"] <= 1024, (name, k)
