"""The decode work split and the fused kernel's row list, replayed on the host (CPU only).

``tests/native/decode_plan_driver.cpp`` compiles the library's own plan
(``spa_plan.h``) with g++ and replays, for every channel split of the fused
decode kernel and every pass of its threads, where each kept row is listed in
the workgroup's LDS list: every slot the stream reads must have been written
exactly once, and none may lie past the list's capacity.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
F32, F16, BF16 = 0, 1, 2


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("plan") / "decode_plan_driver")
    subprocess.run([cxx, "-O2", "-std=c++17", "-Wall", "-I", os.path.join(ROOT, "activation_sparsification_amd", "csrc"),
                    os.path.join(HERE, "native", "decode_plan_driver.cpp"), "-o", exe], check=True)
    return exe


def _replay(exe, cases, rule=1):
    inp = "\n".join(" ".join(str(v) for v in (*c, rule)) for c in cases) + "\n"
    out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout.splitlines()
    assert len(out) == len(cases)
    return [line.split() for line in out]


# (t, k, n_out, dtype, n, m, var): every fused-path shape of the GPU tests plus
# long channel ranges (several passes of the workgroup's threads per split),
# the largest k and the 2 GiB channel-major weight; several tokens stream the
# channel-major weight in float32 only (16-bit ones take the matrix cores)
CASES = [
    (1, 262144, 4096, BF16, 8, 16, 0),       # exactly 2^31 bytes of weight
    (1, 262080, 4096, BF16, 8, 16, 0),
    (1, 32768, 4096, F32, 8, 16, 0),
    (1, 32768, 2048, BF16, 2, 4, 0),
    (1, 65536, 776, F16, 16, 32, 1),
    (1, 1 << 24, 8, BF16, 1, 4, 0),
    (1, 1 << 24, 8, F32, 4, 4, 0),
    (1, 1024, 776, BF16, 8, 16, 0),
    (2, 262144, 1024, F32, 8, 16, 0),
    (3, 1 << 20, 136, F32, 16, 32, 1),
    (4, 1 << 20, 776, F32, 8, 16, 0),
    (2, 8192, 12288, F32, 8, 16, 0),
    (8, 65536, 64, F32, 2, 4, 1),
    (1, 4096, 14336, BF16, 8, 16, 0),        # one-token kernel (the decode layer)
    (8, 14336, 4096, F16, 16, 32, 1),        # matrix-core path (the batched layer)
    (2, 4096, 14336, BF16, 8, 16, 0),        # matrix-core path from two 16-bit tokens
]


def test_fused_lists_stay_inside_lds(driver):
    for case, res in zip(CASES, _replay(driver, CASES)):
        assert res[0] == "ok", (case, res)


def test_fused_lists_need_several_passes(driver):
    # the replay exercises the pass loop: at k = 2^18 one split lists 864
    # blocks with 512 threads, two passes
    res = _replay(driver, [CASES[0]])[0]
    assert res[:2] == ["ok", "fused"], res
    splits, cap, max_slot, entries = map(int, res[2:])
    assert (splits, cap) == (19, 6912) and max_slot == cap - 1 and entries == cap


def test_pass_offset_counted_twice_overruns_the_list(driver):
    # the earlier slot rule, base + (pass * threads + tid) * n, wrote the
    # second pass at slots 8192..11007 of a 6912-entry list and left
    # 4096..6911 unwritten: the stream then read row indices from LDS nobody
    # had written, and the weight loads went far outside the weight
    res = _replay(driver, [CASES[0]], rule=0)[0]
    assert res[0] == "fail" and res[1] in ("slot_past_cap", "slot_unwritten"), res


def test_decode_path_by_tokens_and_dtype(driver):
    # one wide 16-bit token: the one-token kernel; two or more 16-bit tokens:
    # the matrix cores; float32, and a narrow 16-bit token: the fused kernel
    cases = [(1, 4096, 14336, BF16, 8, 16, 0), (2, 4096, 14336, BF16, 8, 16, 0), (4, 512, 136, F16, 16, 32, 1),
             (2, 8192, 12288, F32, 8, 16, 0), (1, 1024, 776, BF16, 8, 16, 0)]
    assert [r[1] for r in _replay(driver, cases)] == ["t1", "mm", "mm", "fused", "fused"]
