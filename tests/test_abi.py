"""Host-side checks of the C ABI (no GPU needed).

The library must load and export every function declared in include/fa.h.
Argument validation runs on the host before anything is launched, so the
error paths below never reach the HIP runtime: every call here returns a
status before a launch.
"""
import ctypes
import os
import re

import pytest

import exact_second_order_fa_amd as fa
from exact_second_order_fa_amd import FaProblem, FaTensor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        from exact_second_order_fa_amd import build

        build.build()
    return fa.load_library()


def declared_functions():
    src = open(os.path.join(ROOT, "include", "fa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_\w+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(fa.SYMBOLS)
    for name in names:
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    # 1.4.0: key/row split partials in fa_bob's workspace, 64 MiB no-alloc array
    # (1.3.0: fa_bob_noalloc; 1.2.0: dropout and seed; 1.1.0: H_kv)
    assert lib.fa_version() == 10400
    for code in range(8):
        s = lib.fa_status_str(code).decode()
        assert s and s != "unknown status"
    assert lib.fa_status_str(99).decode() == "unknown status"


def prob(B=1, H=2, N=100, d=64, scale=-1.0, causal=0, dt=fa.FA_BF16, Hkv=0, dropout=0.0, seed=0):
    return FaProblem(B, H, N, d, scale, causal, dt, Hkv, dropout, 0, seed)


def test_problem_struct_layout(tmp_path):
    """The ctypes mirror of fa_problem and fa_tensor matches include/fa.h as a C
    compiler lays it out."""
    import shutil
    import subprocess

    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "fa.h"\n'
                   'int main(void) { printf("%zu %zu %zu %zu %zu %zu %zu\\n", sizeof(fa_problem), '
                   'offsetof(fa_problem, scale), offsetof(fa_problem, in_dtype), offsetof(fa_problem, H_kv), '
                   'offsetof(fa_problem, dropout), offsetof(fa_problem, seed), '
                   'sizeof(fa_tensor)); return 0; }\n')
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), "-o", str(exe), str(src)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert got == [ctypes.sizeof(FaProblem), FaProblem.scale.offset, FaProblem.in_dtype.offset,
                   FaProblem.H_kv.offset, FaProblem.dropout.offset, FaProblem.seed.offset, ctypes.sizeof(FaTensor)]


def _align64(f):
    return (f + 63) // 64 * 64


def test_workspace_sizes(lib):
    p = prob(2, 3, 130, 64)
    # D, alpha, E ([B,H,N] fp32 each), then four chain inits per row padded to 128 rows
    assert lib.fa_bob_workspace_bytes(ctypes.byref(p)) == _align64(3 * 2 * 3 * 130 + 4 * 2 * 3 * 256) * 4
    # D ([B,H,N] fp32), then two chain inits per row padded to 128 rows
    assert lib.fa_bwd_workspace_bytes(ctypes.byref(p)) == _align64(2 * 3 * 130 + 2 * 2 * 3 * 256) * 4
    # Grouped-query attention with few key blocks splits each key block's
    # query heads over several workgroups, whose partial key-side sums
    # ([2][nsplit][B*H_kv][N][d] fp32) follow: 2 x 1 key/value heads x 2 key
    # blocks = 4 column workgroups, so the group of 3 is split 3 ways.
    assert lib.fa_bob_workspace_bytes(ctypes.byref(prob(2, 3, 130, 64, Hkv=1))) == \
        (_align64(3 * 2 * 3 * 130 + 4 * 2 * 3 * 256) + 2 * 3 * 2 * 1 * 130 * 64) * 4
    assert lib.fa_bwd_workspace_bytes(ctypes.byref(prob(2, 3, 130, 64, Hkv=1))) == \
        (_align64(2 * 3 * 130 + 2 * 2 * 3 * 256) + 2 * 3 * 2 * 1 * 130 * 64) * 4
    # Enough key blocks (B * H_kv * ceil(N/128) >= 256): no split, nothing extra.
    big = prob(1, 8, 32768, 64, Hkv=1)
    assert lib.fa_bob_workspace_bytes(ctypes.byref(big)) == _align64(3 * 8 * 32768 + 4 * 8 * 32768) * 4
    # The smallest divisor of G that reaches 256 workgroups: 1 x 1 x 64 key
    # blocks at N = 8192, G = 8 -> 4 splits.
    mid = prob(1, 8, 8192, 64, Hkv=1)
    assert lib.fa_bob_workspace_bytes(ctypes.byref(mid)) == \
        (_align64(3 * 8 * 8192 + 4 * 8 * 8192) + 2 * 4 * 8192 * 64) * 4
    # Still short of 256 after splitting the group (1 x 1 x 16 key blocks x
    # G = 8 at N = 2048), the non-causal column pass also cuts each query
    # head's rows into two ranges: 16 partials.  The row pass (8 heads x 16
    # row blocks = 128 workgroups) cuts each block's keys into two ranges,
    # whose raw sums follow on a 256-byte boundary: [2][3][B*H][N] row sums
    # and [2][4][B*H][N][d] accumulators.  Causal: the group split only.
    mqa2k = prob(1, 8, 2048, 64, Hkv=1)
    assert lib.fa_bob_workspace_bytes(ctypes.byref(mqa2k)) == \
        (_align64(_align64(3 * 8 * 2048 + 4 * 8 * 2048) + 2 * 16 * 2048 * 64) + 2 * 8 * 2048 * (3 + 4 * 64)) * 4
    assert lib.fa_bob_workspace_bytes(ctypes.byref(prob(1, 8, 2048, 64, Hkv=1, causal=1))) == \
        (_align64(3 * 8 * 2048 + 4 * 8 * 2048) + 2 * 8 * 2048 * 64) * 4
    # Multi-head with few blocks (4 heads x 32 blocks = 128): two row ranges
    # in the column pass, two key ranges in the row pass.  Ranges keep at
    # least two 128-row blocks, so N = 300 (3 blocks) is never cut.
    assert lib.fa_bob_workspace_bytes(ctypes.byref(prob(1, 4, 4096, 64))) == \
        (_align64(_align64(3 * 4 * 4096 + 4 * 4 * 4096) + 2 * 2 * 4 * 4096 * 64) + 2 * 4 * 4096 * (3 + 4 * 64)) * 4
    # Dropout keeps the row pass whole (its key split is not built).
    assert lib.fa_bob_workspace_bytes(ctypes.byref(prob(1, 4, 4096, 64, dropout=0.1))) == \
        (_align64(3 * 4 * 4096 + 4 * 4 * 4096) + 2 * 2 * 4 * 4096 * 64) * 4
    assert lib.fa_bob_workspace_bytes(ctypes.byref(prob(1, 1, 300, 64))) == \
        _align64(3 * 300 + 4 * 384) * 4
    # The first backward keeps the group split only.
    assert lib.fa_bwd_workspace_bytes(ctypes.byref(mqa2k)) == \
        (_align64(8 * 2048 + 2 * 8 * 2048) + 2 * 8 * 2048 * 64) * 4
    # fp32 inputs run the portable kernels, which never split.
    assert lib.fa_bob_workspace_bytes(ctypes.byref(prob(2, 3, 130, 64, Hkv=1, dt=fa.FA_FP32))) == \
        lib.fa_bob_workspace_bytes(ctypes.byref(prob(2, 3, 130, 64, dt=fa.FA_FP32)))
    assert lib.fa_bob_workspace_bytes(ctypes.byref(prob(d=96))) == 0
    assert lib.fa_bob_workspace_bytes(None) == 0


FAKE = 0x10000  # aligned, never dereferenced: validation fails before any launch


def t(ptr=FAKE, sb=2 * 100 * 64, sh=100 * 64, sn=64):
    return FaTensor(ptr, sb, sh, sn)


def bob(lib, p, tensors=None, lse=FAKE, ws=FAKE, ws_bytes=1 << 30):
    ts = tensors or [t() for _ in range(12)]
    return lib.fa_bob(p if p is None else ctypes.byref(p), ts[0], ts[1], ts[2], ts[3], lse, ts[4], ts[5],
                      ts[6], ts[7], ts[8], ts[9], ts[10], ts[11], ws, ws_bytes, None)


@pytest.mark.parametrize("p,status", [
    (None, 1),
    (prob(B=0), 2),
    (prob(N=0), 2),
    (prob(dt=7), 4),
    (prob(d=96), 5),
    (prob(d=32), 5),
    (prob(causal=2), 5),
    (prob(causal=-1), 5),
    (prob(d=128, dt=fa.FA_FP32), 5),
    (prob(scale=float("nan")), 5),
    (prob(scale=float("inf")), 5),
    (prob(N=(1 << 30) + 1), 2),
    (prob(H=2, Hkv=3), 2),   # more key/value heads than query heads
    (prob(H=4, Hkv=3), 2),   # not a divisor
    (prob(H=2, Hkv=-1), 2),
    (prob(dropout=-0.1), 5),
    (prob(dropout=1.0), 5),
    (prob(dropout=0.999), 5),  # rounds to 256/256: nothing kept
    (prob(dropout=float("nan")), 5),
])
def test_problem_validation(lib, p, status):
    assert bob(lib, p) == status


def test_tensor_validation(lib):
    p = prob()
    bad = [t() for _ in range(12)]
    bad[4] = t(ptr=0)
    assert bob(lib, p, bad) == 1  # null dout
    bad = [t() for _ in range(12)]
    bad[0] = t(ptr=FAKE + 8)
    assert bob(lib, p, bad) == 3  # misaligned
    bad = [t() for _ in range(12)]
    bad[1] = t(sn=32)
    assert bob(lib, p, bad) == 3  # row stride shorter than d
    bad = [t() for _ in range(12)]
    bad[2] = t(sn=68)
    assert bob(lib, p, bad) == 3  # row stride not a multiple of 16 bytes (bf16)
    bad = [t() for _ in range(12)]
    bad[3] = t(sn=66)  # o is fp32: 66 floats is not a multiple of 16 bytes
    assert bob(lib, p, bad) == 3
    assert bob(lib, p, lse=0) == 1
    assert bob(lib, p, lse=FAKE + 2) == 3


def test_workspace_validation(lib):
    p = prob()
    need = lib.fa_bob_workspace_bytes(ctypes.byref(p))
    assert bob(lib, p, ws=0) == 6
    assert bob(lib, p, ws_bytes=need - 4) == 6
    assert bob(lib, p, ws=FAKE + 4) == 6
    pb = prob()
    ts = [t() for _ in range(8)]
    assert lib.fa_bwd(ctypes.byref(pb), ts[0], ts[1], ts[2], ts[3], FAKE, ts[4], ts[5], ts[6], ts[7],
                      FAKE, lib.fa_bwd_workspace_bytes(ctypes.byref(pb)) - 1, None) == 6


def test_fwd_validation(lib):
    p = prob(d=80)
    assert lib.fa_fwd(ctypes.byref(p), t(), t(), t(), t(), FAKE, None) == 5
    p = prob()
    assert lib.fa_fwd(ctypes.byref(p), t(), t(), t(ptr=0), t(), FAKE, None) == 1
    assert lib.fa_fwd(ctypes.byref(p), t(), t(), t(), t(), 0, None) == 1


def test_binding_refuses_an_older_library(tmp_path):
    """A library from before fa_problem.H_kv would index key-side tensors with
    the query-head count; the binding refuses to load one (stub built with gcc,
    exporting the ABI's names; never called beyond fa_version)."""
    import shutil
    import subprocess

    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    names = [n for n in fa.SYMBOLS if n != "fa_version"]
    src = tmp_path / "old.c"
    src.write_text("int fa_version(void) { return 10000; }\n" + "".join(f"int {n}(void) {{ return 0; }}\n" for n in names))
    so = tmp_path / "libold.so"
    subprocess.run([cc, "-shared", "-fPIC", "-o", str(so), str(src)], check=True)
    with pytest.raises(fa.FaLibraryError):
        fa.load_library(str(so))


def sched(lib, p, schedule, phase, ts=None):
    ts = ts or [t() for _ in range(12)]
    return lib.fa_bob_schedule(ctypes.byref(p), ts[0], ts[1], ts[2], ts[3], FAKE, ts[4], ts[5], ts[6], ts[7],
                               ts[8], ts[9], ts[10], ts[11], FAKE, 1 << 30, schedule, phase, None)


@pytest.mark.parametrize("schedule,phase,dt", [
    (3, -1, fa.FA_BF16),      # unknown schedule
    (-1, -1, fa.FA_BF16),
    (2, -1, fa.FA_FP32),      # three-pass is bf16-only
    (2, 4, fa.FA_BF16),       # phase outside the three-pass schedule
    (0, 3, fa.FA_BF16),       # phase outside the two-pass schedule
    (1, -2, fa.FA_BF16),
])
def test_schedule_validation(lib, schedule, phase, dt):
    assert sched(lib, prob(dt=dt), schedule, phase) == 5


def test_three_pass_refuses_dropout(lib):
    assert sched(lib, prob(dropout=0.1), 2, -1) == 5
    # a rate that rounds to a zero threshold is no dropout
    assert sched(lib, prob(dropout=0.001), 2, -1, [t(ptr=0)] + [t() for _ in range(11)]) == 1


def test_schedule_checks_tensors_too(lib):
    bad = [t() for _ in range(12)]
    bad[0] = t(ptr=0)
    assert sched(lib, prob(), 2, -1, bad) == 1


def noalloc(lib, p, ts=None):
    ts = ts or [t() for _ in range(12)]
    return lib.fa_bob_noalloc(ctypes.byref(p), ts[0], ts[1], ts[2], ts[3], FAKE, ts[4], ts[5], ts[6], ts[7],
                              ts[8], ts[9], ts[10], ts[11], None)


def test_noalloc_validation(lib):
    """fa_bob_noalloc checks its arguments like fa_bob and refuses a problem
    whose workspace exceeds its static array, all before touching the GPU."""
    bad = [t() for _ in range(12)]
    bad[5] = t(ptr=0)
    assert noalloc(lib, prob(), bad) == 1
    assert noalloc(lib, prob(d=96)) == 5
    small = prob(B=1, H=4, N=65536)
    big = prob(B=1, H=16, N=262144)
    assert lib.fa_bob_workspace_bytes(ctypes.byref(small)) <= fa.NOALLOC_SCRATCH_BYTES
    assert lib.fa_bob_workspace_bytes(ctypes.byref(big)) > fa.NOALLOC_SCRATCH_BYTES
    assert noalloc(lib, big) == 6
    bad = [t() for _ in range(12)]
    bad[11] = t(ptr=0)
    assert noalloc(lib, big, bad) == 1  # argument errors come first


def test_noalloc_scratch_size_matches_header():
    src = open(os.path.join(ROOT, "include", "fa.h")).read()
    m = re.search(r"#define FA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == fa.NOALLOC_SCRATCH_BYTES
