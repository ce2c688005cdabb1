"""The C ABI on the CPU: the library loads, exports every function that
include/fa.h declares, and rejects invalid arguments before touching a GPU.

Only argument checks run here: each call below fails validation (or is an
empty problem), so nothing is launched and no GPU is needed.
"""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from io_aware_softmax_02_amd._lib import LIB
    return LIB


def test_header_declares_the_expected_calls():
    names = declared_functions()
    for n in ("fa_fwd", "fa_bwd", "fa_bwd_workspace_bytes", "fa_fwd_f32", "fa_bwd_f32",
              "fa_status_str", "fa_bwd_preprocess", "fa_bwd_dkdv", "fa_bwd_dq",
              "fa_fwd_split_max", "fa_fwd_split", "fa_merge"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    from io_aware_softmax_02_amd._lib import PROTOTYPES
    names = declared_functions()
    for n in names:
        assert hasattr(lib, n), n
        assert n in PROTOTYPES, f"{n} has no ctypes prototype"
    # and the exported dynamic symbols (nm -D) include them all
    so = os.path.join(ROOT, "io_aware_softmax_02_amd", "libfa_mi355x.so")
    out = subprocess.run(["nm", "-D", "--defined-only", so], capture_output=True, text=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for n in names:
        assert n in exported, n


def test_status_strings(lib):
    from io_aware_softmax_02_amd import _lib as L
    for code in range(0, 10):
        s = lib.fa_status_str(code).decode()
        assert s and "unknown" not in s
    assert "unknown" in lib.fa_status_str(99).decode()
    assert lib.fa_status_str(L.FA_ERR_ALIAS).decode().startswith("FA_ERR_ALIAS")


# Fake, well-aligned, distinct device addresses: validation only compares and
# aligns them; every call below returns before any launch.
A = 1 << 20
P = [A * (i + 1) for i in range(12)]


def fwd(lib, ptrs=None, B=1, H=1, N=64, d=128, scale=0.1, f32=False):
    q, k, v, o, lse = ptrs if ptrs is not None else P[:5]
    fn = lib.fa_fwd_f32 if f32 else lib.fa_fwd
    return fn(q, k, v, o, lse, B, H, N, d, scale, None)


def test_fwd_argument_checks(lib):
    from io_aware_softmax_02_amd import _lib as L
    assert fwd(lib, ptrs=[0, P[1], P[2], P[3], P[4]]) == L.FA_ERR_NULL
    assert fwd(lib, ptrs=[P[0], P[1], P[2], P[3], 0]) == L.FA_ERR_NULL
    assert fwd(lib, N=-1) == L.FA_ERR_SHAPE
    assert fwd(lib, B=-2) == L.FA_ERR_SHAPE
    assert fwd(lib, d=0) == L.FA_ERR_SHAPE
    assert fwd(lib, d=96) == L.FA_ERR_UNSUPPORTED
    assert fwd(lib, d=256) == L.FA_ERR_UNSUPPORTED
    assert fwd(lib, d=256, f32=True) == L.FA_ERR_UNSUPPORTED
    assert fwd(lib, scale=0.0) == L.FA_ERR_SCALE
    assert fwd(lib, scale=-1.0) == L.FA_ERR_SCALE
    assert fwd(lib, scale=float("nan")) == L.FA_ERR_SCALE
    assert fwd(lib, scale=float("inf")) == L.FA_ERR_SCALE
    assert fwd(lib, ptrs=[P[0] + 8, P[1], P[2], P[3], P[4]]) == L.FA_ERR_ALIGN
    assert fwd(lib, ptrs=[P[0], P[1], P[2], P[3], P[4] + 4]) == L.FA_ERR_ALIGN
    # fp32 path needs only 4-byte alignment; 2-byte offsets fail
    assert fwd(lib, ptrs=[P[0] + 2, P[1], P[2], P[3], P[4]], f32=True) == L.FA_ERR_ALIGN
    # aliasing: o overlapping q, lse inside o, o == k
    assert fwd(lib, ptrs=[P[0], P[1], P[2], P[0] + 64, P[4]]) == L.FA_ERR_ALIAS
    assert fwd(lib, ptrs=[P[0], P[1], P[2], P[3], P[3] + 256]) == L.FA_ERR_ALIAS
    assert fwd(lib, ptrs=[P[0], P[1], P[2], P[1], P[4]]) == L.FA_ERR_ALIAS
    # sizes whose element count overflows the accepted range
    assert fwd(lib, B=1 << 20, H=1 << 20, N=1 << 20) == L.FA_ERR_SHAPE
    assert fwd(lib, N=1 << 31) == L.FA_ERR_SHAPE


def test_split_and_merge_argument_checks(lib):
    from io_aware_softmax_02_amd import _lib as L

    def split(ptrs=None, n=2, N=1000, d=128, scale=0.1):
        q, k, v, op, lp = ptrs if ptrs is not None else P[:5]
        return lib.fa_fwd_split(q, k, v, op, lp, 1, 1, N, d, scale, n, None)

    def merge(ptrs=None, n=2, N=64, d=128):
        op, lp, o, lse = ptrs if ptrs is not None else P[:4]
        return lib.fa_merge(op, lp, n, o, lse, 1, 1, N, d, None)

    # key tiles are 128 keys at d = 128 and 64 at d = 64
    assert lib.fa_fwd_split_max(1, 1, 1000, 128) == 8
    assert lib.fa_fwd_split_max(1, 1, 1000, 64) == 16
    assert lib.fa_fwd_split_max(1, 1, 1, 128) == 1
    assert lib.fa_fwd_split_max(1, 1, 0, 128) == 0
    assert lib.fa_fwd_split_max(1, 1, 10, 96) == -1
    assert lib.fa_fwd_split_max(1, 1, -1, 128) == -1
    assert split(n=0) == L.FA_ERR_SHAPE
    assert split(n=-3) == L.FA_ERR_SHAPE
    assert split(n=9) == L.FA_ERR_SHAPE
    # the largest allowed count passes the count check and stops at the next
    # one (a NULL pointer), so nothing is launched on these fake addresses
    assert split(ptrs=[P[0], P[1], P[2], P[3], 0], n=16, d=64) == L.FA_ERR_NULL
    assert split(ptrs=[P[0], P[1], P[2], 0, P[4]]) == L.FA_ERR_NULL
    assert split(ptrs=[P[0], P[1], P[2], P[3] + 4, P[4]]) == L.FA_ERR_ALIGN
    assert split(d=96) == L.FA_ERR_UNSUPPORTED
    assert split(scale=0.0) == L.FA_ERR_SCALE
    # o_part (2 x 1000 x 128 x 4 B) reaching into lse_part, and o_part on q
    assert split(ptrs=[P[0], P[1], P[2], P[3], P[3] + 2 * 1000 * 128 * 4 - 16]) == L.FA_ERR_ALIAS
    assert split(ptrs=[P[0], P[1], P[2], P[0] + 16, P[4]]) == L.FA_ERR_ALIAS
    assert merge(n=0) == L.FA_ERR_SHAPE
    # counts beyond 2^24 are refused before anything else (the kernels count
    # parts in int32); the largest passes on to the pointer checks
    assert merge(n=(1 << 24) + 1, ptrs=[P[0], 0, P[2], P[3]]) == L.FA_ERR_SHAPE
    assert merge(n=(1 << 31) + 7, ptrs=[P[0], 0, P[2], P[3]]) == L.FA_ERR_SHAPE
    assert merge(n=1 << 24, ptrs=[P[0], 0, P[2], P[3]]) == L.FA_ERR_NULL
    assert merge(ptrs=[P[0], 0, P[2], P[3]]) == L.FA_ERR_NULL
    assert merge(ptrs=[P[0], P[1], P[2] + 8, P[3]]) == L.FA_ERR_ALIGN
    assert merge(d=32) == L.FA_ERR_UNSUPPORTED
    # output o overlapping the (2 x 64 x 128 x 4 B) o_part input
    assert merge(ptrs=[P[0], P[1], P[0] + 2 * 64 * 128 * 4 - 16, P[3]]) == L.FA_ERR_ALIAS
    # empty problems: nothing to do, pointers may be NULL
    assert lib.fa_fwd_split(0, 0, 0, 0, 0, 1, 1, 0, 128, 0.1, 1, None) == L.FA_OK
    assert lib.fa_merge(0, 0, 3, 0, 0, 0, 4, 64, 128, None) == L.FA_OK


# Fake addresses 1 TiB apart, for shapes whose tensors are large.
FAR = [(i + 1) << 40 for i in range(12)]


def test_single_head_grid_beyond_one_launch_is_refused(lib):
    """Grids are launched in chunks of whole heads of at most 2^31
    work-items; a head whose own grid exceeds that is FA_ERR_SHAPE, returned
    before any HIP call (the argument checks all pass for these shapes)."""
    from io_aware_softmax_02_amd import _lib as L
    # fp32 on key blocks of 8: 64 lanes per 8 query rows, ceil(N/8) * 64 > 2^31
    N = (1 << 28) + 1
    assert lib.fa_f32_key_block(N, 17) == 8
    assert fwd(lib, ptrs=FAR[:5], N=N, d=17, f32=True) == L.FA_ERR_SHAPE
    ws = lib.fa_bwd_f32_workspace_bytes(1, 1, N, 17)
    assert bwd(lib, ptrs=FAR[:9], ws=FAR[9], ws_bytes=ws, N=N, d=17, f32=True) == L.FA_ERR_SHAPE
    # split forward: 512 lanes per 256 query rows per key range; at N = 2^23
    # that is 2^15 * n_split * 512 lanes, beyond 2^31 from n_split = 129 on
    q, k, v, op, lp = FAR[:5]
    assert lib.fa_fwd_split_max(1, 1, 1 << 23, 64) == 1 << 17
    assert lib.fa_fwd_split(q, k, v, op, lp, 1, 1, 1 << 23, 64, 0.125, 129, None) == \
        L.FA_ERR_SHAPE


def test_empty_problems_are_noops(lib):
    from io_aware_softmax_02_amd import _lib as L
    for B, H, N in ((0, 1, 64), (1, 0, 64), (1, 1, 0)):
        assert fwd(lib, ptrs=[0, 0, 0, 0, 0], B=B, H=H, N=N) == L.FA_OK
        assert fwd(lib, ptrs=[0, 0, 0, 0, 0], B=B, H=H, N=N, d=5, f32=True) == L.FA_OK
        assert lib.fa_bwd(0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, B, H, N, 64, 0.1, None) == L.FA_OK
        assert lib.fa_bwd_workspace_bytes(B, H, N, 64) == 0
    # an empty problem still rejects a bad head dim or scale
    assert fwd(lib, ptrs=[0, 0, 0, 0, 0], N=0, d=96) == L.FA_ERR_UNSUPPORTED
    assert fwd(lib, ptrs=[0, 0, 0, 0, 0], N=0, scale=0.0) == L.FA_ERR_SCALE


def test_workspace_sizing(lib):
    assert lib.fa_bwd_workspace_bytes(1, 16, 8192, 128) == 16 * 8192 * 4
    assert lib.fa_bwd_workspace_bytes(1, 1, 7, 64) == 256      # rounded up to 256
    assert lib.fa_bwd_workspace_bytes(1, 1, 7, 96) == ctypes.c_size_t(-1).value
    assert lib.fa_bwd_f32_workspace_bytes(1, 1, 7, 5) == 256


def bwd(lib, ws=P[9], ws_bytes=1 << 16, ptrs=None, N=64, d=64, f32=False):
    q, k, v, o, lse, dO, dq, dk, dv = ptrs if ptrs is not None else P[:9]
    fn = lib.fa_bwd_f32 if f32 else lib.fa_bwd
    return fn(q, k, v, o, lse, dO, dq, dk, dv, ws, ws_bytes, 1, 1, N, d, 0.125, None)


def test_bwd_argument_checks(lib):
    from io_aware_softmax_02_amd import _lib as L
    assert bwd(lib, ws=0) == L.FA_ERR_NULL
    assert bwd(lib, ws_bytes=255) == L.FA_ERR_WORKSPACE
    assert bwd(lib, ws=P[9] + 4) == L.FA_ERR_ALIGN
    ptrs = list(P[:9])
    ptrs[6] = P[0]                 # dq == q
    assert bwd(lib, ptrs=ptrs) == L.FA_ERR_ALIAS
    ptrs = list(P[:9])
    ptrs[8] = P[7]                 # dv == dk
    assert bwd(lib, ptrs=ptrs) == L.FA_ERR_ALIAS
    assert bwd(lib, ws=P[6]) == L.FA_ERR_ALIAS     # workspace inside dq
    ptrs = list(P[:9])
    ptrs[5] = 0
    assert bwd(lib, ptrs=ptrs) == L.FA_ERR_NULL
    assert bwd(lib, d=32) == L.FA_ERR_UNSUPPORTED
    assert lib.fa_bwd_preprocess(P[0], 0, P[2], 1, 1, 64, 64, None) == L.FA_ERR_NULL
    assert lib.fa_bwd_dkdv(P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[6], 1, 1, 64, 64,
                           0.125, None) == L.FA_ERR_ALIAS
    assert lib.fa_bwd_dq(P[0], P[1], P[2], P[3], P[4], P[5], P[6], 1, 1, 64, 64,
                         float("nan"), None) == L.FA_ERR_SCALE


def test_python_short_names():
    import io_aware_softmax_02_amd as fa
    assert fa.forward is fa.fa_fwd and fa.backward is fa.fa_bwd
    assert issubclass(fa.FAError, RuntimeError)


def test_python_binding_rejects_cpu_tensors():
    import torch
    import io_aware_softmax_02_amd as fa
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        fa.fa_fwd(x, x, x)
    with pytest.raises(ValueError):
        fa.fa_fwd_f32(x.float(), x.float(), x.float()[:, :, :4])


def test_validation_header_under_sanitizers(tmp_path):
    """validate.h is plain C++: compile a driver with g++ and ASan/UBSan and
    run the overflow/alias/alignment edge cases."""
    src = tmp_path / "v.cpp"
    src.write_text(r'''
#include "validate.h"
#include <cstdio>
#include <limits>
using namespace fa;
int main() {
  int bad = 0;
  auto expect = [&](fa_status got, fa_status want, int line) {
    if (got != want) { std::printf("line %d: got %d want %d\n", line, got, want); ++bad; }
  };
  const int64_t big = std::numeric_limits<int64_t>::max();
  expect(check_shape({big, big, big, 64}, true), FA_ERR_SHAPE, __LINE__);
  expect(check_shape({1, 1, big, 64}, true), FA_ERR_SHAPE, __LINE__);
  expect(check_shape({2, 3, 5, 64}, true), FA_OK, __LINE__);
  expect(check_shape({2, 3, 5, 7}, false), FA_OK, __LINE__);
  expect(check_shape({2, 3, 5, 129}, false), FA_ERR_UNSUPPORTED, __LINE__);
  expect(check_shape({-1, 3, 5, 64}, true), FA_ERR_SHAPE, __LINE__);
  expect(check_shape({0, 3, 5, 64}, true), FA_OK, __LINE__);
  expect(check_scale(std::numeric_limits<float>::quiet_NaN()), FA_ERR_SCALE, __LINE__);
  expect(check_scale(1e-30f), FA_OK, __LINE__);
  int buf[64];
  expect(check_alias({{buf, 64}}, {{buf + 15, 64}}), FA_ERR_ALIAS, __LINE__);
  expect(check_alias({{buf, 64}}, {{buf + 16, 64}}), FA_OK, __LINE__);
  expect(check_alias({{buf, 64}}, {{buf + 16, 0}}), FA_OK, __LINE__);
  expect(check_alias({{buf, 16}}, {{buf + 4, 16}, {buf + 8, 16}}), FA_OK, __LINE__);
  expect(check_alias({{buf, 16}}, {{buf + 4, 16}, {buf + 6, 16}}), FA_ERR_ALIAS, __LINE__);
  expect(check_workspace(nullptr, 0, 0), FA_OK, __LINE__);
  expect(check_workspace(buf, 8, 16), FA_ERR_WORKSPACE, __LINE__);
  if (bwd_workspace_bytes({1, 1, 7, 64}, true) != 256) ++bad;
  if (bwd_workspace_bytes({1, 1, 7, 65}, true) != static_cast<size_t>(-1)) ++bad;
  return bad;
}
''')
    exe = tmp_path / "v"
    inc = os.path.join(ROOT, "io_aware_softmax_02_amd", "csrc")
    r = subprocess.run(["g++", "-std=c++17", "-g", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=all", "-I", inc, str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr


def test_f32_key_block(lib):
    # The 64-row example of the fable (8 stacks of 8) runs blocks of 8; long
    # sequences at d = 64 / 128 run the 32-key matrix-core tiles; other head
    # dims always blocks of 8; invalid arguments -1.
    assert lib.fa_f32_key_block(64, 64) == 8
    assert lib.fa_f32_key_block(256, 128) == 8
    assert lib.fa_f32_key_block(257, 128) == 32
    assert lib.fa_f32_key_block(4096, 64) == 32
    assert lib.fa_f32_key_block(4096, 17) == 8
    assert lib.fa_f32_key_block(0, 64) == 8
    assert lib.fa_f32_key_block(-1, 64) == -1
    assert lib.fa_f32_key_block(64, 0) == -1
    assert lib.fa_f32_key_block(64, 129) == -1


def test_bwd_noalloc_argument_checks(lib):
    from io_aware_softmax_02_amd import _lib as L

    def call(ptrs=None, B=1, H=1, N=64, d=64, scale=0.125):
        q, k, v, o, lse, dO, dq, dk, dv = ptrs if ptrs is not None else P[:9]
        return lib.fa_bwd_noalloc(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, None)

    # a problem beyond the fixed array is refused before anything else runs
    assert call(H=2, N=L.FA_BWD_NOALLOC_MAX_ROWS // 2 + 1, d=128) == L.FA_ERR_SCRATCH
    assert "FA_ERR_SCRATCH" in lib.fa_status_str(L.FA_ERR_SCRATCH).decode()
    ptrs = list(P[:9])
    ptrs[3] = 0
    assert call(ptrs=ptrs) == L.FA_ERR_NULL
    ptrs = list(P[:9])
    ptrs[7] = P[0]                 # dk == q
    assert call(ptrs=ptrs) == L.FA_ERR_ALIAS
    assert call(d=96) == L.FA_ERR_UNSUPPORTED
    assert call(scale=0.0) == L.FA_ERR_SCALE
    assert call(ptrs=[0] * 9, N=0) == L.FA_OK
