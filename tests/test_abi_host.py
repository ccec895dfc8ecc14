"""Host-side checks of the C ABI (no GPU work): the library loads, exports
every entry point the header declares, and rejects bad arguments before
enqueuing anything."""
import ctypes
import os
import re

import pytest

from deep_learning_recommendation_amd import _lib as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dlrm.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dlrm_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(C.LIB_PATH):
        pytest.fail("libdlrm.so is not built (run __graft_entry__.build())")
    return C.lib()


def test_every_declared_symbol_is_exported_and_bound(lib):
    declared = _declared()
    assert len(declared) >= 12
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(C.EXPORTS) == declared


def test_version_and_strings(lib):
    assert C.dlrm_abi_version() == 5
    for code in (0, -1, -2, -3, -4):
        assert lib.dlrm_strerror(code)
    assert lib.dlrm_last_hip_error() == 0


NULL = ctypes.c_void_p(0)
FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: validation fails first


def test_embbag_argument_checks(lib):
    f = lib.dlrm_embbag_fwd
    assert f(NULL, 8, 16, FAKE, FAKE, 128, -1, FAKE, 8 * 16, 0, NULL) == C.DLRM_E_INVALID
    assert f(FAKE, 8, 6, FAKE, FAKE, 128, -1, FAKE, 8 * 6, 0, NULL) == C.DLRM_E_INVALID     # d % 4
    assert f(FAKE, 8, 2048, FAKE, FAKE, 128, -1, FAKE, 8 * 2048, 0, NULL) == C.DLRM_E_INVALID  # d > 1024
    assert f(FAKE, 8, 16, FAKE, FAKE, 128, -1, FAKE, 8 * 16 - 4, 0, NULL) == C.DLRM_E_INVALID  # out_ld too small
    assert f(FAKE, 0, 16, FAKE, FAKE, 128, -1, FAKE, 16, 0, NULL) == C.DLRM_E_INVALID
    assert f(FAKE, 8, 16, FAKE, FAKE, 128, -1, ctypes.c_void_p(0x10004), 128, 0, NULL) == C.DLRM_E_INVALID  # alignment


def test_interact_argument_checks(lib):
    f = lib.dlrm_interact_fwd
    assert f(FAKE, 4, 1, 16, 16, FAKE, C.DLRM_F32, 64, NULL) == C.DLRM_E_INVALID       # n < 2
    assert f(FAKE, 4, 9, 16, 9 * 16, FAKE, C.DLRM_F32, 51, NULL) == C.DLRM_E_INVALID   # out_ld < 52
    assert f(FAKE, 4, 9, 16, 9 * 16, FAKE, 7, 52, NULL) == C.DLRM_E_INVALID            # dtype
    assert f(FAKE, 4, 129, 16, 129 * 16, FAKE, C.DLRM_F32, 9000, NULL) == C.DLRM_E_INVALID


def test_interact_bwd_argument_checks(lib):
    P = ctypes.c_void_p
    x, g, dx = P(16), P(16), P(16)  # never dereferenced: every case fails before a launch
    bad = [
        (None, 4, 9, 16, 144, g, 52, dx, 144),      # null X
        (x, 4, 1, 16, 16, g, 16, dx, 16),           # n < 2
        (x, 4, 9, 18, 162, g, 54, dx, 162),         # d % 4
        (x, 4, 9, 16, 140, g, 52, dx, 144),         # x_ld < n*d
        (x, 4, 9, 16, 144, g, 51, dx, 144),         # g_ld < d + n(n-1)/2
        (x, 4, 9, 16, 144, g, 52, dx, 143),         # dx_ld < n*d
    ]
    for args in bad:
        assert lib.dlrm_interact_bwd(*args, None) == -1, args
    # n = 128 with d = 256 does not fit one workgroup's LDS
    assert lib.dlrm_interact_bwd(x, 1, 128, 256, 128 * 256, g, 256 + 128 * 127 // 2, dx, 128 * 256, None) == -4


def test_mlp_workspace_and_checks(lib):
    dims = (ctypes.c_int32 * 4)(13, 512, 256, 128)
    a = lib.dlrm_mlp_workspace_size(32768, 3, dims, C.DLRM_BF16, 0)
    b = lib.dlrm_mlp_workspace_size(32768, 3, dims, C.DLRM_BF16, 1)
    assert a > 0 and b > 0 and a % 256 == 0 and b % 256 == 0
    # bf16 net: layer 0's input (16 padded) plus two ping-pong hidden buffers,
    # or every hidden layer's input when saving for the backward pass
    assert a >= 32768 * (16 + 2 * 512) * 2
    assert b >= 32768 * (16 + 512 + 256) * 2
    assert lib.dlrm_mlp_bwd_workspace_size(8192, 3, dims) > 0
    bad = (ctypes.c_int32 * 4)(13, 0, 256, 128)
    assert lib.dlrm_mlp_workspace_size(32768, 3, bad, C.DLRM_BF16, 0) == 0
    Ws = (ctypes.c_void_p * 3)(FAKE.value, FAKE.value, FAKE.value)
    bs = (ctypes.c_void_p * 3)(FAKE.value, FAKE.value, FAKE.value)
    # workspace too small
    rc = lib.dlrm_mlp_fwd(FAKE, C.DLRM_F32, 13, 32768, 3, dims, Ws, None, bs, C.DLRM_BF16, C.DLRM_ACT_RELU, FAKE, 128,
                          NULL, ctypes.c_void_p(0x100000), 256, 0, NULL)
    assert rc == C.DLRM_E_WORKSPACE
    # fp32 weights need fp32 input
    rc = lib.dlrm_mlp_fwd(FAKE, C.DLRM_BF16, 13, 32768, 3, dims, Ws, None, bs, C.DLRM_F32, C.DLRM_ACT_RELU, FAKE, 128,
                          NULL, ctypes.c_void_p(0x100000), 1 << 30, 0, NULL)
    assert rc == C.DLRM_E_INVALID
    # prob requires a single output column
    rc = lib.dlrm_mlp_fwd(FAKE, C.DLRM_F32, 13, 32768, 3, dims, Ws, None, bs, C.DLRM_BF16, C.DLRM_ACT_RELU, FAKE, 128,
                          FAKE, ctypes.c_void_p(0x100000), 1 << 30, 0, NULL)
    assert rc == C.DLRM_E_INVALID


def test_sparse_checks(lib):
    rows = (ctypes.c_int64 * 8)(*([50_000_000] * 8))
    ws = lib.dlrm_embbag_bwd_sgd_workspace_size(8, 8192, 6553600, 128)
    assert ws >= 6553600 * 16
    f = lib.dlrm_embbag_bwd_sgd
    assert f(FAKE, 8, 128, rows, FAKE, FAKE, 8192, 6553600, FAKE, 9 * 128, 128, ctypes.c_float(0.01),
             ctypes.c_void_p(0x100000), 256, NULL) == C.DLRM_E_WORKSPACE
    big = (ctypes.c_int64 * 8)(*([1 << 31] * 8))  # 31 row bits + 3 table bits > 32
    assert f(FAKE, 8, 128, big, FAKE, FAKE, 8192, 100, FAKE, 9 * 128, 128, ctypes.c_float(0.01),
             ctypes.c_void_p(0x100000), 1 << 30, NULL) == C.DLRM_E_UNSUPPORTED
    assert f(FAKE, 8, 128, rows, FAKE, FAKE, 8192, 100, FAKE, 9 * 128 - 4, 128, ctypes.c_float(0.01),
             ctypes.c_void_p(0x100000), 1 << 30, NULL) == C.DLRM_E_INVALID


def test_sparse_prepare_apply_checks(lib):
    """The two-call form rejects what the one-call form rejects, before
    enqueueing any work."""
    rows = (ctypes.c_int64 * 8)(*([50_000_000] * 8))
    prep, apply = lib.dlrm_embbag_bwd_sgd_prepare, lib.dlrm_embbag_bwd_sgd_apply
    lr = ctypes.c_float(0.01)
    assert prep(8, rows, FAKE, FAKE, 8192, 6553600, ctypes.c_void_p(0x100000), 256, NULL) == C.DLRM_E_WORKSPACE
    assert prep(8, rows, NULL, FAKE, 8192, 100, ctypes.c_void_p(0x100000), 1 << 30, NULL) == C.DLRM_E_INVALID
    assert prep(8, rows, FAKE, FAKE, 8192, -1, ctypes.c_void_p(0x100000), 1 << 30, NULL) == C.DLRM_E_INVALID
    big = (ctypes.c_int64 * 8)(*([1 << 31] * 8))
    assert prep(8, big, FAKE, FAKE, 8192, 100, ctypes.c_void_p(0x100000), 1 << 30, NULL) == C.DLRM_E_UNSUPPORTED
    assert prep(8, rows, FAKE, FAKE, 8192, 0, None, 0, NULL) == C.DLRM_OK  # nothing to sort
    assert apply(FAKE, 8, 128, rows, 8192, 6553600, FAKE, 9 * 128, 128, lr, ctypes.c_void_p(0x100000), 256,
                 NULL, NULL) == C.DLRM_E_WORKSPACE
    assert apply(NULL, 8, 128, rows, 8192, 100, FAKE, 9 * 128, 128, lr, ctypes.c_void_p(0x100000), 1 << 30,
                 NULL, NULL) == C.DLRM_E_INVALID
    assert apply(FAKE, 8, 128, rows, 8192, 100, FAKE, 9 * 128 - 4, 128, lr, ctypes.c_void_p(0x100000), 1 << 30,
                 NULL, NULL) == C.DLRM_E_INVALID
    assert apply(FAKE, 8, 130, rows, 8192, 100, FAKE, 9 * 130, 130, lr, ctypes.c_void_p(0x100000), 1 << 30,
                 NULL, NULL) == C.DLRM_E_INVALID
    assert apply(FAKE, 8, 128, big, 8192, 100, FAKE, 9 * 128, 128, lr, ctypes.c_void_p(0x100000), 1 << 30,
                 NULL, NULL) == C.DLRM_E_UNSUPPORTED


def test_linear_argument_checks(lib):
    f = lib.dlrm_linear_fwd
    act = C.DLRM_ACT_RELU
    assert f(NULL, 64, FAKE, 64, NULL, FAKE, C.DLRM_BF16, 128, 100, 128, 64, act, NULL) == C.DLRM_E_INVALID
    assert f(FAKE, 63, FAKE, 64, NULL, FAKE, C.DLRM_BF16, 128, 100, 128, 64, act, NULL) == C.DLRM_E_INVALID  # lda < K
    assert f(FAKE, 64, FAKE, 64, NULL, FAKE, C.DLRM_BF16, 127, 100, 128, 64, act, NULL) == C.DLRM_E_INVALID  # ldc < N
    assert f(FAKE, 64, FAKE, 64, NULL, FAKE, 7, 128, 100, 128, 64, act, NULL) == C.DLRM_E_INVALID            # dtype
    assert f(FAKE, 64, FAKE, 64, NULL, FAKE, C.DLRM_BF16, 128, 100, 128, 64, 5, NULL) == C.DLRM_E_INVALID    # act
    assert f(FAKE, 64, FAKE, 64, NULL, FAKE, C.DLRM_BF16, 1, 100, 1, 64, act, NULL) == C.DLRM_E_INVALID      # N=1 bf16
    assert f(FAKE, 64, FAKE, 64, NULL, FAKE, C.DLRM_F32, 128, 0, 128, 64, act, NULL) == C.DLRM_E_INVALID     # M = 0


def test_library_creates_no_streams_or_events():
    """The library enqueues on the caller's stream only: no source creates a
    stream or an event, or synchronises the device."""
    import glob
    import re

    srcs = glob.glob(os.path.join(os.path.dirname(C.LIB_PATH), "csrc", "*"))
    assert srcs
    pat = re.compile(r"hip(StreamCreate\w*|EventCreate\w*|DeviceSynchronize|StreamSynchronize|Malloc\w*|Free)\s*\(")
    for p in srcs:
        with open(p) as f:
            text = f.read()
        assert not pat.search(text), (p, pat.search(text).group(0))
