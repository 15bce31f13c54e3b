"""The C ABI library: it loads, exports every declared entry point, and rejects
bad arguments before touching the GPU (these calls never launch a kernel, so
they run without a GPU)."""
import ctypes
import os
import re

import pytest

from exact_io_aware_23_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")
PROBE_HEADER = os.path.join(ROOT, "include", "attn_probe.h")

FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: validation fails first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from exact_io_aware_23_amd.build import build

        build()
    return binding.load_library()


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_expected_entry_points():
    assert declared_functions() == sorted([
        "attn_fwd", "attn_bwd", "attn_bwd_workspace_bytes", "attn_bwd_preprocess", "attn_bwd_dkdv",
        "attn_bwd_dq", "attn_bwd_dq_fused", "attn_status_string", "attn_abi_version", "attn_fwd_block_sparse",
        "attn_bwd_block_sparse", "attn_fwd_dropout", "attn_bwd_dropout", "attn_decode_workspace_bytes",
        "attn_decode", "attn_fwd_fp8", "attn_bwd_noalloc", "attn_bwd_noalloc_max_rows"])


def test_probe_header_declares_the_probes():
    assert declared_functions(PROBE_HEADER) == sorted([
        "attn_probe_lds_rate", "attn_probe_issue", "attn_probe_wave_simd", "attn_probe_atomic", "attn_probe_exp2",
        "attn_probe_read_rate"])


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions() + declared_functions(PROBE_HEADER)
    for name in names:
        assert hasattr(lib, name), name
    # and as plain C symbols (no C++ mangling)
    out = os.popen(f"nm -D --defined-only {binding.LIB_PATH}").read()
    for name in names:
        assert re.search(rf"\bT {name}$", out, flags=re.M), name


def test_probe_validation(lib):
    """Probes refuse out-of-range arguments with 1 before launching anything."""
    assert lib.attn_probe_lds_rate(2, 4, FAKE, FAKE, None) == 1
    assert lib.attn_probe_lds_rate(0, 0, FAKE, FAKE, None) == 1
    assert lib.attn_probe_lds_rate(0, 4, None, FAKE, None) == 1
    assert lib.attn_probe_issue(FAKE, 9, 4, FAKE, FAKE, None) == 1
    assert lib.attn_probe_issue(FAKE, 4, 0, FAKE, FAKE, None) == 1
    assert lib.attn_probe_wave_simd(0, FAKE, None) == 1
    assert lib.attn_probe_atomic(FAKE, 100, 1, None) == 1  # not a multiple of 16384
    assert lib.attn_probe_atomic(None, 16384, 1, None) == 1
    assert lib.attn_probe_exp2(FAKE, FAKE, 0, None) == 1
    assert lib.attn_probe_read_rate(FAKE, 100, 4, 8, FAKE, None) == 1  # not a multiple of 16
    assert lib.attn_probe_read_rate(FAKE, 1 << 20, 3, 8, FAKE, None) == 1  # unroll not 1, 2, 4 or 8
    assert lib.attn_probe_read_rate(FAKE, 1 << 20, 4, 0, FAKE, None) == 1
    assert lib.attn_probe_read_rate(None, 1 << 20, 4, 8, FAKE, None) == 1


def test_abi_version_matches_header(lib):
    m = re.search(r"#define ATTN_ABI_VERSION (\d+)", open(HEADER).read())
    assert lib.attn_abi_version() == int(m.group(1))


def test_status_strings(lib):
    for s in range(5):
        assert lib.attn_status_string(s)
    assert lib.attn_status_string(99) == b"unknown status"


def test_workspace_bytes(lib):
    assert lib.attn_bwd_workspace_bytes(2, 32, 8192, 128) == 2 * 32 * 8192 * 4
    assert lib.attn_bwd_workspace_bytes(1, 1, 3, 64) == 256
    assert lib.attn_bwd_workspace_bytes(0, 1, 3, 64) == 0
    assert lib.attn_bwd_workspace_bytes(1, 1, -1, 64) == 0


def fwd(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, N=16, d=64, dtype=1, scale=0.125, causal=0):
    return lib.attn_fwd(q, k, v, o, lse, B, H, N, d, dtype, scale, causal, None)


def test_fwd_validation(lib):
    INV, UNS = binding.ATTN_ERR_INVALID, binding.ATTN_ERR_UNSUPPORTED
    for kw in ("q", "k", "v", "o", "lse"):
        assert fwd(lib, **{kw: None}) == INV
    assert fwd(lib, B=0) == INV
    assert fwd(lib, H=-1) == INV
    assert fwd(lib, N=0) == INV
    assert fwd(lib, B=1 << 16, H=1 << 16, N=1) == INV  # B*H*N >= 2^31
    # any finite scale is accepted (a negative or zero one is valid attention;
    # such calls would launch, so they are exercised by the GPU parity tests)
    assert fwd(lib, scale=float("nan")) == INV
    assert fwd(lib, scale=float("-inf")) == INV
    assert fwd(lib, scale=float("inf")) == INV
    assert fwd(lib, causal=2) == INV
    assert fwd(lib, d=96) == UNS
    assert fwd(lib, d=256) == UNS
    assert fwd(lib, dtype=7) == UNS
    assert fwd(lib, N=(1 << 22) + 1) == UNS  # one head is addressed with 32-bit byte offsets


def test_bwd_validation(lib):
    INV, UNS = binding.ATTN_ERR_INVALID, binding.ATTN_ERR_UNSUPPORTED
    ws = lib.attn_bwd_workspace_bytes(1, 2, 100, 64)

    def bwd(ptrs=None, ws_bytes=ws, B=1, H=2, N=100, d=64, dtype=1, scale=0.125, causal=1):
        p = ptrs or [FAKE] * 10
        return lib.attn_bwd(*p, ws_bytes, B, H, N, d, dtype, scale, causal, None)

    for i in range(10):
        p = [FAKE] * 10
        p[i] = None
        assert bwd(p) == INV, i
    assert bwd(ws_bytes=ws - 1) == INV
    assert bwd(N=0) == INV
    assert bwd(scale=float("nan")) == INV
    assert bwd(causal=-1) == INV
    assert bwd(d=32) == UNS
    assert bwd(dtype=0) == UNS  # fp32 backward is not provided
    assert bwd(N=(1 << 22) + 1) == UNS
    assert lib.attn_bwd_preprocess(FAKE, FAKE, FAKE, 1, 1, (1 << 22) + 1, 64, 1, None) == UNS
    assert lib.attn_bwd_dkdv(*([FAKE] * 8), 1, 1, (1 << 22) + 1, 64, 1, 0.1, 0, None) == UNS
    assert lib.attn_bwd_dq(*([FAKE] * 8), 1, 1, (1 << 22) + 1, 64, 1, 0.1, 0, None) == UNS
    assert lib.attn_bwd_preprocess(FAKE, FAKE, None, 1, 1, 8, 64, 1, None) == INV
    assert lib.attn_bwd_preprocess(FAKE, FAKE, FAKE, 1, 1, 8, 80, 1, None) == UNS
    assert lib.attn_bwd_dkdv(*([FAKE] * 7), None, 1, 1, 8, 64, 1, 0.1, 0, None) == INV
    assert lib.attn_bwd_dkdv(*([FAKE] * 8), 1, 1, 8, 64, 0, 0.1, 0, None) == UNS
    assert lib.attn_bwd_dq(*([FAKE] * 6), None, FAKE, 1, 1, 8, 64, 1, 0.1, 0, None) == INV
    assert lib.attn_bwd_dq(*([FAKE] * 7), None, 1, 1, 8, 64, 1, 0.1, 0, None) == INV
    assert lib.attn_bwd_dq(*([FAKE] * 8), 1, 1, 8, 128, 1, 0.1, 5, None) == INV
    for i in range(8):
        p = [FAKE] * 8
        p[i] = None
        assert lib.attn_bwd_dq_fused(*p, 1, 1, 8, 64, 1, 0.1, 0, None) == INV, i
    assert lib.attn_bwd_dq_fused(*([FAKE] * 8), 1, 1, (1 << 22) + 1, 64, 1, 0.1, 0, None) == UNS
    assert lib.attn_bwd_dq_fused(*([FAKE] * 8), 1, 1, 8, 96, 1, 0.1, 0, None) == UNS
    assert lib.attn_bwd_dq_fused(*([FAKE] * 8), 1, 1, 8, 64, 0, 0.1, 0, None) == UNS
    assert lib.attn_bwd_dq_fused(*([FAKE] * 8), 1, 1, 8, 64, 1, float("nan"), 0, None) == INV
    assert lib.attn_bwd_dq_fused(*([FAKE] * 8), 1, 1, 8, 64, 1, 0.1, 2, None) == INV


def test_block_sparse_validation(lib):
    INV, UNS = binding.ATTN_ERR_INVALID, binding.ATTN_ERR_UNSUPPORTED

    def fwd_s(ptrs=None, mask=FAKE, mh=1, B=1, H=2, N=300, d=64, dtype=1, scale=0.125, causal=0):
        p = ptrs or [FAKE] * 5
        return lib.attn_fwd_block_sparse(*p, mask, mh, B, H, N, d, dtype, scale, causal, None)

    for i in range(5):
        p = [FAKE] * 5
        p[i] = None
        assert fwd_s(p) == INV, i
    assert fwd_s(mask=None) == INV
    assert fwd_s(mh=0) == INV
    assert fwd_s(mh=3) == INV  # neither 1 nor B*H = 2
    assert fwd_s(causal=3) == INV
    assert fwd_s(scale=float("inf")) == INV
    assert fwd_s(N=65536 + 1) == UNS  # longest block-sparse sequence is 65536
    assert fwd_s(dtype=0) == UNS  # fp32 block-sparse is not provided
    assert fwd_s(d=80) == UNS
    ws = lib.attn_bwd_workspace_bytes(1, 2, 300, 64)

    def bwd_s(ptrs=None, mask=FAKE, mh=2, ws_bytes=ws, N=300, d=64, dtype=1):
        p = ptrs or [FAKE] * 9
        return lib.attn_bwd_block_sparse(*p, mask, mh, FAKE, ws_bytes, 1, 2, N, d, dtype, 0.125, 1, None)

    for i in range(9):
        p = [FAKE] * 9
        p[i] = None
        assert bwd_s(p) == INV, i
    assert bwd_s(mask=None) == INV
    assert bwd_s(mh=4) == INV
    assert bwd_s(ws_bytes=ws - 1) == INV
    assert bwd_s(N=70000) == UNS
    assert bwd_s(dtype=0) == UNS


def test_dropout_validation(lib):
    INV, UNS = binding.ATTN_ERR_INVALID, binding.ATTN_ERR_UNSUPPORTED

    def fwd_d(ptrs=None, p=0.1, seed=7, N=100, d=64, dtype=1, causal=0):
        pp = ptrs or [FAKE] * 5
        return lib.attn_fwd_dropout(*pp, p, seed, 1, 2, N, d, dtype, 0.125, causal, None)

    for i in range(5):
        pp = [FAKE] * 5
        pp[i] = None
        assert fwd_d(pp) == INV, i
    assert fwd_d(p=-0.01) == INV
    assert fwd_d(p=float("nan")) == INV
    assert fwd_d(p=0.999) == INV  # round(256 p) = 256 is past the last threshold
    assert fwd_d(p=1.0) == INV
    assert fwd_d(causal=2) == INV
    assert fwd_d(dtype=0) == UNS
    assert fwd_d(d=32) == UNS
    ws = lib.attn_bwd_workspace_bytes(1, 2, 100, 64)

    def bwd_d(ptrs=None, p=0.25, ws_bytes=ws, dtype=1):
        pp = ptrs or [FAKE] * 9
        return lib.attn_bwd_dropout(*pp, p, 7, FAKE, ws_bytes, 1, 2, 100, 64, dtype, 0.125, 0, None)

    for i in range(9):
        pp = [FAKE] * 9
        pp[i] = None
        assert bwd_d(pp) == INV, i
    assert bwd_d(p=2.0) == INV
    assert bwd_d(ws_bytes=ws - 1) == INV
    assert bwd_d(dtype=0) == UNS


def test_decode_workspace_and_validation(lib):
    INV, UNS = binding.ATTN_ERR_INVALID, binding.ATTN_ERR_UNSUPPORTED
    # chunks of 512 keys, or 256 / 128 when 512 would give the call fewer than 1024 workgroups (B*H*chunks);
    # per chunk and query: m, l and d floats, rounded up to 256 bytes
    def chunks(BH, Nk):
        for ch in (512, 256):
            if BH * -(-Nk // ch) >= 1024:
                return -(-Nk // ch)
        return -(-Nk // 128)

    def expect(B, H, Nq, Nk, d):
        return ((B * H * chunks(B * H, Nk) * Nq * (d + 2) * 4 + 255) // 256) * 256

    assert lib.attn_decode_workspace_bytes(2, 3, 1, 1000, 128) == expect(2, 3, 1, 1000, 128) == 25088  # 8 chunks of 128
    assert lib.attn_decode_workspace_bytes(1, 1, 8, 512, 64) == expect(1, 1, 8, 512, 64) == 4 * 8 * 66 * 4
    assert lib.attn_decode_workspace_bytes(4, 32, 8, 16384, 128) == expect(4, 32, 8, 16384, 128)  # 512-key chunks
    assert chunks(128, 16384) == 32 and chunks(8, 32768) == 128 and chunks(1, 1 << 23) == (1 << 23) // 512
    assert lib.attn_decode_workspace_bytes(1, 1, 9, 512, 64) == 0
    assert lib.attn_decode_workspace_bytes(1, 1, 1, 0, 64) == 0
    assert lib.attn_decode_workspace_bytes(1, 1, 1, 100, 96) == 0
    ws = lib.attn_decode_workspace_bytes(1, 2, 4, 700, 64)

    def dec(ptrs=None, ws_bytes=ws, Nq=4, Nk=700, d=64, dtype=1, scale=0.125, causal=1):
        p = ptrs or [FAKE] * 6
        return lib.attn_decode(*p, ws_bytes, 1, 2, Nq, Nk, d, dtype, scale, causal, None)

    for i in range(6):
        p = [FAKE] * 6
        p[i] = None
        assert dec(p) == INV, i
    assert dec(ws_bytes=ws - 1) == INV
    assert dec(Nq=0) == INV
    assert dec(Nk=0) == INV
    assert dec(Nq=5, Nk=4) == INV  # causal needs Nq <= Nk
    assert dec(scale=float("inf")) == INV
    assert dec(causal=3) == INV
    assert dec(Nq=9) == UNS
    assert dec(Nk=(1 << 23) + 1) == UNS
    assert dec(d=80) == UNS
    assert dec(dtype=0) == UNS


def test_fp8_validation(lib):
    INV, UNS = binding.ATTN_ERR_INVALID, binding.ATTN_ERR_UNSUPPORTED

    def f8(ptrs=None, dq=0.01, dk=0.01, dv=0.01, N=300, d=128, scale=0.088, causal=1):
        p = ptrs or [FAKE] * 5
        return lib.attn_fwd_fp8(p[0], p[1], p[2], dq, dk, dv, p[3], p[4], 1, 2, N, d, scale, causal, None)

    for i in range(5):
        p = [FAKE] * 5
        p[i] = None
        assert f8(p) == INV, i
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert f8(dq=bad) == INV and f8(dk=bad) == INV and f8(dv=bad) == INV
    for bad in (float("inf"), float("-inf"), float("nan")):
        assert f8(scale=bad) == INV
    assert f8(dq=1e-30, dk=1e-30) == INV  # scale dq dk underflows fp32
    assert f8(dq=1e-30, dk=1e-30, scale=-0.088) == INV  # |scale dq dk| underflows fp32
    assert f8(dq=1e30, dk=1e30) == INV  # overflows
    assert f8(N=0) == INV
    assert f8(causal=2) == INV
    assert f8(d=96) == UNS
    assert f8(N=(1 << 22) + 1) == UNS


def test_binding_checks_block_mask_shape():
    import torch

    q = torch.zeros(1, 2, 300, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):  # CPU tensors are refused before the mask is looked at
        binding.fwd_block_sparse(q, q, q, torch.ones(3, 3, dtype=torch.uint8))
    with pytest.raises(ValueError):
        binding._block_mask(torch.ones(2, 2, dtype=torch.uint8), 1, 2, 300)  # nb is 3
    with pytest.raises(ValueError):
        binding._block_mask(torch.ones(3, 3, 3, dtype=torch.uint8), 1, 2, 300)  # 3 heads of masks for B*H = 2


def test_binding_refuses_cpu_tensors():
    """Every tensor-taking entry point of the binding refuses CPU tensors before
    any pointer reaches the library (no GPU is needed: the check comes first)."""
    import torch

    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    f = torch.zeros(1, 1, 4, dtype=torch.float32)
    m = torch.ones(1, 1, 1, dtype=torch.uint8)
    u8 = torch.zeros(1, 1, 4, 64, dtype=torch.uint8)
    calls = {
        "fwd": lambda: binding.fwd(q, q, q),
        "bwd": lambda: binding.bwd(q, q, q, q, f, q),
        "bwd_preprocess": lambda: binding.bwd_preprocess(q, q),
        "bwd_dkdv": lambda: binding.bwd_dkdv(q, q, q, f, q, f),
        "bwd_dq": lambda: binding.bwd_dq(q, q, q, f, q, f),
        "bwd_dq_fused": lambda: binding.bwd_dq_fused(q, q, q, q, f, q),
        "fwd_block_sparse": lambda: binding.fwd_block_sparse(q, q, q, m),
        "bwd_block_sparse": lambda: binding.bwd_block_sparse(q, q, q, q, f, q, m),
        "fwd_dropout": lambda: binding.fwd_dropout(q, q, q, 0.1, 1),
        "bwd_dropout": lambda: binding.bwd_dropout(q, q, q, q, f, q, 0.1, 1),
        "decode": lambda: binding.decode(q, q, q),
        "fwd_fp8": lambda: binding.fwd_fp8(u8, u8, u8, 1.0, 1.0, 1.0),
    }
    for name, call in calls.items():
        with pytest.raises(ValueError):
            call()


def test_autograd_wrapper_refuses_cpu_tensors():
    import torch

    from exact_io_aware_23_amd import attention

    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        attention(q, q, q)


def test_noalloc_validation(lib):
    """attn_bwd_noalloc validates like attn_bwd and rejects problems larger than
    its static scratch array with ATTN_ERR_SCRATCH, before any launch."""
    INV, UNS, SCR = binding.ATTN_ERR_INVALID, binding.ATTN_ERR_UNSUPPORTED, binding.ATTN_ERR_SCRATCH
    rows = lib.attn_bwd_noalloc_max_rows()
    assert rows == (16 << 20) // 4

    def call(ptrs=None, B=1, H=2, N=100, d=64, dtype=1, scale=0.125, causal=1):
        p = ptrs or [FAKE] * 9
        return lib.attn_bwd_noalloc(*p, B, H, N, d, dtype, scale, causal, None)

    for i in range(9):
        p = [FAKE] * 9
        p[i] = None
        assert call(p) == INV, i
    assert call(N=0) == INV
    assert call(scale=float("nan")) == INV
    assert call(causal=2) == INV
    assert call(d=96) == UNS
    assert call(dtype=0) == UNS
    assert call(B=2, H=2, N=(1 << 20) + 1) == SCR  # one row past the scratch array
    assert call(B=1, H=3, N=1 << 21) == SCR
