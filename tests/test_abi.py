"""The C ABI without a GPU: symbols, argument validation, one HIP runtime.

Every call made here fails validation by construction (null pointers, bad
sizes, bad dtype), so nothing is ever launched; the library promises to make
no HIP call before validation passes.
"""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


@pytest.fixture(scope="module")
def lib():
    from exact_softmax_attention_attn_amd import binding, build_lib
    if not os.path.exists(binding.LIB_PATH):
        build_lib.build()
    return binding.load()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(attn_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    assert _declared() == sorted([
        "attn_bwd", "attn_bwd_bwd", "attn_bwd_bwd_masked", "attn_bwd_bwd_workspace_bytes",
        "attn_bwd_dkdv",
        "attn_bwd_dkdv_masked", "attn_bwd_dq", "attn_bwd_dq_masked", "attn_bwd_masked",
        "attn_bwd_noalloc", "attn_bwd_preprocess", "attn_bwd_workspace_bytes", "attn_fwd_lse",
        "attn_fwd_lse_masked", "attn_last_error", "attn_status_string"])


def test_library_exports_every_declared_symbol(lib):
    from exact_softmax_attention_attn_amd import binding
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH],
                         stdout=subprocess.PIPE, text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for name in _declared():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_library_never_allocates_device_memory(lib):
    # the caller owns every buffer: no allocation or free entry point is imported
    from exact_softmax_attention_attn_amd import binding
    out = subprocess.run(["nm", "-D", "--undefined-only", binding.LIB_PATH],
                         stdout=subprocess.PIPE, text=True, check=True).stdout
    imported = [line.split()[-1] for line in out.splitlines() if line.strip()]
    bad = [s for s in imported if re.match(r"hip(Ext)?(Malloc|Free|MallocAsync|FreeAsync|HostMalloc)", s)]
    assert bad == []


def test_every_kernel_launched_has_its_host_stub(lib):
    # a kernel template whose host-side instantiation was dropped leaves its
    # launch stub undefined; the library would then fail to load at run time
    from exact_softmax_attention_attn_amd import binding
    out = subprocess.run(["nm", "-D", "--undefined-only", binding.LIB_PATH],
                         stdout=subprocess.PIPE, text=True, check=True).stdout
    missing = [line.split()[-1] for line in out.splitlines() if "__device_stub__" in line]
    assert missing == []


def test_status_strings(lib):
    assert lib.attn_status_string(0) == b"ok"
    assert lib.attn_status_string(1) == b"invalid argument"
    assert lib.attn_status_string(2).startswith(b"unsupported")
    assert lib.attn_status_string(3).startswith(b"HIP")
    assert lib.attn_status_string(99) == b"unknown status"
    assert lib.attn_last_error() == b""


def test_workspace_bytes(lib):
    assert lib.attn_bwd_workspace_bytes(1, 16, 16384, 128) == 2 * 16 * 16384 * 4
    assert lib.attn_bwd_workspace_bytes(3, 2, 8, 4) == 2 * 48 * 4
    assert lib.attn_bwd_workspace_bytes(0, 2, 8, 4) == 0
    assert lib.attn_bwd_workspace_bytes(1, 1, -5, 4) == 0


FAKE = ctypes.c_void_p(0x10000)      # never dereferenced: every call below fails validation
NUL = ctypes.c_void_p(0)
MIS = ctypes.c_void_p(0x10008)       # not 16-byte aligned


def _fwd(lib, ptrs, B=1, H=1, N=8, d=8, causal=1, scale=0.5, dtype=0):
    return lib.attn_fwd_lse(*ptrs, B, H, N, d, causal, scale, dtype, NUL)


def _bwd(lib, ptrs, B=1, H=1, N=8, d=8, causal=1, scale=0.5, dtype=0):
    return lib.attn_bwd(*ptrs, B, H, N, d, causal, scale, dtype, NUL)


def test_validation_rejects_bad_arguments_without_launching(lib):
    f5 = [FAKE] * 5
    b10 = [FAKE] * 10
    # null or misaligned pointers
    for i in range(5):
        p = list(f5); p[i] = NUL
        assert _fwd(lib, p, d=132) == 1           # pointer checked before d
        p[i] = MIS
        assert _fwd(lib, p, d=132) == 1
    for i in range(10):
        p = list(b10); p[i] = NUL
        assert _bwd(lib, p, d=132) == 1
    # sizes < 1
    for kw in ({"B": 0}, {"H": 0}, {"N": 0}, {"d": 0}, {"N": -3}):
        assert _fwd(lib, f5, **kw) == 1
        assert _bwd(lib, b10, **kw) == 1
    # scale and causal flag
    for kw in ({"scale": 0.0}, {"scale": -1.0}, {"scale": float("inf")}, {"scale": float("nan")},
               {"causal": 2}, {"causal": -1}):
        assert _fwd(lib, f5, **kw) == 1
        assert _bwd(lib, b10, **kw) == 1
    # unsupported head dims and dtypes
    for kw in ({"d": 136}, {"d": 264, "dtype": 1}, {"d": 6}, {"d": 4, "dtype": 1},
               {"d": 12, "dtype": 1}, {"dtype": 2},
               {"dtype": -1}, {"B": 70000}, {"H": 70000}, {"B": 65535, "H": 65535, "N": 1024}):
        assert _fwd(lib, f5, **kw) == 2, kw
        assert _bwd(lib, b10, **kw) == 2, kw
    # wide heads split their output columns over two workgroups per block
    # along the grid's y axis (bf16 d > 128, f32 d > 64): H * 2 must fit 65535
    for kw in ({"H": 32768, "d": 256, "dtype": 1}, {"H": 40000, "d": 136, "dtype": 1},
               {"H": 32768, "d": 128}, {"H": 32768, "d": 68}):
        assert _fwd(lib, f5, **kw) == 2, kw
        assert _bwd(lib, b10, **kw) == 2, kw
        assert lib.attn_bwd_dkdv(*([FAKE] * 7), 1, kw["H"], 8, kw["d"], 1, 0.5,
                                 kw.get("dtype", 0), NUL) == 2, kw
    # row count B*H*N < 2^31 (so B*N*H*d < 2^39 with d <= 256)
    assert _bwd(lib, b10, B=65535, H=16, N=2049, d=8) == 2      # 2^31 + 917,488 rows
    assert _fwd(lib, f5, B=8192, H=16, N=16384, d=256, dtype=1) == 2   # exactly 2^31 rows
    # the stage entry points validate the same way
    assert lib.attn_bwd_preprocess(FAKE, NUL, FAKE, FAKE, 1, 1, 8, 8, 0, NUL) == 1
    assert lib.attn_bwd_preprocess(FAKE, FAKE, NUL, FAKE, 1, 1, 8, 8, 0, NUL) == 1
    assert lib.attn_bwd_preprocess(FAKE, FAKE, FAKE, FAKE, 1, 1, 8, 6, 0, NUL) == 2
    assert lib.attn_bwd_dkdv(*([FAKE] * 6), NUL, 1, 1, 8, 8, 1, 0.5, 0, NUL) == 1
    assert lib.attn_bwd_dkdv(*([FAKE] * 7), 1, 1, 8, 8, 1, 0.0, 0, NUL) == 1
    assert lib.attn_bwd_dq(*([FAKE] * 5), NUL, 1, 1, 8, 8, 1, 0.5, 0, NUL) == 1
    assert lib.attn_bwd_dq(*([FAKE] * 6), 1, 1, 8, 264, 1, 0.5, 1, NUL) == 2
    assert lib.attn_last_error() == b""


def test_masked_entry_points_validate_the_mask(lib):
    f5 = [FAKE] * 5
    b10 = [FAKE] * 10

    def fwd(mask, heads, B=1, H=1, N=8, d=8, causal=1, scale=0.5, dtype=0):
        return lib.attn_fwd_lse_masked(*f5, mask, heads, B, H, N, d, causal, scale, dtype, NUL)

    def bwd(mask, heads, B=1, H=1, N=8, d=8, causal=1, scale=0.5, dtype=0):
        return lib.attn_bwd_masked(*b10, mask, heads, B, H, N, d, causal, scale, dtype, NUL)

    for call in (fwd, bwd):
        assert call(NUL, 1) == 1                              # no mask
        assert call(FAKE, 0) == 1                             # mask_heads not 1 or B * H
        assert call(FAKE, 3, B=2, H=2) == 1
        assert call(FAKE, 1, N=65537) == 2                    # longer walks than the lists hold
        assert call(FAKE, 1, d=136) == 2                      # the shared checks still apply
        assert call(FAKE, 1, scale=0.0) == 1
    p = list(b10); p[3] = NUL
    assert lib.attn_bwd_masked(*p, FAKE, 1, 1, 1, 8, 8, 1, 0.5, 0, NUL) == 1
    assert lib.attn_bwd_dkdv_masked(*([FAKE] * 7), NUL, 1, 1, 1, 8, 8, 1, 0.5, 0, NUL) == 1
    assert lib.attn_bwd_dkdv_masked(*([FAKE] * 7), FAKE, 2, 1, 1, 8, 8, 1, 0.5, 0, NUL) == 1
    assert lib.attn_bwd_dq_masked(*([FAKE] * 6), FAKE, 1, 1, 1, 70000, 8, 1, 0.5, 0, NUL) == 2
    assert lib.attn_bwd_dq_masked(*([FAKE] * 5), NUL, FAKE, 1, 1, 1, 8, 8, 1, 0.5, 0, NUL) == 1
    assert lib.attn_last_error() == b""


def test_bwd_bwd_entry_point_validates(lib):
    p14 = [FAKE] * 14

    def call(ptrs=p14, B=1, H=1, N=8, d=8, causal=1, scale=0.5, dtype=0):
        return lib.attn_bwd_bwd(*ptrs, B, H, N, d, causal, scale, dtype, NUL)

    for i in range(14):
        p = list(p14); p[i] = NUL
        assert call(p) == 1
        p[i] = MIS
        assert call(p) == 1
    assert call(N=0) == 1 and call(scale=-1.0) == 1 and call(causal=3) == 1
    assert call(d=68) == 2                      # f32 stops at 64
    assert call(d=136, dtype=1) == 2            # bf16 stops at 128
    assert call(dtype=5) == 2
    assert lib.attn_bwd_bwd_workspace_bytes(2, 3, 10, 64) == 4 * 60 * 4
    assert lib.attn_bwd_bwd_workspace_bytes(0, 3, 10, 64) == 0
    assert lib.attn_last_error() == b""


def test_masked_bwd_bwd_entry_point_validates(lib):
    p14 = [FAKE] * 14

    def call(mask=FAKE, heads=1, ptrs=p14, B=1, H=1, N=8, d=8, causal=1, scale=0.5, dtype=0):
        return lib.attn_bwd_bwd_masked(*ptrs, mask, heads, B, H, N, d, causal, scale, dtype, NUL)

    for i in range(14):
        p = list(p14); p[i] = NUL
        assert call(ptrs=p) == 1
    assert call(mask=NUL) == 1                  # no mask
    assert call(heads=0) == 1                   # mask_heads not 1 or B * H
    assert call(heads=3, B=2, H=2) == 1
    assert call(N=65537) == 2                   # longer walks than the visit lists hold
    assert call(d=68) == 2 and call(d=136, dtype=1) == 2
    assert call(scale=0.0) == 1 and call(causal=3) == 1
    assert lib.attn_last_error() == b""


def test_binding_marshals_and_checks_before_calling():
    torch = pytest.importorskip("torch")
    from exact_softmax_attention_attn_amd import binding
    q = torch.zeros(1, 8, 1, 8)
    with pytest.raises(ValueError):
        binding.attn_fwd_lse(q, q, q)          # CPU tensors are refused before any call
    with pytest.raises(TypeError):
        binding._dtype_code(torch.zeros(1, dtype=torch.float16))


def test_one_hip_runtime_is_mapped(lib):
    maps = open("/proc/self/maps").read()
    hip = set(l.split()[-1] for l in maps.splitlines() if "libamdhip64" in l)
    assert len(hip) == 1, hip


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    # no CPU fallback: with the library absent, loading (and so every call) raises
    from exact_softmax_attention_attn_amd import binding
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        binding.load(str(tmp_path / "libattn.so"))


def test_noalloc_entry_point_validates_before_any_hip_call(lib):
    p9 = [FAKE] * 9

    def call(ptrs=p9, B=1, H=1, N=8, d=8, causal=1, scale=0.5, dtype=0):
        return lib.attn_bwd_noalloc(*ptrs, B, H, N, d, causal, scale, dtype, NUL)

    for i in range(9):
        p = list(p9); p[i] = NUL
        assert call(p) == 1
        p[i] = MIS
        assert call(p) == 1
    assert call(N=0) == 1 and call(scale=0.0) == 1 and call(causal=2) == 1
    assert call(d=136) == 2 and call(dtype=3) == 2
    assert lib.attn_last_error() == b""
    # the static workspace holds 2 * 2,097,152 floats: one row more is refused
    assert call(B=1, H=1, N=2097153) == 2
    assert b"exceeds" in lib.attn_last_error()
    assert call(B=2, H=16, N=65537) == 2
    # (last in this file: it leaves attn_last_error() set on this thread)
