"""The C ABI on the host: the library loads, exports every declared symbol, and
validates arguments before touching any device (no GPU needed)."""
import ctypes
import os
import re
import subprocess

import pytest

import exact_attention_65_amd as fa
from exact_attention_65_amd import build as fab

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def gpu_visible() -> bool:
    import torch
    return torch.cuda.device_count() > 0


@pytest.fixture(scope="module", autouse=True)
def built_library():
    if not os.path.exists(fab.LIB_PATH):
        fab.build()
    return fab.LIB_PATH


def declared_functions():
    text = open(os.path.join(ROOT, "include", "fa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(fa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(fa.EXPORTED)


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(fab.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", fab.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (fa_\w+)$", out, flags=re.M))
    assert exported == set(declared_functions())


def test_probe_library_exports_what_its_header_declares():
    if not os.path.exists(fab.PROBE_LIB_PATH):
        fab.build()
    text = open(os.path.join(ROOT, "include", "fa_probe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    declared = set(re.findall(r"^\s*\w+\**\s+\**(fa_probe_\w+)\s*\(", text, flags=re.M))
    assert declared == {"fa_probe_stamp", "fa_probe_mfma_query", "fa_probe_mfma", "fa_probe_wallclock_khz"}
    out = subprocess.run(["nm", "-D", "--defined-only", fab.PROBE_LIB_PATH], capture_output=True, text=True).stdout
    assert set(re.findall(r" T (fa_\w+)$", out, flags=re.M)) == declared
    from exact_attention_65_amd import probe
    assert probe.STAMP_BLOCKS == int(re.search(r"#define FA_PROBE_STAMP_BLOCKS (\d+)", text).group(1))
    lib = probe.lib()
    blocks, flops = ctypes.c_int(0), ctypes.c_double(0.0)
    assert lib.fa_probe_mfma_query(0, ctypes.byref(blocks), ctypes.byref(flops)) == -1
    assert lib.fa_probe_stamp(None, None) == -1


def test_probe_clock_from_stamps():
    from exact_attention_65_amd import probe
    # 64 compute-unit tags; the second stamp 1 ms later at 2000 MHz (counters per
    # unit start at different values, and the second stamp's blocks land on the
    # units in another order), constant rate 100 MHz
    a, b = [], []
    for blk in range(probe.STAMP_BLOCKS):
        x, y = blk % 64, (blk * 7 + 3) % 64
        a += [10**9 * (x + 1), 5 * 10**6, x]
        b += [10**9 * (y + 1) + 2 * 10**6, 5 * 10**6 + 10**5, y]
    assert abs(probe.clock_mhz(a, b, 100000) - 2000.0) < 1e-9


def test_version_and_strings():
    assert fa.fa_abi_version() == 9
    for st in range(10):
        s = fa.fa_status_str(st)
        assert s.startswith("FA_")
    assert fa.fa_status_str(99) == "unknown fa_status"


def test_query_sizes():
    st, sz = fa.fa_fwd_query(2, 32, 4096, 128, 0, fa.FA_DTYPE_BF16)
    assert st == fa.FA_OK
    assert sz.q_bytes == sz.k_bytes == sz.v_bytes == sz.o_bytes == 2 * 32 * 4096 * 128 * 2
    assert sz.lse_bytes == 2 * 32 * 4096 * 4 and sz.workspace_bytes == 0
    st, sz = fa.fa_fwd_query(1, 8, 131072, 128, 1, fa.FA_DTYPE_BF16)
    assert st == fa.FA_OK and sz.workspace_bytes == 0
    st, sz = fa.fa_fwd_query(1, 1, 256, 64, 0, fa.FA_DTYPE_F32)
    assert st == fa.FA_OK and sz.q_bytes == 256 * 64 * 4
    st, sz = fa.fa_fwd_query(1, 1, 256, 64, 0, fa.FA_DTYPE_F16)
    assert st == fa.FA_OK and sz.q_bytes == 256 * 64 * 2
    assert fa.fa_fwd_split_query(1, 1, 16, 256, 64, 1, 0, fa.FA_DTYPE_F16)[0] == fa.FA_OK
    assert fa.fa_bwd_query(1, 1, 256, 64, 0, fa.FA_DTYPE_F16)[0] == fa.FA_OK
    assert fa.fa_bwd_query(1, 1, 256, 96, 0, fa.FA_DTYPE_F16)[0] == fa.FA_OK
    assert fa.fa_bwd_query(1, 1, 256, 96, 0, fa.FA_DTYPE_F32)[0] == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_fwd_query(1, 1, 256, 96, 0, fa.FA_DTYPE_BF16)[0] == fa.FA_OK
    assert fa.fa_fwd_query(1, 1, 256, 96, 0, fa.FA_DTYPE_F32)[0] == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_fwd_query(1, 1, 256, 80, 0, fa.FA_DTYPE_BF16)[0] == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_fwd_query(1, 1, 256, 256, 0, fa.FA_DTYPE_BF16)[0] == fa.FA_OK
    assert fa.fa_fwd_query(1, 1, 256, 256, 0, fa.FA_DTYPE_F16)[0] == fa.FA_OK
    assert fa.fa_fwd_query(1, 1, 256, 256, 0, fa.FA_DTYPE_F32)[0] == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_fwd_split_query(1, 1, 16, 512, 256, 1, 0, fa.FA_DTYPE_BF16)[0] == fa.FA_OK
    assert fa.fa_bwd_query(1, 1, 256, 256, 0, fa.FA_DTYPE_BF16)[0] == fa.FA_OK
    assert fa.fa_bwd_query(1, 1, 256, 512, 0, fa.FA_DTYPE_BF16)[0] == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_fwd_fp8_query(1, 1, 256, 256, 0)[0] == fa.FA_OK
    assert fa.fa_fwd_fp8_query(1, 1, 256, 96, 0)[0] == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_fwd_query(1, 1, 1 << 24, 128, 0, fa.FA_DTYPE_BF16)[0] == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_fwd_query(0, 1, 256, 64, 0, fa.FA_DTYPE_BF16)[0] == fa.FA_ERR_BAD_SHAPE
    assert fa.fa_fwd_query(1, 1, -3, 64, 0, fa.FA_DTYPE_BF16)[0] == fa.FA_ERR_BAD_SHAPE
    assert fa.fa_fwd_query(1 << 40, 1 << 40, 256, 64, 0, fa.FA_DTYPE_BF16)[0] == fa.FA_ERR_BAD_SHAPE
    assert fa.fa_fwd_query(1, 1, 256, 64, 0, 7)[0] == fa.FA_ERR_BAD_DTYPE
    assert fa.fa_fwd_query(1, 1, 256, 64, 0, 3)[0] == fa.FA_ERR_BAD_DTYPE
    assert fa.lib().fa_fwd_query(1, 1, 256, 64, 0, 1, None) == fa.FA_ERR_NULL_POINTER
    # too many workgroups for one launch
    assert fa.fa_fwd_query(1 << 20, 1 << 10, 256, 64, 0, fa.FA_DTYPE_BF16)[0] == fa.FA_ERR_UNSUPPORTED


# fake, never-dereferenced addresses: validation rejects these calls on the host
A = 1 << 20
SZ = 1 << 20  # spacing of the fake buffers: larger than any tensor used below


def call(q=A, k=A + SZ, v=A + 2 * SZ, o=A + 3 * SZ, lse=A + 4 * SZ, B=1, H=2, N=100, D=64,
         causal=0, scale=0.125, dtype=fa.FA_DTYPE_BF16):
    return fa.fa_fwd(q, k, v, o, lse, B, H, N, D, causal, scale, dtype, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=0), fa.FA_ERR_NULL_POINTER),
    (dict(lse=0), fa.FA_ERR_NULL_POINTER),
    (dict(N=0), fa.FA_ERR_BAD_SHAPE),
    (dict(B=-1), fa.FA_ERR_BAD_SHAPE),
    (dict(scale=float("nan")), fa.FA_ERR_BAD_SCALE),
    (dict(scale=float("inf")), fa.FA_ERR_BAD_SCALE),
    (dict(dtype=5), fa.FA_ERR_BAD_DTYPE),
    (dict(k=A + SZ + 8), fa.FA_ERR_MISALIGNED),
    (dict(lse=A + 4 * SZ + 4), fa.FA_ERR_MISALIGNED),
    (dict(o=A + SZ), fa.FA_ERR_ALIASING),               # o on top of k
    (dict(lse=A + 3 * SZ + 16), fa.FA_ERR_ALIASING),    # lse inside o
    (dict(o=A + 2 * SZ + 2 * 100 * 64 * 2 - 16), fa.FA_ERR_ALIASING),  # o starts in v's last 16 bytes
    (dict(o=A + 2 * SZ + 2 * 100 * 64 * 2), fa.FA_ERR_HIP),  # o right after v: valid
    (dict(lse=A), fa.FA_ERR_ALIASING),                  # lse on top of q
    (dict(D=80), fa.FA_ERR_UNSUPPORTED),
    (dict(D=32), fa.FA_ERR_UNSUPPORTED),
])
def test_validation_before_any_device_call(kw, expect):
    if expect == fa.FA_ERR_HIP and gpu_visible():
        pytest.skip("valid arguments would launch on fake addresses when a GPU is visible")
    assert call(**kw) == expect


def test_inputs_may_alias_each_other():
    # q = k = v is valid; with no GPU visible the call then fails at the device query
    if gpu_visible():
        pytest.skip("valid arguments would launch on fake addresses when a GPU is visible")
    assert call(k=A, v=A) == fa.FA_ERR_HIP


def test_valid_call_without_device_reports_hip_error():
    if gpu_visible():
        pytest.skip("a GPU is visible here")
    assert call() == fa.FA_ERR_HIP


def test_binding_rejects_bad_tensors():
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.float64)
    with pytest.raises(TypeError):
        fa.attention_forward(q, q, q)
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.attention_forward(q, q, q)  # CPU tensors


def test_binding_checks_given_outputs():
    """Caller-supplied outputs and workspaces are checked for shape, dtype,
    device and layout (the C ABI sees only their addresses)."""
    import torch
    dev = torch.device("cpu")
    good = torch.empty(2, 3, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="dtype"):
        fa._check_given(good.float(), "out", good.shape, torch.bfloat16, dev)
    with pytest.raises(ValueError, match="on"):
        fa._check_given(good, "out", good.shape, torch.bfloat16, torch.device("cuda", 0))
    with pytest.raises(ValueError, match="contiguous"):
        fa._check_given(good.transpose(2, 3), "out", None, torch.bfloat16, dev)
    with pytest.raises(ValueError, match="shape"):
        fa._check_given(torch.empty(2, 3, 7, 64, dtype=torch.bfloat16), "out", good.shape, torch.bfloat16, dev)
    with pytest.raises(ValueError, match="bytes"):
        fa._check_workspace(torch.empty(10, dtype=torch.uint8), 11, dev)


@pytest.mark.slow
@pytest.mark.parametrize("source", ["fa_fwd.hip", "fa_bwd.hip", "fa_fp8.hip"])
def test_device_code_has_no_packed_fp32_and_no_spills(source):
    asm = fab.device_asm(source)
    assert not re.search(r"v_pk_(add|mul|fma)_f32", asm)
    found = 0
    for m in re.finditer(r"\.name:\s+(\S+)\n(?:.*\n){0,12}?\s+\.vgpr_spill_count:\s+(\d+)", asm):
        found += 1
        assert int(m.group(2)) == 0, m.group(1)
    assert found > 0


def test_every_kernel_stub_is_defined():
    """The host pass can silently drop a kernel's launch stub; the library must define all of them."""
    out = subprocess.run(["nm", "-D", fab.LIB_PATH], capture_output=True, text=True).stdout
    undefined = [l for l in out.splitlines() if " U " in l and "_ZN2fa" in l]
    assert undefined == []
    kernels = set(re.findall(r"(_ZN2fa\d+fa_\w+_kernelI\w+)", out))
    # bf16 and fp16: D (64, 96, 128, 256) x causal x split; fp32: D x causal; merge: D x (bf16, fp16);
    # backward: (bf16, fp16) x 3 kernels (dq, dk/dv, both in one grid) x D (64, 96, 128) x causal, the
    # Delta kernel (bf16, fp16) x D and at D = 256 (bf16, fp16) x (dq, 16-key dk/dv) x causal;
    # fp8: D (64, 128, 256) x causal; one-query-row: (bf16, fp16) x
    # D (64, 128, 256); 16-row-wave kernel: (bf16, fp16) x causal x (64-row form for small grids: D 64, 96
    # and 128 with one or two waves per slice, D 256 with two; 128-row form: D 256)
    assert len(kernels) == 32 + 4 + 8 + 36 + 6 + 8 + 6 + 6 + 28 + 4, kernels


# ---------------------------------------------------------------- fa_fwd_split
def test_split_query_sizes_and_ranges():
    st, sz, s = fa.fa_fwd_split_query(4, 32, 1, 16384, 128, 1, fa.FA_SPLIT_AUTO, fa.FA_DTYPE_BF16)
    assert st == fa.FA_OK
    assert sz.q_bytes == sz.o_bytes == 4 * 32 * 1 * 128 * 2
    assert sz.k_bytes == sz.v_bytes == 4 * 32 * 16384 * 128 * 2
    assert sz.lse_bytes == 4 * 32 * 4
    # one query row: the vector-unit kernel, 4 ranges give 512 workgroups
    assert s == 4 and sz.workspace_bytes == 4 * 4 * 32 * 1 * (128 + 1) * 4
    # ... with at least 1024 keys a range
    st, sz, s = fa.fa_fwd_split_query(1, 1, 1, 5000, 64, 0, fa.FA_SPLIT_AUTO, fa.FA_DTYPE_BF16)
    assert st == fa.FA_OK and s == 4
    # ... but not at D = 96 (the 128-row kernel's rule: 8 tiles a range)
    st, sz, s = fa.fa_fwd_split_query(1, 1, 1, 5000, 96, 0, fa.FA_SPLIT_AUTO, fa.FA_DTYPE_BF16)
    assert st == fa.FA_OK and s == 9
    # one range: no workspace
    st, sz, s = fa.fa_fwd_split_query(2, 32, 4096, 4096, 128, 0, 1, fa.FA_DTYPE_BF16)
    assert st == fa.FA_OK and s == 1 and sz.workspace_bytes == 0
    # enough query blocks already: the automatic choice is one range
    st, sz, s = fa.fa_fwd_split_query(2, 32, 4096, 4096, 128, 0, fa.FA_SPLIT_AUTO, fa.FA_DTYPE_BF16)
    assert st == fa.FA_OK and s == 1 and sz.workspace_bytes == 0
    # caps: 8 key tiles per range ...
    st, sz, s = fa.fa_fwd_split_query(1, 1, 16, 8192, 64, 1, fa.FA_SPLIT_AUTO, fa.FA_DTYPE_BF16)
    assert st == fa.FA_OK and s == 16
    st, sz, s = fa.fa_fwd_split_query(1, 1, 16, 300, 64, 1, fa.FA_SPLIT_AUTO, fa.FA_DTYPE_BF16)
    assert st == fa.FA_OK and s == 1
    # ... partial results within a quarter of the K/V bytes ...
    st, sz, s = fa.fa_fwd_split_query(1, 32, 512, 8192, 128, 1, fa.FA_SPLIT_AUTO, fa.FA_DTYPE_BF16)
    assert st == fa.FA_OK and s == 4
    # ... so square shapes stay on one range
    st, sz, s = fa.fa_fwd_split_query(1, 32, 512, 512, 128, 1, fa.FA_SPLIT_AUTO, fa.FA_DTYPE_BF16)
    assert st == fa.FA_OK and s == 1 and sz.workspace_bytes == 0
    # an explicit count is used as given
    st, sz, s = fa.fa_fwd_split_query(1, 2, 100, 900, 64, 0, 7, fa.FA_DTYPE_BF16)
    assert st == fa.FA_OK and s == 7 and sz.workspace_bytes == 7 * 2 * 100 * 65 * 4


@pytest.mark.parametrize("args,expect", [
    ((1, 1, 10, 5, 64, 1, 0, fa.FA_DTYPE_BF16), fa.FA_ERR_BAD_SHAPE),     # causal with Nq > Nk
    ((1, 1, 10, 5, 64, 0, 0, fa.FA_DTYPE_BF16), fa.FA_OK),                # fine without the mask
    ((1, 1, 0, 5, 64, 0, 0, fa.FA_DTYPE_BF16), fa.FA_ERR_BAD_SHAPE),
    ((1, 1, 4, 64, 64, 0, -1, fa.FA_DTYPE_BF16), fa.FA_ERR_BAD_SHAPE),
    ((1, 1, 4, 64, 64, 0, 257, fa.FA_DTYPE_BF16), fa.FA_ERR_BAD_SHAPE),
    ((1, 1, 4, 64, 64, 0, 256, fa.FA_DTYPE_BF16), fa.FA_OK),
    ((1, 1, 4, 64, 64, 0, 0, fa.FA_DTYPE_F32), fa.FA_ERR_UNSUPPORTED),
    ((1, 1, 4, 64, 80, 0, 0, fa.FA_DTYPE_BF16), fa.FA_ERR_UNSUPPORTED),
    ((1, 1, 4, 64, 96, 0, 0, fa.FA_DTYPE_BF16), fa.FA_OK),
    ((1, 1, 4, 64, 64, 0, 0, 3), fa.FA_ERR_BAD_DTYPE),
])
def test_split_query_validation(args, expect):
    assert fa.fa_fwd_split_query(*args)[0] == expect


def split_call(q=A, k=A + SZ, v=A + 2 * SZ, o=A + 3 * SZ, lse=A + 4 * SZ, ws=A + 5 * SZ, ws_bytes=SZ,
               B=1, H=2, Nq=10, Nk=300, D=64, causal=1, scale=0.125, n_splits=3, dtype=fa.FA_DTYPE_BF16):
    return fa.fa_fwd_split(q, k, v, o, lse, ws, ws_bytes, B, H, Nq, Nk, D, causal, scale, n_splits, dtype, None)


WS3 = 3 * 2 * 10 * 65 * 4  # workspace of the default split_call


@pytest.mark.parametrize("kw,expect", [
    (dict(ws=0), fa.FA_ERR_NULL_POINTER),
    (dict(ws=0, n_splits=1), fa.FA_ERR_HIP),              # one range needs no workspace
    (dict(ws_bytes=WS3 - 1), fa.FA_ERR_WORKSPACE),
    (dict(ws_bytes=WS3), fa.FA_ERR_HIP),                  # exactly enough: valid
    (dict(ws=A + 5 * SZ + 8), fa.FA_ERR_MISALIGNED),
    (dict(ws=A + 2 * SZ), fa.FA_ERR_ALIASING),            # workspace on top of v
    (dict(ws=A + 3 * SZ + 16), fa.FA_ERR_ALIASING),       # workspace inside o
    (dict(Nq=301), fa.FA_ERR_BAD_SHAPE),                  # causal, more queries than keys
    (dict(scale=float("nan")), fa.FA_ERR_BAD_SCALE),
    (dict(dtype=fa.FA_DTYPE_F32), fa.FA_ERR_UNSUPPORTED),
    (dict(o=A + SZ), fa.FA_ERR_ALIASING),
    (dict(lse=0), fa.FA_ERR_NULL_POINTER),
])
def test_split_validation_before_any_device_call(kw, expect):
    if expect == fa.FA_ERR_HIP and gpu_visible():
        pytest.skip("valid arguments would launch on fake addresses when a GPU is visible")
    assert split_call(**kw) == expect


# ---------------------------------------------------------------- fa_bwd
def test_split_static_validation_before_any_device_call():
    """fa_fwd_split_static checks its arguments and the scratch limit on the host."""
    p = 1 << 20
    ok = dict(q=p, k=p, v=p, o=8 * p, lse=16 * p, B=1, H=32, Nq=512, Nk=8192, D=128, causal=1, scale=0.1,
              n_splits=4, dtype=fa.FA_DTYPE_BF16, stream=None)

    def call(**kw):
        a = dict(ok, **kw)
        return fa.fa_fwd_split_static(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"], a["Nk"],
                                      a["D"], a["causal"], a["scale"], a["n_splits"], a["dtype"], a["stream"])

    assert call(q=None) == fa.FA_ERR_NULL_POINTER
    assert call(B=0) == fa.FA_ERR_BAD_SHAPE
    assert call(Nq=9000) == fa.FA_ERR_BAD_SHAPE  # Nq > Nk under the causal mask
    assert call(scale=float("nan")) == fa.FA_ERR_BAD_SCALE
    assert call(dtype=fa.FA_DTYPE_F32) == fa.FA_ERR_UNSUPPORTED
    # 4 ranges x 32 heads x 512 rows x 129 floats = 33.8 MB fits; 8 ranges (67.6 MB) does not
    st, sz, n = fa.fa_fwd_split_query(1, 32, 512, 8192, 128, 1, 8, fa.FA_DTYPE_BF16)
    assert st == fa.FA_OK and n == 8 and sz.workspace_bytes > fa.FA_STATIC_SCRATCH_BYTES
    assert call(n_splits=8) == fa.FA_ERR_WORKSPACE
    assert call(B=2) == fa.FA_ERR_WORKSPACE
    if not gpu_visible():
        # valid arguments within the limit reach the device check
        assert call() in (fa.FA_ERR_HIP, fa.FA_ERR_UNSUPPORTED)


def test_bwd_query_sizes():
    st, sz = fa.fa_bwd_query(2, 32, 4096, 128, 1, fa.FA_DTYPE_BF16)
    assert st == fa.FA_OK
    assert sz.q_bytes == sz.k_bytes == sz.v_bytes == sz.o_bytes == 2 * 32 * 4096 * 128 * 2
    assert sz.lse_bytes == 2 * 32 * 4096 * 4 and sz.workspace_bytes == 2 * sz.lse_bytes
    assert fa.fa_bwd_query(1, 1, 256, 64, 0, fa.FA_DTYPE_F32)[0] == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_bwd_query(1, 1, 256, 96, 0, fa.FA_DTYPE_BF16)[0] == fa.FA_OK
    assert fa.fa_bwd_query(1, 1, 256, 256, 0, fa.FA_DTYPE_BF16)[0] == fa.FA_OK
    assert fa.fa_bwd_query(1, 1, 256, 80, 0, fa.FA_DTYPE_BF16)[0] == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_bwd_query(1, 1, 0, 64, 0, fa.FA_DTYPE_BF16)[0] == fa.FA_ERR_BAD_SHAPE
    assert fa.fa_bwd_query(1, 1, 256, 64, 0, 9)[0] == fa.FA_ERR_BAD_DTYPE
    assert fa.lib().fa_bwd_query(1, 1, 256, 64, 0, 1, None) == fa.FA_ERR_NULL_POINTER


BN_ = 100 * 64 * 2 * 2  # bytes of one [1, 2, 100, 64] bf16 tensor
WSB = 2 * 2 * 100 * 4   # workspace of the default bwd_call


def bwd_call(q=A, k=A + SZ, v=A + 2 * SZ, o=A + 3 * SZ, do=A + 4 * SZ, lse=A + 5 * SZ, dq=A + 6 * SZ,
             dk=A + 7 * SZ, dv=A + 8 * SZ, ws=A + 9 * SZ, ws_bytes=WSB, B=1, H=2, N=100, D=64, causal=1,
             scale=0.125, dtype=fa.FA_DTYPE_BF16):
    return fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, ws_bytes, B, H, N, D, causal, scale, dtype, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(), fa.FA_ERR_HIP),                              # valid: fails only at the device query
    (dict(k=A, v=A, o=A), fa.FA_ERR_HIP),                 # read-only inputs may alias
    (dict(q=0), fa.FA_ERR_NULL_POINTER),
    (dict(do=0), fa.FA_ERR_NULL_POINTER),
    (dict(dv=0), fa.FA_ERR_NULL_POINTER),
    (dict(ws=0), fa.FA_ERR_NULL_POINTER),
    (dict(ws_bytes=WSB - 1), fa.FA_ERR_WORKSPACE),
    (dict(ws=A + 9 * SZ + 4), fa.FA_ERR_MISALIGNED),
    (dict(dk=A + 7 * SZ + 8), fa.FA_ERR_MISALIGNED),
    (dict(dq=A), fa.FA_ERR_ALIASING),                     # dq on top of q
    (dict(dk=A + 6 * SZ + BN_ - 16), fa.FA_ERR_ALIASING),  # dk starts in dq's last 16 bytes
    (dict(dk=A + 6 * SZ + BN_), fa.FA_ERR_HIP),           # dk right after dq: valid
    (dict(dv=A + 4 * SZ), fa.FA_ERR_ALIASING),            # dv on top of dout
    (dict(ws=A + 5 * SZ), fa.FA_ERR_ALIASING),            # workspace on top of lse
    (dict(ws=A + 8 * SZ + 16), fa.FA_ERR_ALIASING),       # workspace inside dv
    (dict(scale=float("nan")), fa.FA_ERR_BAD_SCALE),
    (dict(N=0), fa.FA_ERR_BAD_SHAPE),
    (dict(D=512), fa.FA_ERR_UNSUPPORTED),                 # the backward takes D in {64, 96, 128, 256}
    (dict(D=80), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=fa.FA_DTYPE_F32), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=4), fa.FA_ERR_BAD_DTYPE),
])
def test_bwd_validation_before_any_device_call(kw, expect):
    if expect == fa.FA_ERR_HIP and gpu_visible():
        pytest.skip("valid arguments would launch on fake addresses when a GPU is visible")
    assert bwd_call(**kw) == expect


# ---------------------------------------------------------------- fa_bwd_qk
def test_bwd_qk_query_sizes():
    st, sz = fa.fa_bwd_qk_query(2, 8, 500, 3000, 96, 1, fa.FA_DTYPE_F16)
    assert st == fa.FA_OK
    assert sz.q_bytes == sz.o_bytes == 2 * 8 * 500 * 96 * 2
    assert sz.k_bytes == sz.v_bytes == 2 * 8 * 3000 * 96 * 2
    assert sz.lse_bytes == 2 * 8 * 500 * 4 and sz.workspace_bytes == 2 * sz.lse_bytes
    # the square case gives fa_bwd_query's sizes
    a, b = fa.fa_bwd_qk_query(1, 4, 777, 777, 128, 0, fa.FA_DTYPE_BF16)[1], fa.fa_bwd_query(1, 4, 777, 128, 0,
                                                                                               fa.FA_DTYPE_BF16)[1]
    assert (a.q_bytes, a.k_bytes, a.lse_bytes, a.workspace_bytes) == (b.q_bytes, b.k_bytes, b.lse_bytes,
                                                                      b.workspace_bytes)
    # causal needs Nq <= Nk (queries are the last Nq positions); without the mask any Nq
    assert fa.fa_bwd_qk_query(1, 1, 300, 200, 64, 1, fa.FA_DTYPE_BF16)[0] == fa.FA_ERR_BAD_SHAPE
    assert fa.fa_bwd_qk_query(1, 1, 300, 200, 64, 0, fa.FA_DTYPE_BF16)[0] == fa.FA_OK
    assert fa.fa_bwd_qk_query(1, 1, 0, 200, 64, 0, fa.FA_DTYPE_BF16)[0] == fa.FA_ERR_BAD_SHAPE
    assert fa.fa_bwd_qk_query(1, 1, 100, 200, 256, 0, fa.FA_DTYPE_BF16)[0] == fa.FA_OK
    assert fa.fa_bwd_qk_query(1, 1, 100, 200, 512, 0, fa.FA_DTYPE_BF16)[0] == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_bwd_qk_query(1, 1, 100, 200, 64, 0, fa.FA_DTYPE_F32)[0] == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_bwd_qk_query(1, 1, 100, 200, 64, 0, 9)[0] == fa.FA_ERR_BAD_DTYPE
    assert fa.lib().fa_bwd_qk_query(1, 1, 100, 200, 64, 0, 1, None) == fa.FA_ERR_NULL_POINTER


QB_ = 60 * 64 * 2 * 2   # bytes of one [1, 2, 60, 64] bf16 tensor (q, o, dout, dq)
KB_ = 100 * 64 * 2 * 2  # bytes of one [1, 2, 100, 64] bf16 tensor (k, v, dk, dv)
WSQ = 2 * 2 * 60 * 4    # workspace of the default bwd_qk_call


def bwd_qk_call(q=A, k=A + SZ, v=A + 2 * SZ, o=A + 3 * SZ, do=A + 4 * SZ, lse=A + 5 * SZ, dq=A + 6 * SZ,
                dk=A + 7 * SZ, dv=A + 8 * SZ, ws=A + 9 * SZ, ws_bytes=WSQ, B=1, H=2, Nq=60, Nk=100, D=64, causal=1,
                scale=0.125, dtype=fa.FA_DTYPE_BF16):
    return fa.fa_bwd_qk(q, k, v, o, do, lse, dq, dk, dv, ws, ws_bytes, B, H, Nq, Nk, D, causal, scale, dtype, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(), fa.FA_ERR_HIP),                              # valid: fails only at the device query
    (dict(q=0), fa.FA_ERR_NULL_POINTER),
    (dict(ws_bytes=WSQ - 1), fa.FA_ERR_WORKSPACE),
    (dict(dk=A + 7 * SZ + 8), fa.FA_ERR_MISALIGNED),
    (dict(dk=A + 6 * SZ + QB_ - 16), fa.FA_ERR_ALIASING),  # dk starts in dq's last 16 bytes (dq has Nq rows)
    (dict(dk=A + 6 * SZ + QB_), fa.FA_ERR_HIP),           # dk right after dq: valid
    (dict(dv=A + 7 * SZ + KB_ - 16), fa.FA_ERR_ALIASING),  # dv starts in dk's last 16 bytes (dk has Nk rows)
    (dict(dv=A + 7 * SZ + KB_), fa.FA_ERR_HIP),
    (dict(ws=A + 5 * SZ + 2 * 60 * 4 - 16), fa.FA_ERR_ALIASING),  # workspace starts in lse's last 16 bytes
    (dict(Nq=101), fa.FA_ERR_BAD_SHAPE),                  # causal: Nq <= Nk
    (dict(Nq=101, causal=0, ws_bytes=2 * 2 * 101 * 4), fa.FA_ERR_HIP),
    (dict(scale=float("inf")), fa.FA_ERR_BAD_SCALE),
    (dict(D=512), fa.FA_ERR_UNSUPPORTED),
])
def test_bwd_qk_validation_before_any_device_call(kw, expect):
    if expect == fa.FA_ERR_HIP and gpu_visible():
        pytest.skip("valid arguments would launch on fake addresses when a GPU is visible")
    assert bwd_qk_call(**kw) == expect


# ---------------------------------------------------------------- fa_fwd_fp8
def test_fp8_query_sizes():
    st, sz = fa.fa_fwd_fp8_query(2, 32, 4096, 128, 0)
    assert st == fa.FA_OK
    assert sz.q_bytes == sz.k_bytes == sz.v_bytes == 2 * 32 * 4096 * 128
    assert sz.o_bytes == 2 * sz.q_bytes and sz.lse_bytes == 2 * 32 * 4096 * 4 and sz.workspace_bytes == 0
    assert fa.fa_fwd_fp8_query(2, 16, 4096, 256, 0)[0] == fa.FA_OK
    assert fa.fa_fwd_fp8_query(1, 1, 64, 96, 0)[0] == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_fwd_fp8_query(1, 1, 64, 512, 0)[0] == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_fwd_fp8_query(1, 1, 0, 64, 0)[0] == fa.FA_ERR_BAD_SHAPE
    assert fa.lib().fa_fwd_fp8_query(1, 1, 64, 64, 0, None) == fa.FA_ERR_NULL_POINTER


def fp8_call(q=A, qs=A + SZ, k=A + 2 * SZ, ks=A + 3 * SZ, v=A + 4 * SZ, vs=A + 5 * SZ, o=A + 6 * SZ,
             lse=A + 7 * SZ, B=1, H=2, N=100, D=64, causal=0, scale=0.125):
    return fa.fa_fwd_fp8(q, qs, k, ks, v, vs, o, lse, B, H, N, D, causal, scale, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(), fa.FA_ERR_HIP),                                # valid: fails only at the device query
    (dict(k=A, v=A, ks=A + SZ, vs=A + SZ), fa.FA_ERR_HIP),  # inputs may alias
    (dict(qs=0), fa.FA_ERR_NULL_POINTER),
    (dict(lse=0), fa.FA_ERR_NULL_POINTER),
    (dict(q=A + 8), fa.FA_ERR_MISALIGNED),
    (dict(vs=A + 5 * SZ + 2), fa.FA_ERR_MISALIGNED),
    (dict(vs=A + 5 * SZ + 4), fa.FA_ERR_HIP),               # scales need only 4-byte alignment
    (dict(o=A + 5 * SZ), fa.FA_ERR_ALIASING),               # o on top of v's scales
    (dict(lse=A + 6 * SZ + 16), fa.FA_ERR_ALIASING),        # lse inside o
    (dict(o=A + 4 * SZ + 100 * 64 * 2 - 16), fa.FA_ERR_ALIASING),  # o starts in v's last 16 bytes
    (dict(o=A + 4 * SZ + 100 * 64 * 2), fa.FA_ERR_HIP),     # o right after v: valid
    (dict(scale=float("nan")), fa.FA_ERR_BAD_SCALE),
    (dict(D=96), fa.FA_ERR_UNSUPPORTED),
    (dict(N=-1), fa.FA_ERR_BAD_SHAPE),
])
def test_fp8_validation_before_any_device_call(kw, expect):
    if expect == fa.FA_ERR_HIP and gpu_visible():
        pytest.skip("valid arguments would launch on fake addresses when a GPU is visible")
    assert fp8_call(**kw) == expect
