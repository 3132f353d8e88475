"""The C-ABI library loads without a GPU, exports every function include/svdq.h declares, and
rejects invalid arguments with the documented status before touching the HIP runtime."""
import os
import re

import pytest

from bit_post_quantized_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "svdq.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libsvdq.so is not built (run python -m bit_post_quantized_amd.build)")
    return binding.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert len(names) == 24, names
    assert set(names) == set(binding.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.svdq_abi_version() == 8
    assert lib.svdq_status_str(0) == b"ok"
    assert lib.svdq_status_str(2) == b"unsupported shape"
    assert lib.svdq_status_str(99) == b"unknown status"


# a fake, 16-byte aligned, never dereferenced address: every call below must fail validation
FAKE = 0x10000
ODD = 0x10008


def test_pack_weights_validation(lib):
    assert lib.svdq_pack_weights(FAKE, 100, 8, FAKE, FAKE, None) == binding.SVDQ_ESHAPE
    assert lib.svdq_pack_weights(FAKE, 0, 8, FAKE, FAKE, None) == binding.SVDQ_EINVAL
    assert lib.svdq_pack_weights(FAKE, 64, 0, FAKE, FAKE, None) == binding.SVDQ_EINVAL
    assert lib.svdq_pack_weights(None, 64, 8, FAKE, FAKE, None) == binding.SVDQ_EINVAL
    assert lib.svdq_pack_weights(ODD, 64, 8, FAKE, FAKE, None) == binding.SVDQ_EALIGN
    lib.svdq_pack_weights(FAKE, 100, 8, FAKE, FAKE, None)
    assert b"multiple of 64" in lib.svdq_last_error()


def test_pack_lowrank_validation(lib):
    f = lib.svdq_pack_lowrank
    assert f(FAKE, 100, 16, FAKE, None) == binding.SVDQ_ESHAPE   # K % 64
    assert f(FAKE, 128, 24, FAKE, None) == binding.SVDQ_ESHAPE   # r % 16
    assert f(FAKE, 128, 144, FAKE, None) == binding.SVDQ_ESHAPE  # r > 128
    assert f(FAKE, 128, 0, FAKE, None) == binding.SVDQ_ESHAPE    # nothing to relay out
    assert f(None, 128, 16, FAKE, None) == binding.SVDQ_EINVAL
    assert f(FAKE, 128, 16, None, None) == binding.SVDQ_EINVAL


def test_pack_lowrank_up_validation(lib):
    f = lib.svdq_pack_lowrank_up
    assert f(FAKE, 24, 128, FAKE, None) == binding.SVDQ_ESHAPE       # r % 16
    assert f(FAKE, 144, 128, FAKE, None) == binding.SVDQ_ESHAPE      # r > 128
    assert f(FAKE, 0, 128, FAKE, None) == binding.SVDQ_ESHAPE        # nothing to relay out
    assert f(FAKE, 16, 0, FAKE, None) == binding.SVDQ_EINVAL
    assert f(FAKE, 16, (1 << 24) + 1, FAKE, None) == binding.SVDQ_ESHAPE
    assert f(None, 16, 128, FAKE, None) == binding.SVDQ_EINVAL
    assert f(FAKE, 16, 128, None, None) == binding.SVDQ_EINVAL


def test_quantize_act_validation(lib):
    f = lib.svdq_quantize_act
    assert f(FAKE, FAKE, FAKE, 4, 128, 20, FAKE, FAKE, FAKE, None) == binding.SVDQ_ESHAPE
    assert f(FAKE, FAKE, FAKE, 4, 128, 144, FAKE, FAKE, FAKE, None) == binding.SVDQ_ESHAPE
    assert f(FAKE, FAKE, FAKE, 4, 96, 16, FAKE, FAKE, FAKE, None) == binding.SVDQ_ESHAPE
    assert f(FAKE, FAKE, FAKE, -1, 128, 16, FAKE, FAKE, FAKE, None) == binding.SVDQ_EINVAL
    assert f(FAKE, FAKE, None, 4, 128, 16, FAKE, FAKE, FAKE, None) == binding.SVDQ_EINVAL
    assert f(FAKE, FAKE, FAKE, 4, 128, 16, FAKE, FAKE, None, None) == binding.SVDQ_EINVAL
    assert f(ODD, FAKE, FAKE, 4, 128, 16, FAKE, FAKE, FAKE, None) == binding.SVDQ_EALIGN
    # M = 0 is valid and enqueues nothing (no HIP call is made)
    assert f(FAKE, FAKE, FAKE, 0, 128, 16, FAKE, FAKE, FAKE, None) == binding.SVDQ_OK


def test_gemm_validation(lib):
    g = lib.svdq_w4a4_gemm
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None]
    assert g(*args, 8, 8, 100, 0, FAKE, 0, None) == binding.SVDQ_ESHAPE
    assert g(*args, 8, 0, 128, 0, FAKE, 0, None) == binding.SVDQ_EINVAL
    assert g(*args, 8, 8, 128, 0, FAKE, 7, None) == binding.SVDQ_EINVAL  # bad out_dtype
    assert g(*args, 8, 8, 128, 24, FAKE, 0, None) == binding.SVDQ_ESHAPE
    assert g(*args, 8, 8, 64 * 65536, 0, FAKE, 0, None) == binding.SVDQ_ESHAPE  # K / 64 > 65535
    # N beyond 2^24: 32-bit row offsets inside an output tile would wrap
    assert g(*args, 8, (1 << 24) + 1, 128, 0, FAKE, 0, None) == binding.SVDQ_ESHAPE
    assert b"2^24" in lib.svdq_last_error()
    assert lib.svdq_w4a4_gemm_e3m2(*args, 8, (1 << 24) + 1, 128, 0, FAKE, 0, None) == binding.SVDQ_ESHAPE
    assert lib.svdq_w4a8_gemm(*args, 8, (1 << 24) + 1, 128, 0, FAKE, 0, None) == binding.SVDQ_ESHAPE
    assert lib.svdq_w4a4_partials(FAKE, FAKE, 8, (1 << 24) + 1, 128, FAKE, None) == binding.SVDQ_ESHAPE
    assert g(FAKE, FAKE, None, FAKE, FAKE, FAKE, None, 8, 8, 128, 16, FAKE, 0, None) == binding.SVDQ_EINVAL
    assert g(*args, 8, 8, 128, 0, ODD, 0, None) == binding.SVDQ_EALIGN
    assert g(*args, 0, 8, 128, 16, FAKE, 1, None) == binding.SVDQ_OK
    p = lib.svdq_w4a4_partials
    assert p(FAKE, FAKE, 8, 8, 96, FAKE, None) == binding.SVDQ_ESHAPE
    assert p(FAKE, FAKE, 8, 8, 128, None, None) == binding.SVDQ_EINVAL


def test_e3m2_container_size(lib):
    assert lib.svdq_e3m2_bytes(4608, 3072) == 144 * 48 * 1536
    assert lib.svdq_e3m2_bytes(33, 128) == 2 * 2 * 1536
    assert lib.svdq_e3m2_bytes(0, 128) == 0 and lib.svdq_e3m2_bytes(8, 100) == 0


def test_e3m2_entry_points_validate_like_their_nibble_twins(lib):
    assert lib.svdq_pack_weights_e3m2(FAKE, 100, 8, FAKE, FAKE, None) == binding.SVDQ_ESHAPE
    assert lib.svdq_pack_weights_e3m2(ODD, 64, 8, FAKE, FAKE, None) == binding.SVDQ_EALIGN
    assert b"svdq_pack_weights_e3m2" not in lib.svdq_last_error()  # validation message, not HIP
    f = lib.svdq_quantize_act_e3m2
    assert f(FAKE, FAKE, FAKE, 4, 128, 20, FAKE, FAKE, FAKE, None) == binding.SVDQ_ESHAPE
    assert f(FAKE, FAKE, None, 4, 128, 16, FAKE, FAKE, FAKE, None) == binding.SVDQ_EINVAL
    assert f(FAKE, FAKE, FAKE, 0, 128, 16, FAKE, FAKE, FAKE, None) == binding.SVDQ_OK
    g = lib.svdq_w4a4_gemm_e3m2
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None]
    assert g(*args, 8, 8, 100, 0, FAKE, 0, None) == binding.SVDQ_ESHAPE
    assert g(*args, 8, 8, 128, 0, FAKE, 7, None) == binding.SVDQ_EINVAL
    assert g(*args, 8, 8, 128, 0, ODD, 0, None) == binding.SVDQ_EALIGN
    assert g(*args, 0, 8, 128, 16, FAKE, 1, None) == binding.SVDQ_OK
    p = lib.svdq_w4a4_partials_e3m2
    assert p(FAKE, FAKE, 8, 8, 96, FAKE, None) == binding.SVDQ_ESHAPE
    assert p(FAKE, FAKE, 8, 8, 128, None, None) == binding.SVDQ_EINVAL


def test_w4a8_entry_points_validate_like_their_w4a4_twins(lib):
    f = lib.svdq_quantize_act_a8
    assert f(FAKE, FAKE, FAKE, 4, 128, 20, FAKE, FAKE, FAKE, None) == binding.SVDQ_ESHAPE
    assert f(FAKE, FAKE, FAKE, 4, 96, 16, FAKE, FAKE, FAKE, None) == binding.SVDQ_ESHAPE
    assert f(FAKE, FAKE, None, 4, 128, 16, FAKE, FAKE, FAKE, None) == binding.SVDQ_EINVAL
    assert f(FAKE, FAKE, FAKE, 4, 128, 16, ODD, FAKE, FAKE, None) == binding.SVDQ_EALIGN
    assert f(FAKE, FAKE, FAKE, 0, 128, 16, FAKE, FAKE, FAKE, None) == binding.SVDQ_OK
    g = lib.svdq_w4a8_gemm
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None]
    assert g(*args, 8, 8, 100, 0, FAKE, 0, None) == binding.SVDQ_ESHAPE
    assert g(*args, 8, 0, 128, 0, FAKE, 0, None) == binding.SVDQ_EINVAL
    assert g(*args, 8, 8, 128, 0, FAKE, 7, None) == binding.SVDQ_EINVAL
    assert g(ODD, FAKE, FAKE, FAKE, FAKE, FAKE, None, 8, 8, 128, 0, FAKE, 0, None) == binding.SVDQ_EALIGN
    assert g(*args, 0, 8, 128, 16, FAKE, 1, None) == binding.SVDQ_OK
    p = lib.svdq_w4a8_partials
    assert p(FAKE, FAKE, 8, 8, 96, FAKE, None) == binding.SVDQ_ESHAPE
    assert p(FAKE, FAKE, 8, 8, 128, None, None) == binding.SVDQ_EINVAL
    lib.svdq_w4a8_partials(FAKE, FAKE, 8, 8, 96, FAKE, None)
    assert b"multiple of 64" in lib.svdq_last_error()


def test_kv_validation(lib):
    q = lib.kv_int8_quant
    assert lib.kv_int8_workspace_bytes(0, 4096) == 0
    # the larger of the two schedules' needs: lo/hi partials of 160 chunks of 64 tokens
    assert lib.kv_int8_workspace_bytes(10240, 4096) == 2 * 160 * 4096 * 4
    assert q(FAKE, 16, 12, FAKE, FAKE, FAKE, FAKE, None) == binding.SVDQ_ESHAPE
    assert q(FAKE, -1, 16, FAKE, FAKE, FAKE, FAKE, None) == binding.SVDQ_EINVAL
    assert q(FAKE, 16, 16, FAKE, FAKE, FAKE, None, None) == binding.SVDQ_EINVAL
    assert q(FAKE, 16, 16, FAKE, ODD, FAKE, FAKE, None) == binding.SVDQ_EALIGN
    assert q(FAKE, 0, 16, FAKE, FAKE, FAKE, None, None) == binding.SVDQ_OK
    d = lib.kv_int8_dequant
    assert d(FAKE, FAKE, FAKE, 16, 0, FAKE, None) == binding.SVDQ_EINVAL
    assert d(FAKE, FAKE, FAKE, 16, 16, ODD, None) == binding.SVDQ_EALIGN
    # the dequantization's grid: at most 65535 blocks of 32 tokens, for both calls
    assert q(FAKE, 65535 * 32 + 1, 8, FAKE, FAKE, FAKE, FAKE, None) == binding.SVDQ_ESHAPE
    assert d(FAKE, FAKE, FAKE, 65535 * 32 + 1, 8, FAKE, None) == binding.SVDQ_ESHAPE
    assert b"2097120" in lib.svdq_last_error()
    # small token counts: the paired single pass's two regions of published part ranges
    # (32 slabs x 8 parts x 256 tagged 8-byte words each) exceed one 64-token chunk's partials
    assert lib.kv_int8_workspace_bytes(64, 4096) == 2 * 32 * 8 * 256 * 8


def test_kv_pair_validation(lib):
    p = lib.kv_int8_quant_pair
    f8 = [FAKE] * 8
    assert p(FAKE, FAKE, 16, 12, *f8[:6], FAKE, None) == binding.SVDQ_ESHAPE
    assert p(FAKE, FAKE, -1, 16, *f8[:6], FAKE, None) == binding.SVDQ_EINVAL
    assert p(FAKE, None, 16, 16, *f8[:6], FAKE, None) == binding.SVDQ_EINVAL
    assert p(FAKE, FAKE, 16, 16, *f8[:6], None, None) == binding.SVDQ_EINVAL
    assert p(FAKE, FAKE, 16, 16, FAKE, FAKE, FAKE, FAKE, ODD, FAKE, FAKE, None) == \
        binding.SVDQ_EALIGN
    assert p(FAKE, FAKE, 65535 * 32 + 1, 8, *f8[:6], FAKE, None) == binding.SVDQ_ESHAPE
    assert p(FAKE, FAKE, 0, 16, *f8[:6], None, None) == binding.SVDQ_OK


def test_kv_pair_noalloc_validation(lib):
    p = lib.kv_int8_quant_pair_noalloc
    f6 = [FAKE] * 6
    assert p(FAKE, FAKE, 16, 12, *f6, None) == binding.SVDQ_ESHAPE
    assert p(FAKE, None, 16, 16, *f6, None) == binding.SVDQ_EINVAL
    assert p(FAKE, FAKE, 16, 16, FAKE, FAKE, ODD, FAKE, FAKE, FAKE, None) == binding.SVDQ_EALIGN
    assert p(FAKE, FAKE, 0, 16, *f6, None) == binding.SVDQ_OK
    # beyond the 16 MiB of device scratch it holds: rejected before any HIP call
    assert lib.kv_int8_workspace_bytes(65536, 4096) > 16 << 20
    assert p(FAKE, FAKE, 65536, 4096, *f6, None) == binding.SVDQ_ESHAPE
    assert b"holds 16777216" in lib.svdq_last_error()
    assert lib.kv_int8_workspace_bytes(10240, 4096) <= 16 << 20


def test_kv_attention_validation(lib):
    assert lib.kv_int8_attention_workspace_bytes(1, 10240, 32, 128) == 32 * 40 * 130 * 4
    assert lib.kv_int8_attention_workspace_bytes(2, 257, 4, 64) == 2 * 4 * 2 * 66 * 4
    assert lib.kv_int8_attention_workspace_bytes(0, 16, 4, 64) == 0
    a = lib.kv_int8_attention
    p7 = [FAKE] * 7
    assert a(*p7, 1, 16, 4, 96, 0.1, FAKE, FAKE, None) == binding.SVDQ_ESHAPE     # dim
    assert a(*p7, 0, 16, 4, 64, 0.1, FAKE, FAKE, None) == binding.SVDQ_EINVAL     # nq
    assert a(*p7, 1, 0, 4, 64, 0.1, FAKE, FAKE, None) == binding.SVDQ_EINVAL      # no tokens
    assert a(*p7, 1, 16, 4, 64, 0.1, FAKE, None, None) == binding.SVDQ_EINVAL     # workspace
    assert a(*p7, 1, 1048577, 1, 64, 0.1, FAKE, FAKE, None) == binding.SVDQ_ESHAPE  # 4097 chunks
    assert a(ODD, *p7[1:], 1, 16, 4, 64, 0.1, FAKE, FAKE, None) == binding.SVDQ_EALIGN
    assert a(*p7, 1, 16, 4, 64, float("nan"), FAKE, FAKE, None) == binding.SVDQ_EINVAL
    assert b"sm_scale" in lib.svdq_last_error()


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(RuntimeError, match="not found"):
        binding.load(str(tmp_path / "missing.so"))


def test_validation_paths_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    """abi.cpp built for the host with AddressSanitizer and UndefinedBehaviorSanitizer and
    linked with the library's kernel objects; tests/abi_sanitize_main.cpp calls every entry
    point with invalid, misaligned, out-of-range and overflowing arguments (no call reaches a
    kernel launch, so no GPU is needed) and checks the statuses; any sanitizer report fails."""
    import glob
    import shutil
    import subprocess

    from bit_post_quantized_amd import build

    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no g++")
    objs = sorted(o for o in glob.glob(os.path.join(build.OBJDIR, "*.o"))
                  if os.path.basename(o) not in ("abi.o", "peaks.o"))
    if not objs:
        pytest.fail("kernel objects are not built (run python -m bit_post_quantized_amd.build)")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    sanitize = ["-fsanitize=" + "address,undefined", "-fno-sanitize-recover=all",
                "-fno-omit-frame-pointer"]
    common = ["-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", f"-I{rocm}/include",
              f"-I{os.path.join(ROOT, 'include')}", f"-I{build.CSRC}", *sanitize]
    abi_o, main_o, exe = (str(tmp_path / n) for n in ("abi.o", "main.o", "abi_check"))
    for src, obj in ((os.path.join(build.CSRC, "abi.cpp"), abi_o),
                     (os.path.join(ROOT, "tests", "abi_sanitize_main.cpp"), main_o)):
        res = subprocess.run([gxx, *common, "-c", src, "-o", obj], capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-3000:]
    res = subprocess.run([gxx, *sanitize, main_o, abi_o, *objs, f"-L{rocm}/lib", "-lamdhip64",
                          f"-Wl,-rpath,{rocm}/lib", "-o", exe], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    report = run.stdout + run.stderr
    assert run.returncode == 0, report[-3000:]
    assert "runtime error" not in report and "AddressSanitizer" not in report, report[-3000:]
    assert "all ABI validation checks passed" in run.stdout
