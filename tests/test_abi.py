"""The C-ABI library loads, exports every function include/kda.h declares (and the
measurement library every function include/kda_probe.h declares, the product
library none of them), and the host-side validation answers without a GPU (no
call here reaches the device)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]

import kimi_delta_attention_conv_amd as kda  # noqa: E402
from kimi_delta_attention_conv_amd import probe as kprobe  # noqa: E402


def declared_functions(header=None):
    names = set()
    for path in HEADERS:
        if header is not None and os.path.basename(path) != header:
            continue
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names.update(re.findall(r"^\s*(?:const\s+)?[\w\*\s]+?\b(kda_\w+)\s*\(", text,
                                flags=re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.LIB_PATH):
        pytest.skip("libkda.so not built (run __graft_entry__.build())")
    return kda.load_library()


@pytest.fixture(scope="module")
def plib():
    if not os.path.exists(kprobe.LIB_PATH):
        pytest.skip("libkda_probe.so not built (run __graft_entry__.build())")
    return kprobe.load_probe_library()


def test_header_declares_the_boundary():
    names = declared_functions("kda.h")
    for n in ("kda_prepare", "kda_decode", "kda_verify", "kda_device_errors", "kda_destroy",
              "kda_status_string", "kda_last_hip_error", "kda_linear", "kda_in_proj",
              "kda_o_proj", "kda_linear_workspace_bytes", "kda_linear_noalloc",
              "kda_noalloc_scratch_bytes"):
        assert n in names, n
    probes = declared_functions("kda_probe.h")
    for n in ("kda_probe_copy", "kda_probe_write", "kda_probe_read", "kda_probe_sink_floats",
              "kda_probe_state_stream", "kda_probe_copy_runs", "kda_probe_write_runs"):
        assert n in probes, n


def _exported(path):
    out = subprocess.run(["nm", "-D", "--defined-only", path], check=True,
                         capture_output=True, text=True).stdout
    return set(line.split()[-1] for line in out.splitlines() if line.strip())


def test_every_declared_symbol_is_exported(lib, plib):
    exported = _exported(kda.LIB_PATH)
    for n in declared_functions("kda.h"):
        assert n in exported, f"{n} declared in kda.h but not exported"
        assert getattr(lib, n) is not None
    probe_exported = _exported(kprobe.LIB_PATH)
    for n in declared_functions("kda_probe.h"):
        assert n in probe_exported, f"{n} declared in kda_probe.h but not exported"
        assert n not in exported, f"{n} (measurement only) exported by the product library"
        assert getattr(plib, n) is not None


def test_status_strings(lib):
    seen = set()
    for code in range(0, -9, -1):
        s = kda.kda_status_string(code)
        assert s and s not in seen
        seen.add(s)
    assert lib.kda_last_hip_error() == b""


def _weights(**kw):
    fake = 0x10000  # never dereferenced: validation fails before any HIP call
    base = dict(heads=2, conv_width=4, conv_weight=fake, conv_bias=None, f_b=fake, A_log=fake,
                dt_bias=fake, norm_weight=fake, norm_head_stride=0, gate_lower_bound=-5.0,
                norm_eps=1e-6, l2_eps=1e-6)
    base.update(kw)
    return kda.KdaWeights(**base)


def _caches(**kw):
    D = 256
    base = dict(conv=0x20000, conv_slot_stride=9 * D, conv_dim_stride=3, conv_pos_stride=1,
                state=0x40000, state_slot_stride=2 * 128 * 128, num_slots=4)
    base.update(kw)
    return kda.KdaCaches(**base)


@pytest.mark.parametrize("weights,caches,status", [
    (None, _caches(), -1),
    (_weights(f_b=None), _caches(), -1),
    (_weights(), _caches(state=None), -1),
    (_weights(heads=0), _caches(), -2),
    (_weights(conv_width=3), _caches(), -4),
    (_weights(norm_head_stride=64), _caches(), -2),
    (_weights(norm_eps=float("nan")), _caches(), -2),
    (_weights(l2_eps=-1.0), _caches(), -2),
    (_weights(l2_eps=0.0), _caches(), -2),
    (_weights(norm_eps=0.0), _caches(), -2),
    (_weights(), _caches(check_distinct=2), -2),
    (_weights(), _caches(check_distinct=-1), -2),
    (_weights(rounding=2), _caches(), -2),
    (_weights(rounding=-1), _caches(), -2),
    (_weights(), _caches(num_slots=0), -2),
    (_weights(), _caches(state_slot_stride=128 * 128), -2),
    (_weights(), _caches(conv_slot_stride=100), -2),
    (_weights(), _caches(conv_dim_stride=-3), -2),
    (_weights(), _caches(state=0x40004), -3),
    (_weights(), _caches(state_slot_stride=2 * 128 * 128 + 2), -3),
    (_weights(A_log=0x10002), _caches(), -3),
    (_weights(dt_bias=0x10001, dt_bias_dtype=1), _caches(), -3),
    (_weights(norm_weight=0x10002, norm_weight_dtype=0), _caches(), -3),
    (_weights(A_log_dtype=2), _caches(), -2),
    (_weights(norm_weight_dtype=-1), _caches(), -2),
], ids=lambda v: str(v) if isinstance(v, int) else "")
def test_prepare_validation_without_gpu(lib, weights, caches, status):
    h = ctypes.c_void_p()
    wp = None if weights is None else ctypes.byref(weights)
    got = lib.kda_prepare(wp, ctypes.byref(caches), None, ctypes.byref(h))
    assert got == status
    assert h.value is None


def test_probe_validation_without_gpu(plib):
    lib = plib
    assert lib.kda_probe_copy(None, 0x1000, 16, None) == -1
    assert lib.kda_probe_write(0x1008, 16, 1.0, None) == -3
    assert lib.kda_probe_read(0x1000, 24, 0x2000, None) == -3
    assert lib.kda_probe_copy_runs(0x1000, None, 16, None) == -1
    assert lib.kda_probe_write_runs(0x1000, 20, 1.0, None) == -3
    assert lib.kda_probe_sink_floats() > 0


def test_state_stream_probe_validation_without_gpu(plib):
    lib = plib
    fake = 0x10000   # never dereferenced: validation fails before any HIP call
    tile = 128 * 128
    call = lambda state=fake, stride=12 * tile, slots_n=16, slots=fake, rs=8, acc=fake, R=4, L=8, \
        H=12, opt=0: lib.kda_probe_state_stream(state, stride, slots_n, slots, rs, acc, R, L, H,
                                                opt, None)
    assert call(opt=4) == -2
    assert call(opt=-1) == -2
    assert call(L=0) == -2
    assert call(L=9) == -2
    assert call(H=0) == -2
    assert call(H=4097) == -2
    assert call(R=-1) == -2
    assert call(slots_n=0) == -2
    assert call(rs=7) == -2
    assert call(stride=12 * tile - 4) == -2
    assert call(R=1 << 20, H=4096) == -2
    assert call(R=0) == 0                  # nothing to do, nothing enqueued
    assert call(state=None) == -1
    assert call(slots=None) == -1
    assert call(state=fake + 8) == -3
    assert call(stride=12 * tile + 2) == -3
    assert call(slots=fake + 2) == -3
    assert call(acc=fake + 1) == -3


def test_linear_validation_without_gpu(lib):
    fake = 0x10000   # never dereferenced: validation fails before any HIP call
    for M, N, K, status in [(-1, 16, 64, -2), (4, 0, 64, -2), (4, 16, 60, -2), (4, 16, 0, -2),
                            ((1 << 20) + 1, 16, 64, -2), (1 << 20, 1 << 24, 64, -2)]:
        assert lib.kda_linear(fake, max(K, 8), fake, fake, max(N, 1), M, N, K, None, 0,
                              None) == status, (M, N, K)
    assert lib.kda_linear(None, 64, fake, fake, 16, 4, 16, 64, None, 0, None) == -1
    assert lib.kda_linear(fake + 8, 64, fake, fake, 16, 4, 16, 64, None, 0, None) == -3
    assert lib.kda_linear(fake, 64, fake, fake, 16, 4, 16, 64, fake + 4, 1024, None) == -3
    assert lib.kda_in_proj(fake, 64, fake, fake, 16, 4, 64, 0, None, 0, None) == -2
    assert lib.kda_o_proj(fake, 64, fake, fake, 16, 4, 5000, 64, None, 0, None) == -2


def test_noalloc_validation_without_gpu(lib):
    """kda_linear_noalloc validates like kda_linear and rejects shapes whose K split
    needs more than the static scratch buffer, all before any HIP call."""
    fake = 0x10000
    cap = lib.kda_noalloc_scratch_bytes()
    assert cap == 32 * 1024 * 1024
    for M, N, K, status in [(-1, 16, 64, -2), (4, 0, 64, -2), (4, 16, 60, -2),
                            ((1 << 20) + 1, 16, 64, -2), (1 << 20, 1 << 24, 64, -2)]:
        assert lib.kda_linear_noalloc(fake, max(K, 8), fake, fake, max(N, 1), M, N, K,
                                      None) == status, (M, N, K)
    assert lib.kda_linear_noalloc(None, 64, fake, fake, 16, 4, 16, 64, None) == -1
    assert lib.kda_linear_noalloc(fake + 8, 64, fake, fake, 16, 4, 16, 64, None) == -3
    assert lib.kda_linear_noalloc(fake, 64, fake, fake, 16, 0, 16, 64, None) == 0
    # 256 rows of a 40,000-wide projection split K over 4 x 313 tiles: 164 MB
    big = lib.kda_linear_workspace_bytes(256, 40000, 4096)
    assert big > cap
    assert lib.kda_linear_noalloc(fake, 4096, fake, fake, 40000, 256, 40000, 4096, None) == -8
    # in_proj up to 256 rows fits
    assert lib.kda_linear_workspace_bytes(256, 6284, 7168) <= cap


def test_linear_workspace_bytes(lib):
    # 33..256 rows, K >= 4096 and a multiple of 256: 4 K slices of fp32 tiles of
    # 64, 128 or 256 rows x 128 columns
    assert lib.kda_linear_workspace_bytes(64, 6284, 7168) == 4 * 50 * 64 * 128 * 4
    assert lib.kda_linear_workspace_bytes(33, 128, 4096) == 4 * 64 * 128 * 4
    assert lib.kda_linear_workspace_bytes(65, 6284, 7168) == 4 * 50 * 128 * 128 * 4
    assert lib.kda_linear_workspace_bytes(256, 6284, 7168) == 4 * 50 * 256 * 128 * 4
    for M, N, K in [(32, 6284, 7168), (257, 6284, 7168), (64, 7168, 1536), (64, 100, 4160),
                    (0, 10, 4096), (64, 0, 4096), (64, 10, 4100)]:
        assert lib.kda_linear_workspace_bytes(M, N, K) == 0, (M, N, K)


def test_calls_on_null_handle(lib):
    n = ctypes.c_int32(7)
    assert lib.kda_decode(None, 0x1000, 1154, 1, 0x2000, 0x3000, None) == -1
    assert lib.kda_verify(None, 0x1000, 1154, 1, 4, 0x2000, 4, 0x4000, 0x3000, None) == -1
    assert lib.kda_device_errors(None, ctypes.byref(n), None) == -1
    assert n.value == 7
    assert lib.kda_destroy(None) == 0


def test_binding_fails_loudly_without_library(tmp_path):
    saved = kda._lib
    try:
        kda._lib = None
        with pytest.raises(ImportError):
            kda.load_library(str(tmp_path / "missing.so"))
    finally:
        kda._lib = saved


def test_headers_are_plain_c_and_a_c_program_links(lib, tmp_path):
    """The boundary is a C ABI: both headers compile as pedantic C99, and a C program
    links against the library and calls its host-only entry points (no GPU call)."""
    inc = os.path.join(ROOT, "include")
    for path in HEADERS:
        subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                        "-fsyntax-only", "-x", "c", path], check=True)
    src = tmp_path / "abi.c"
    src.write_text(
        '#include <string.h>\n#include "kda.h"\n#include "kda_probe.h"\n'
        "int main(void) {\n"
        "    kda_handle h = 0;\n"
        "    if (kda_linear_workspace_bytes(64, 6284, 7168) != 4u * 50 * 64 * 128 * 4) return 1;\n"
        "    if (kda_linear_workspace_bytes(512, 6284, 7168) != 0) return 2;\n"
        "    if (strcmp(kda_status_string(KDA_OK), \"ok\") != 0) return 3;\n"
        "    if (kda_destroy(h) != KDA_OK) return 4;\n"
        "    if (kda_decode(h, 0, 0, 1, 0, 0, 0) != KDA_ERR_NULL) return 5;\n"
        "    if (kda_noalloc_scratch_bytes() != KDA_NOALLOC_SCRATCH_BYTES) return 6;\n"
        "    if (kda_linear_noalloc(0, 64, 0, 0, 16, 4, 16, 64, 0) != KDA_ERR_NULL) return 7;\n"
        "    return 0;\n}\n")
    exe = tmp_path / "abi"
    libdir = os.path.dirname(kda.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I" + inc, str(src),
                    "-L" + libdir, "-l:" + os.path.basename(kda.LIB_PATH),
                    "-Wl,-rpath," + libdir, "-o", str(exe)], check=True)
    assert subprocess.run([str(exe)]).returncode == 0
