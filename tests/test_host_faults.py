"""The host layer's error paths on the CPU.

* A HIP failure at launch time comes back as TT_ERR_HIP from every entry point:
  forced by TT_INJECT_HIP_ERROR (validation runs, nothing is launched), and the
  real failure of a launch on a machine without a GPU.
* The library's host code (validation, planning, dispatch) and the oracle, built
  with AddressSanitizer and UndefinedBehaviorSanitizer for the host side only,
  run the ABI tests and the oracle pins without a report.

Every call here either fails validation or cannot launch: no kernel ever runs.
"""
import glob
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# calls with valid arguments and fake device pointers: each must return TT_ERR_HIP (7)
CALLS = textwrap.dedent("""
    import ctypes, sys
    sys.path.insert(0, {tests!r})
    from attention_eq_block_amd import _lib
    from attention_eq_block_amd._lib import TT_F32, KvAppendParams
    from test_abi import attn_ok, unmask_ok, nll_ok, FAKE
    L = _lib.lib()
    out = {{}}
    p = attn_ok()
    nb = L.tt_block_attn_workspace_bytes(ctypes.byref(p))
    out["tt_block_attn"] = L.tt_block_attn(ctypes.byref(p), FAKE, nb, None)
    out["tt_block_attn f32"] = L.tt_block_attn(ctypes.byref(attn_ok(dtype=TT_F32, o_dtype=TT_F32)), None, 0, None)
    out["tt_block_attn_noalloc"] = L.tt_block_attn_noalloc(ctypes.byref(p), None)
    out["tt_lse_merge"] = L.tt_lse_merge(2, FAKE, FAKE, 2, 16, 32, 128, FAKE, 0, FAKE, None)
    u = unmask_ok()
    nb = L.tt_conf_unmask_workspace_bytes(ctypes.byref(u))
    out["tt_conf_unmask"] = L.tt_conf_unmask(ctypes.byref(u), FAKE, nb, None)
    q = nll_ok()
    nb = L.tt_masked_nll_workspace_bytes(ctypes.byref(q))
    out["tt_masked_nll"] = L.tt_masked_nll(ctypes.byref(q), FAKE, nb, None)
    k = KvAppendParams()
    k.dtype, k.B, k.S, k.Hkv, k.head_dim = 1, 2, 16, 2, 128
    k.Kctx = k.Vctx = k.page_table = k.ctx_len = k.Knew = k.Vnew = k.status = FAKE
    k.page_size, k.num_pages, k.max_pages = 16, 64, 8
    k.new_stride_h, k.new_stride_s, k.new_stride_b = 128, 256, 4096
    out["tt_kv_append"] = L.tt_kv_append(ctypes.byref(k), None)
    print(out)
    sys.exit(0 if all(v == 7 for v in out.values()) else 1)
""").format(tests=os.path.join(ROOT, "tests"))


def gpu_visible() -> bool:
    import torch
    return torch.cuda.device_count() > 0  # counts devices without initialising one


def run_calls(env_extra):
    env = dict(os.environ, **env_extra)
    r = subprocess.run([sys.executable, "-c", CALLS], cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    return r.returncode, r.stdout + r.stderr


@pytest.mark.skipif(gpu_visible(), reason="these calls carry fake device pointers: never run them where a GPU "
                                          "could execute a launch")
def test_injected_hip_error_from_every_entry_point():
    rc, out = run_calls({"TT_INJECT_HIP_ERROR": "1"})
    assert rc == 0, out


@pytest.mark.skipif(gpu_visible(), reason="needs a machine without a GPU, where every launch fails")
def test_launch_failure_without_a_gpu_is_tt_err_hip():
    rc, out = run_calls({"TT_INJECT_HIP_ERROR": "0"})
    assert rc == 0, out


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.skipif(_asan_runtime() is None, reason="no clang AddressSanitizer runtime in /opt/rocm/llvm")
def test_host_code_under_address_and_undefined_behavior_sanitizers(tmp_path):
    sys.path.insert(0, ROOT)
    from attention_eq_block_amd import build as hip_build

    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    lib = hip_build.build(out=str(tmp_path / "libtwotower_attn_san.so"), extra=san,
                          link_extra=["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                                      "-shared-libsan"])
    oracle_lib = str(tmp_path / "libtt_oracle_san.so")
    clang = "/opt/rocm/llvm/bin/clang"
    subprocess.run([clang, "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-shared-libsan", os.path.join(ROOT, "oracle", "tt_oracle.c"),
                    "-o", oracle_lib, "-lm"], check=True, capture_output=True)
    logs = tmp_path / "san"
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(),
               ASAN_OPTIONS=f"detect_leaks=0:halt_on_error=1:log_path={logs}",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={logs}", TT_LIBRARY=lib,
               TT_ORACLE_LIBRARY=oracle_lib, TT_INJECT_HIP_ERROR="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_abi.py", "tests/test_oracle_pins.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    reports = "".join(open(f).read() for f in glob.glob(str(logs) + "*"))
    assert not reports, reports[:4000]
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
