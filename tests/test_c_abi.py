"""The C-ABI driven from plain C (tests/c/kda_c_caller.c), without Python in
between: host-side checks on the CPU, and one decode call on the GPU whose
output and state match the oracle."""
import os
import subprocess

import numpy as np
import pytest

from hybrid_linear_attention_rule_amd import kda
from kda_inputs import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c", "kda_c_caller.c")
LIBDIR = os.path.dirname(kda.LIB_PATH)


def build_caller(tmp_path):
    if not os.path.exists(kda.LIB_PATH):
        pytest.skip("libkda.so is not built")
    exe = str(tmp_path / "kda_c_caller")
    subprocess.run(["gcc", "-O1", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", "-o", exe,
                    SRC, "-L", LIBDIR, "-lkda", "-L", "/opt/rocm/lib", "-lamdhip64",
                    f"-Wl,-rpath,{LIBDIR}", "-Wl,-rpath,/opt/rocm/lib"], check=True)
    return exe


def test_c_caller_host_checks(tmp_path):
    exe = build_caller(tmp_path)
    r = subprocess.run([exe, "host"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr


@pytest.mark.gpu
def test_c_caller_decode_matches_oracle(tmp_path):
    from gpu_util import assert_parity, need_gpu
    import oracle
    need_gpu()
    exe = build_caller(tmp_path)
    B, H, d = 3, 2, 64
    case = wl.make_decode(141, B=B, H=H, dk=d, dv=d, steps=1, act="f32", state="f32",
                          init="zero", name="c_caller")
    t = case.tokens
    w = case.weights
    (tmp_path / "meta.txt").write_text(f"{B} {H} {d}\n")
    for name, arr in (("q", t.q[0]), ("k", t.k[0]), ("v", t.v[0]), ("alpha", t.alpha[0]),
                      ("beta", t.beta[0]), ("g", t.g[0]), ("wq", w.conv_q.reshape(-1, 4)),
                      ("wk", w.conv_k.reshape(-1, 4)), ("wv", w.conv_v.reshape(-1, 4))):
        np.ascontiguousarray(arr, dtype=np.float32).tofile(str(tmp_path / f"{name}.f32"))
    print(f"case {case.name}: B={B} H={H} d={d}", flush=True)
    r = subprocess.run([exe, "decode", str(tmp_path)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    y = np.fromfile(str(tmp_path / "y.f32"), dtype=np.float32).reshape(B, H, d)
    S = np.fromfile(str(tmp_path / "state.f32"), dtype=np.float32).reshape(B, H, d, d)
    y_ref, S_ref, _ = oracle.decode_case(case)
    assert_parity(y, y_ref[0], 2e-5, "y from the C caller")
    assert_parity(S, S_ref, 2e-5, "state from the C caller")


def _write_inputs(tmp_path, rows, case):
    t, w = case.tokens, case.weights
    for name, arr in (("q", t.q), ("k", t.k), ("v", t.v), ("alpha", t.alpha),
                      ("beta", t.beta), ("g", t.g)):
        np.ascontiguousarray(arr, dtype=np.float32).reshape(rows, -1).tofile(
            str(tmp_path / f"{name}.f32"))
    for name, arr in (("wq", w.conv_q), ("wk", w.conv_k), ("wv", w.conv_v)):
        np.ascontiguousarray(arr, dtype=np.float32).reshape(-1, 4).tofile(
            str(tmp_path / f"{name}.f32"))


@pytest.mark.gpu
def test_c_caller_verify_and_commit_match_oracle(tmp_path):
    from gpu_util import assert_parity, need_gpu
    import oracle
    need_gpu()
    exe = build_caller(tmp_path)
    B, H, d, n = 5, 2, 128, 4
    case = wl.make_verify(142, B=B, H=H, dk=d, dv=d, n_draft=n, act="f32", state="f32",
                          init="zero", name="c_caller_verify")
    case.accepted[:] = [0, 1, 2, 3, 4]
    (tmp_path / "meta.txt").write_text(f"{B} {H} {d} {n}\n")
    _write_inputs(tmp_path, B * n, case)
    np.asarray(case.accepted, dtype=np.int32).tofile(str(tmp_path / "accepted.i32"))
    print(f"case {case.name}: B={B} H={H} d={d} n={n}", flush=True)
    r = subprocess.run([exe, "verify", str(tmp_path)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    y = np.fromfile(str(tmp_path / "y.f32"), dtype=np.float32).reshape(B, n, H, d)
    rec = np.fromfile(str(tmp_path / "records.f32"), dtype=np.float32).reshape(B, n, H, d, d)
    S = np.fromfile(str(tmp_path / "state.f32"), dtype=np.float32).reshape(B, H, d, d)
    y_ref, rec_ref, S_ref, _ = oracle.verify_case(case)
    assert_parity(y, y_ref, 2e-5, "verify y from the C caller")
    assert_parity(rec, rec_ref, 2e-5, "records from the C caller")
    # m = 0 leaves the (zero) pool slot untouched; the others hold record m
    assert np.all(S[0] == 0.0)
    assert_parity(S[1:], S_ref[1:], 2e-5, "committed states from the C caller")


@pytest.mark.gpu
def test_c_caller_prefill_matches_oracle(tmp_path):
    from gpu_util import assert_parity, need_gpu
    import oracle
    need_gpu()
    exe = build_caller(tmp_path)
    lens = [150, 1, 64]
    B, H, d = len(lens), 2, 128
    case = wl.make_prefill(143, lens=lens, H=H, dk=d, dv=d, act="f32", state="f32",
                           init="zero", slice_len=32, name="c_caller_prefill")
    T = int(case.cu_seqlens[-1])
    (tmp_path / "meta.txt").write_text(f"{B} {H} {d}\n")
    _write_inputs(tmp_path, T, case)
    np.asarray(case.cu_seqlens, dtype=np.int32).tofile(str(tmp_path / "cu_seqlens.i32"))
    print(f"case {case.name}: lens={lens} H={H}", flush=True)
    r = subprocess.run([exe, "prefill", str(tmp_path)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    y = np.fromfile(str(tmp_path / "y.f32"), dtype=np.float32).reshape(T, H, d)
    S = np.fromfile(str(tmp_path / "state.f32"), dtype=np.float32).reshape(B, H, d, d)
    y_ref, S_ref, _ = oracle.prefill_case(case)
    assert_parity(y, y_ref, 2e-5, "prefill y from the C caller")
    assert_parity(S, S_ref, 2e-5, "prefill states from the C caller")
