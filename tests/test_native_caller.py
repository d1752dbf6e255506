"""The C ABI from a native caller: tests/native/decode_caller.c, plain C99 over
the HIP runtime's C API with no Python or torch in the process, runs a decode
batch through the allocating entry point and through the workspace entry
point; its outputs are compared with the oracle here, and the two entry
points' outputs with each other bitwise (the kernels are deterministic)."""
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from helpers import gqa_oracle, assert_close_gqa, assert_out_close, TOL_LSE

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "native", "decode_caller")


def _exe():
    if not os.path.exists(EXE):
        import importlib.util
        spec = importlib.util.spec_from_file_location("_da_native", os.path.join(HERE, "native", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    return EXE


def test_native_caller_resolves_every_symbol_it_uses():
    """With eager binding the loader resolves each library and HIP entry point
    the caller names before main runs; a missing input directory then ends it
    with status 1 before any HIP call."""
    env = dict(os.environ, LD_BIND_NOW="1")
    r = subprocess.run([_exe(), os.path.join(HERE, "native", "no-such-dir")], capture_output=True, text=True,
                       env=env, timeout=60)
    assert r.returncode == 1, (r.returncode, r.stderr)
    assert "cannot open" in r.stderr, r.stderr


def _f32_text(x: float) -> str:
    """a decimal that reads back as exactly float32(x)"""
    return repr(float(np.float32(x)))


def _write(d, name, a):
    np.ascontiguousarray(a).tofile(os.path.join(d, name))


def _run(d):
    print(f"native caller on {d}", flush=True)
    r = subprocess.run([_exe(), str(d)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"status {r.returncode}: {r.stderr}"
    return r.stdout


def _read_bf16(d, name, shape):
    raw = np.fromfile(os.path.join(d, name), dtype=np.uint16)
    return torch.from_numpy(raw.view(np.int16).copy()).view(torch.bfloat16).reshape(shape)


def _read_f32(d, name, shape):
    return torch.from_numpy(np.fromfile(os.path.join(d, name), dtype=np.float32)).reshape(shape)


def _same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


@pytest.mark.gpu
@pytest.mark.parametrize("kd,Hq,Hkv,P", [(wl.BF16, 32, 8, 16), (wl.FP8, 16, 4, 64), (wl.BF16, 6, 2, 32)])
def test_native_gqa_call(tmp_path, kd, Hq, Hkv, P):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = wl.GQAConfig("native", 41, 24, Hq, Hkv, 128, P, wl.BF16, kd, "lognormal:1200:0.9:0:6000")
    case = wl.make_gqa_case(cfg, poison=True, extra_pages=3, seed=41)
    d = str(tmp_path)
    B, maxp = case.page_table.shape
    with open(os.path.join(d, "meta.txt"), "w") as f:
        f.write(f"gqa {B} {Hq} {Hkv} 128 {P} {case.kv.shape[0]} {maxp} {wl.BF16} {kd} {_f32_text(case.scale)}\n")
    _write(d, "q.bin", case.q)
    _write(d, "kv.bin", case.kv)
    _write(d, "page_table.bin", case.page_table.astype(np.int32))
    _write(d, "seq_lens.bin", case.seq_lens.astype(np.int32))
    if kd == wl.FP8:
        _write(d, "k_scale.bin", case.k_scale.astype(np.float32))
        _write(d, "v_scale.bin", case.v_scale.astype(np.float32))
    _run(d)
    out, lse = _read_bf16(d, "out.bin", (B, Hq, 128)), _read_f32(d, "lse.bin", (B, Hq))
    out_ws, lse_ws = _read_bf16(d, "out_ws.bin", (B, Hq, 128)), _read_f32(d, "lse_ws.bin", (B, Hq))
    ro, rl = gqa_oracle(case)
    assert_close_gqa(case, out, lse, ro, rl, label="native decode_attn_paged")
    assert _same_bits(out, out_ws) and _same_bits(lse, lse_ws), "the workspace entry point differs"


@pytest.mark.gpu
@pytest.mark.parametrize("H", [128, 16])
def test_native_mla_call(tmp_path, H):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = wl.MLAConfig("native", 42, 12, H, 576, 512, 64, "lognormal:1500:0.8:0:6000")
    case = wl.make_mla_case(cfg, poison=True, extra_pages=2, seed=42)
    d = str(tmp_path)
    B, maxp = case.page_table.shape
    with open(os.path.join(d, "meta.txt"), "w") as f:
        f.write(f"mla {B} {H} 576 512 64 {case.kv.shape[0]} {maxp} {_f32_text(case.scale)}\n")
    _write(d, "q.bin", case.q)
    _write(d, "kv.bin", case.kv)
    _write(d, "page_table.bin", case.page_table.astype(np.int32))
    _write(d, "seq_lens.bin", case.seq_lens.astype(np.int32))
    _run(d)
    out, lse = _read_bf16(d, "out.bin", (B, H, 512)), _read_f32(d, "lse.bin", (B, H))
    out_ws, lse_ws = _read_bf16(d, "out_ws.bin", (B, H, 512)), _read_f32(d, "lse_ws.bin", (B, H))
    ro, rl = oracle.mla_decode_attention(case.q, case.kv, case.page_table, case.seq_lens, 64, case.scale, 512)
    o = out.float().numpy().astype(np.float64)
    l = lse.numpy().astype(np.float64)
    assert np.all(np.isfinite(o)), "non-finite output"
    assert_out_close(o, ro, wl.BF16, True, "native decode_attn_mla")
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(l), fin) and np.all(l[~fin] == -np.inf)
    rel = np.abs(l[fin] - rl[fin]) / np.maximum(1.0, np.abs(rl[fin]))
    assert float(rel.max()) <= TOL_LSE[wl.BF16], f"lse rel err {rel.max():.3e}"
    assert _same_bits(out, out_ws) and _same_bits(lse, lse_ws), "the workspace entry point differs"
