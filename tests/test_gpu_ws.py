"""Caller-owned workspace entry points (decode_attn_paged_ws, decode_attn_mla_ws)
and the input validator, on the GPU through the C ABI.

The _ws calls run the same kernels as the allocating entry points, so their
results must be bitwise equal to them (and within the oracle bounds); one
workspace of decode_attn_workspace_size bytes serves consecutive calls, the
second one smaller; one byte less is refused before any launch.  The
validator is run on good inputs and on inputs with one precondition broken
(no attention kernel runs on those)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from helpers import gqa_to_dev, mla_to_dev, gqa_oracle, assert_close_gqa, to_dev_storage, out_to_f64

pytestmark = pytest.mark.gpu

da = None


def setup_module(module):
    global da
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_471_amd as _da
    da = _da


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("qd,kd,Hq,Hkv,D,rows", [
    (wl.BF16, wl.BF16, 32, 8, 128, 1),       # the llama-8B head shape (matrix-core kernel)
    (wl.BF16, wl.FP8, 16, 2, 128, 2),        # fp8 with two query rows
    (wl.F32, wl.F32, 8, 2, 64, 1),           # vector kernel
])
def test_gqa_ws_matches_allocating_path(qd, kd, Hq, Hkv, D, rows):
    cfg = wl.GQAConfig("ws", 11, 12, Hq, Hkv, D, 16, qd, kd, "lognormal:900:1.0:1:6000")
    first = wl.make_gqa_case(cfg, poison=True, seed=41)
    cases = [first, wl.make_gqa_case(cfg, seq_lens=first.seq_lens[:5] // 2, poison=True, seed=42)]
    t0 = gqa_to_dev(cases[0])
    d = da.paged_desc(t0["q"], t0["kv"], t0["page_table"], k_scale=t0["k_scale"], v_scale=t0["v_scale"])
    need = da.workspace_size(d, rows)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(5)
    for i, case in enumerate(cases):          # one workspace, two calls, the second smaller
        t = gqa_to_dev(case)
        B = len(case.seq_lens)
        if rows == 1:
            q = t["q"]
            ref_out, ref_lse = da.decode_attn_paged(q, t["kv"], t["page_table"], t["seq_lens"], case.scale,
                                                    k_scale=t["k_scale"], v_scale=t["v_scale"])
        else:
            q32 = rng.standard_normal((B, rows, Hq, D)).astype(np.float32)
            qh = q32 if qd == wl.F32 else wl.to_bf16_bits(q32)
            q = to_dev_storage(qh, qd)
            ref_out, ref_lse = da.decode_attn_paged_rows(q, t["kv"], t["page_table"], t["seq_lens"], case.scale,
                                                         k_scale=t["k_scale"], v_scale=t["v_scale"])
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")
        da.decode_attn_paged_ws(q, t["kv"], t["page_table"], t["seq_lens"], case.scale, ws, out, lse,
                                k_scale=t["k_scale"], v_scale=t["v_scale"])
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(ref_out)), f"call {i}: out differs from the allocating path"
        assert torch.equal(lse, ref_lse), f"call {i}: lse differs from the allocating path"
        if rows == 1:
            ro, rl = gqa_oracle(case)
            assert_close_gqa(case, out, lse, ro, rl, label=f"ws call {i}")
    B0 = len(first.seq_lens)
    qz = torch.zeros((B0, Hq, D) if rows == 1 else (B0, rows, Hq, D), dtype=t0["q"].dtype, device="cuda")
    with pytest.raises(da.DecodeAttnError) as err:         # one byte short: refused before any launch
        da.decode_attn_paged_ws(qz, t0["kv"], t0["page_table"], t0["seq_lens"], first.scale, ws[:need - 1],
                                torch.empty_like(qz), k_scale=t0["k_scale"], v_scale=t0["v_scale"])
    assert err.value.status == -5


@pytest.mark.parametrize("H,rows", [(128, 1), (64, 2)])
def test_mla_ws_matches_allocating_path(H, rows):
    cfg = wl.MLAConfig("ws", 12, 6, H, 576, 512, 64, "lognormal:1500:1.0:1:9000")
    first = wl.make_mla_case(cfg, poison=True, seed=51)
    cases = [first, wl.make_mla_case(cfg, seq_lens=first.seq_lens[:3] // 2, poison=True, seed=52)]
    m0 = mla_to_dev(cases[0])
    P = 64
    d = da.MLADesc(len(cases[0].seq_lens), H, 576, 512, P, m0["kv"].shape[0], m0["page_table"].shape[1], 0)
    need = da.workspace_size(d, rows)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(6)
    for i, case in enumerate(cases):
        t = mla_to_dev(case)
        B = len(case.seq_lens)
        if rows == 1:
            q = t["q"]
            ref_out, ref_lse = da.decode_attn_mla(q, t["kv"], t["page_table"], t["seq_lens"], case.scale)
        else:
            q = to_dev_storage(wl.to_bf16_bits((0.5 * rng.standard_normal((B, rows, H, 576))).astype(np.float32)),
                               wl.BF16)
            ref_out, ref_lse = da.decode_attn_mla_rows(q, t["kv"], t["page_table"], t["seq_lens"], case.scale)
        out = torch.empty(q.shape[:-1] + (512,), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")
        da.decode_attn_mla_ws(q, t["kv"], t["page_table"], t["seq_lens"], case.scale, ws, out, lse)
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(ref_out)), f"call {i}: out differs from the allocating path"
        assert torch.equal(lse, ref_lse), f"call {i}: lse differs from the allocating path"
        if rows == 1:
            ro, rl = oracle.mla_decode_attention(case.q, case.kv, case.page_table, case.seq_lens, P, case.scale, 512)
            err = float(np.max(np.abs(out_to_f64(out) - ro)))
            assert err <= 1.5e-2, f"ws call {i}: max |out - oracle| = {err:.3e}"


def test_validate_inputs_gqa():
    cfg = wl.GQAConfig("val", 13, 6, 8, 2, 128, 16, wl.BF16, wl.BF16, "uniform:1:400")
    case = wl.make_gqa_case(cfg, seed=61)
    t = gqa_to_dev(case)
    d = da.paged_desc(t["q"], t["kv"], t["page_table"])
    assert da.validate_inputs(d, t["page_table"], t["seq_lens"]) == 0
    b = int(np.argmax(case.seq_lens))
    used = (int(case.seq_lens[b]) + 15) // 16
    for bad in (d.num_pages, -1):
        pt = t["page_table"].clone()
        pt[b, used - 1] = bad
        assert da.validate_inputs(d, pt, t["seq_lens"]) == -7
    if used < d.max_pages_per_seq:            # entries past the history are never read
        pt = t["page_table"].clone()
        pt[b, used:] = -1
        assert da.validate_inputs(d, pt, t["seq_lens"]) == 0
    for bad in (d.max_pages_per_seq * 16 + 1, -1):
        sl = t["seq_lens"].clone()
        sl[0] = bad
        assert da.validate_inputs(d, t["page_table"], sl) == -7
    sl = t["seq_lens"].clone()
    sl[0] = 0                                 # an empty history is valid
    assert da.validate_inputs(d, t["page_table"], sl) == 0


def test_validate_inputs_mla():
    cfg = wl.MLAConfig("val", 14, 4, 16, 576, 512, 64, "uniform:1:500")
    case = wl.make_mla_case(cfg, seed=62)
    t = mla_to_dev(case)
    d = da.MLADesc(4, 16, 576, 512, 64, t["kv"].shape[0], t["page_table"].shape[1], 0)
    assert da.validate_inputs(d, t["page_table"], t["seq_lens"]) == 0
    pt = t["page_table"].clone()
    pt[0, 0] = d.num_pages
    assert da.validate_inputs(d, pt, t["seq_lens"]) == -7


def test_ws_calls_replay_from_a_captured_graph():
    """The _ws calls allocate nothing and launch only kernels, so a decode step
    can be captured into a HIP graph: every replay (with eager work and a
    synchronisation between replays) equals the eager result bitwise."""
    cfg = wl.GQAConfig("graph", 15, 12, 32, 8, 128, 16, wl.BF16, wl.BF16, "lognormal:900:1.0:1:6000")
    case = wl.make_gqa_case(cfg, poison=True, seed=71)
    t = gqa_to_dev(case)
    workers = 512                     # explicit: no device query on the captured path
    ref_out, ref_lse = da.decode_attn_paged(t["q"], t["kv"], t["page_table"], t["seq_lens"], case.scale,
                                            workers=workers)
    d = da.paged_desc(t["q"], t["kv"], t["page_table"], workers=workers)
    ws = torch.empty(da.workspace_size(d), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(t["q"])
    lse = torch.empty(t["q"].shape[:2], dtype=torch.float32, device="cuda")
    da.decode_attn_paged_ws(t["q"], t["kv"], t["page_table"], t["seq_lens"], case.scale, ws, out, lse,
                            workers=workers)                  # eager call first
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        da.decode_attn_paged_ws(t["q"], t["kv"], t["page_table"], t["seq_lens"], case.scale, ws, out, lse,
                                workers=workers)
    torch.cuda.synchronize()
    for rep in range(4):
        out.zero_()                   # eager work between replays
        lse.fill_(7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(ref_out)), f"replay {rep}: out differs"
        assert torch.equal(lse, ref_lse), f"replay {rep}: lse differs"

    mcfg = wl.MLAConfig("graph", 16, 6, 128, 576, 512, 64, "lognormal:1500:1.0:1:9000")
    mc = wl.make_mla_case(mcfg, poison=True, seed=72)
    m = mla_to_dev(mc)
    mref, mref_lse = da.decode_attn_mla(m["q"], m["kv"], m["page_table"], m["seq_lens"], mc.scale, workers=100)
    md = da.MLADesc(6, 128, 576, 512, 64, m["kv"].shape[0], m["page_table"].shape[1], 100)
    mws = torch.empty(da.workspace_size(md), dtype=torch.uint8, device="cuda")
    mout = torch.empty((6, 128, 512), dtype=torch.bfloat16, device="cuda")
    mlse = torch.empty((6, 128), dtype=torch.float32, device="cuda")
    da.decode_attn_mla_ws(m["q"], m["kv"], m["page_table"], m["seq_lens"], mc.scale, mws, mout, mlse, workers=100)
    torch.cuda.synchronize()
    mgraph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(mgraph):
        da.decode_attn_mla_ws(m["q"], m["kv"], m["page_table"], m["seq_lens"], mc.scale, mws, mout, mlse,
                              workers=100)
    torch.cuda.synchronize()
    for rep in range(4):
        mout.zero_()
        mlse.fill_(7.0)
        torch.cuda.synchronize()
        mgraph.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(mout), _bits(mref)), f"MLA replay {rep}: out differs"
        assert torch.equal(mlse, mref_lse), f"MLA replay {rep}: lse differs"
