#!/usr/bin/env python3
"""Benchmark: one decode step of paged attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one call of the library's decode attention over one batch (planner,
split attention and merge kernels).  The headline workload is the
Llama-3-8B-shaped GQA batch (64 requests, 32 query / 8 KV heads, head_dim 128,
bf16, page 16, lognormal lengths with median 2048).  Inputs are seeded and
synthetic and already resident in HBM when timing starts; two copies of the
KV cache are alternated so that consecutive steps cannot hit in the 256 MB
last-level cache.

Printed: one JSON line with the metric (algorithmic KV GB/s), tokens/s, the
dominant kernel's roofline (its own duration from hipExtLaunchKernel events,
recorded over a second pass of the same number of steps, since the events
lengthen the steps they bracket), HBM traffic from committed rocprofv3 counter
runs when they match the current kernel source, the float64 CPU oracle's
throughput on a bounded sample, the other workloads as secondary figures, and
the paged KV append (this step's K/V or latent written into its page slot)
timed on the headline, MLA and fp8 workloads, the headline's per-call latency
percentiles (each call between its own events, a separate pass), a 1 GiB
device copy's bandwidth on the same GPU, and the device's properties.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attention KV GB/s (% of HBM peak) + tokens/s per step, 1 MI355X"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK = 2.5e15         # dense bf16 FLOP/s, MI355X
# sources of the headline's dominant kernel (gqa_mfma_kernel: bf16, 4 query heads per KV head)
KERNEL_SOURCES = ["paged_kv_cache_471_amd/csrc/gqa_mfma.hip", "paged_kv_cache_471_amd/csrc/da_gqa_mfma.h",
                  "paged_kv_cache_471_amd/csrc/da_common.h", "paged_kv_cache_471_amd/csrc/da_launch.h",
                  "paged_kv_cache_471_amd/csrc/da_plan.h"]
PMC_FILE = os.path.join(ROOT, "profiles", "gqa_llama8b_pmc.md")
# sources of the 128-head MLA kernel and its merge
MLA_KERNEL_SOURCES = ["paged_kv_cache_471_amd/csrc/mla_wave.hip", "paged_kv_cache_471_amd/csrc/da_mla.h",
                      "paged_kv_cache_471_amd/csrc/da_common.h", "paged_kv_cache_471_amd/csrc/da_launch.h",
                      "paged_kv_cache_471_amd/csrc/da_plan.h"]
MLA_PMC_FILE = os.path.join(ROOT, "profiles", "mla_pmc.md")


def kernel_hash(sources=None) -> str:
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES if sources is None else sources):
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(path=PMC_FILE, sources=None):
    """HBM bytes per launch of a kernel from its committed counter summary, or
    None when the summary is missing or was taken on a different kernel source."""
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("pmc: "):
            d = json.loads(line[5:])
            if d.get("kernel_hash") != kernel_hash(sources):
                return None
            return d.get("traffic_bytes_per_launch")
    return None


def counters_from_profiles(path, sources):
    """The machine-readable `sq:` line of a committed SQ-counter summary, or
    None when it is missing or was taken on a different kernel source."""
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("sq: "):
            d = json.loads(line[4:])
            return d if d.get("kernel_hash") == kernel_hash(sources) else None
    return None


def gqa_kernel_name(cfg, rows: int = 1) -> str:
    """The GQA attention kernel the library runs for this head shape (the
    library's own host query, so that this never drifts from its dispatch)."""
    import workloads as wl
    import paged_kv_cache_471_amd as da
    fp8 = cfg.kv_dtype == wl.FP8
    d = da.PagedDesc(max(1, cfg.batch), cfg.q_heads, cfg.kv_heads, cfg.head_dim, cfg.page_size, 1, 1,
                     cfg.q_dtype, cfg.kv_dtype, 0, 16 if fp8 else None, 16 if fp8 else None)
    name = da.kernel_name(d, rows)
    if name is None:
        raise ValueError(f"the library refuses this shape: {cfg}, {rows} rows")
    return name


def headline_kernel(cfg, rows: int, default_shape: bool):
    """(kernel name, its source list, its committed HBM-counter summary or None)
    for the dominant kernel of a headline workload.  The counter summaries hold
    one workload each (llama8b; mla at 128 heads): any other headline reports
    traffic as null rather than another workload's bytes."""
    import workloads as wl
    if isinstance(cfg, wl.MLAConfig):
        if cfg.q_heads == 128:
            pmc = MLA_PMC_FILE if (cfg.name == "mla" and rows == 1 and default_shape) else None
            return "mla_wave_kernel", MLA_KERNEL_SOURCES, pmc
        return "mla_attn_kernel", None, None
    name = gqa_kernel_name(cfg, rows)
    pmc = PMC_FILE if (cfg.name == "llama8b" and rows == 1 and default_shape and name == "gqa_mfma_kernel") else None
    return name, KERNEL_SOURCES if name == "gqa_mfma_kernel" else None, pmc


def workload_desc(cfg) -> str:
    import workloads as wl
    if isinstance(cfg, wl.MLAConfig):
        return (f"{cfg.name}: batch {cfg.batch}, {cfg.q_heads} heads over a {cfg.latent_dim}-wide bf16 latent "
                f"(values {cfg.v_dim}), page {cfg.page_size}, lengths {cfg.lengths}")
    return (f"{cfg.name}: batch {cfg.batch}, {cfg.q_heads}/{cfg.kv_heads} heads, head_dim {cfg.head_dim}, "
            f"q {wl.DTYPE_NAMES[cfg.q_dtype]}, kv {wl.DTYPE_NAMES[cfg.kv_dtype]}, page {cfg.page_size}, "
            f"lengths {cfg.lengths}")


def config_fields(cfg, runner):
    import workloads as wl
    d = {"workload": workload_desc(cfg), "batch": runner.batch, "q_heads": cfg.q_heads}
    if isinstance(cfg, wl.MLAConfig):
        d.update(latent_dim=cfg.latent_dim, v_dim=cfg.v_dim)
    else:
        d.update(kv_heads=cfg.kv_heads, head_dim=cfg.head_dim)
    d.update(page_size=cfg.page_size, sum_seq_len=runner.tokens, seed=cfg.seed)
    return d


class GqaRunner:
    def __init__(self, cfg, sets=2):
        import torch
        import workloads as wl
        from workloads import accounting
        self.cfg = cfg
        t0 = time.time()
        self.case = wl.make_gqa_case(cfg)
        self.gen_s = time.time() - t0
        c = self.case
        dev = "cuda"
        to = lambda x, dt: _to_dev(x, dt, dev)
        self.q = to(c.q, cfg.q_dtype)
        kv0 = to(c.kv, cfg.kv_dtype)
        self.kvs = [kv0] + [kv0.clone() for _ in range(sets - 1)]
        self.pt = torch.from_numpy(c.page_table).to(dev)
        self.sl = torch.from_numpy(c.seq_lens).to(dev)
        self.ks = None if c.k_scale is None else torch.from_numpy(c.k_scale).to(dev)
        self.vs = None if c.v_scale is None else torch.from_numpy(c.v_scale).to(dev)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty(self.q.shape[:2], dtype=torch.float32, device=dev)
        self.bytes = accounting.gqa_bytes(c.seq_lens, cfg.page_size, cfg.q_heads, cfg.kv_heads, cfg.head_dim,
                                          cfg.q_dtype, cfg.kv_dtype)
        self.flops = accounting.gqa_flops(c.seq_lens, cfg.q_heads, cfg.head_dim)
        self.i = 0

    def step(self):
        import paged_kv_cache_471_amd as da
        kv = self.kvs[self.i % len(self.kvs)]
        self.i += 1
        da.decode_attn_paged(self.q, kv, self.pt, self.sl, self.case.scale, self.out, self.lse,
                             k_scale=self.ks, v_scale=self.vs)

    @property
    def batch(self):
        return len(self.case.seq_lens)

    @property
    def tokens(self):
        return int(self.case.seq_lens.astype("int64").sum())



class MlaRunner:
    def __init__(self, cfg, sets=2):
        import torch
        import workloads as wl
        from workloads import accounting
        self.cfg = cfg
        t0 = time.time()
        self.case = wl.make_mla_case(cfg)
        self.gen_s = time.time() - t0
        c = self.case
        dev = "cuda"
        self.q = _to_dev(c.q, wl.BF16, dev)
        kv0 = _to_dev(c.kv, wl.BF16, dev)
        self.kvs = [kv0] + [kv0.clone() for _ in range(sets - 1)]
        self.pt = torch.from_numpy(c.page_table).to(dev)
        self.sl = torch.from_numpy(c.seq_lens).to(dev)
        B, H = c.q.shape[:2]
        self.out = torch.empty((B, H, cfg.v_dim), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((B, H), dtype=torch.float32, device=dev)
        self.bytes = accounting.mla_bytes(c.seq_lens, cfg.page_size, H, cfg.latent_dim, cfg.v_dim)
        self.flops = accounting.mla_flops(c.seq_lens, H, cfg.latent_dim, cfg.v_dim)
        self.i = 0

    def step(self):
        import paged_kv_cache_471_amd as da
        kv = self.kvs[self.i % len(self.kvs)]
        self.i += 1
        da.decode_attn_mla(self.q, kv, self.pt, self.sl, self.case.scale, self.cfg.v_dim, self.out, self.lse)

    @property
    def batch(self):
        return len(self.case.seq_lens)

    @property
    def tokens(self):
        return int(self.case.seq_lens.astype("int64").sum())


class AppendRunner:
    """This step's K/V (or MLA latent) written into the cache of an attention
    runner's workload.  Each request writes its last history slot, which has
    the bytes and the addressing of an append at the next position without
    needing a fresh page."""

    def __init__(self, attn):
        import numpy as np
        import torch
        import workloads as wl
        self.attn = attn
        c, cfg = attn.case, attn.cfg
        rng = np.random.default_rng(wl.BASE_SEED)
        B = len(c.seq_lens)
        self.pos = torch.from_numpy((c.seq_lens - 1).astype(np.int32)).cuda()
        self.mla = isinstance(cfg, wl.MLAConfig)
        if self.mla:
            shape = (B, cfg.latent_dim)
            self.new = [_to_dev(wl.to_bf16_bits(rng.standard_normal(shape).astype(np.float32)), wl.BF16, "cuda")]
            self.bytes = B * cfg.latent_dim * 2 * 2 + 2 * B * 4
            self.kv_dtype = wl.BF16
        else:
            shape = (B, cfg.kv_heads, cfg.head_dim)
            self.new = [_to_dev(wl.to_bf16_bits(rng.standard_normal(shape).astype(np.float32)) if cfg.q_dtype == wl.BF16
                                else rng.standard_normal(shape).astype(np.float32), cfg.q_dtype, "cuda")
                        for _ in range(2)]
            n = 2 * B * cfg.kv_heads * cfg.head_dim
            self.bytes = n * (wl.ELEM_BYTES[cfg.q_dtype] + wl.ELEM_BYTES[cfg.kv_dtype]) + 2 * B * 4
            self.kv_dtype = cfg.kv_dtype

    def step(self):
        import paged_kv_cache_471_amd as da
        a = self.attn
        if self.mla:
            da.decode_kv_append_mla(self.new[0], a.kvs[0], a.pt, self.pos)
        else:
            da.decode_kv_append(self.new[0], self.new[1], a.kvs[0], a.pt, self.pos, k_scale=a.ks, v_scale=a.vs)


def time_append(attn, steps, warmup, step_ms):
    import workloads as wl
    r = AppendRunner(attn)
    ms, kms, _ = time_runner(r, steps, warmup, warm_s=0.1)
    # ms_per_call is the rate at which the Python binding issues calls; the
    # kernel itself is what a captured or native serving loop would pay.
    return {"kv_dtype": "bf16" if r.mla else wl.DTYPE_NAMES[r.kv_dtype], "requests": attn.batch,
            "ms_per_call": ms, "kernel_ms": kms, "algorithmic_bytes": r.bytes,
            "kernel_GBps": round(r.bytes / (kms * 1e-3) / 1e9, 2) if kms else None,
            "kernel_pct_of_attention_step": round(100 * kms / step_ms, 2) if kms else None}


class RowsRunner(GqaRunner):
    """A GQA workload with several query rows per request (multi-token
    prediction): the same histories, q and out [B][rows][Hq][D]."""

    def __init__(self, cfg, rows, sets=2):
        import numpy as np
        import workloads as wl
        from workloads import accounting
        super().__init__(cfg, sets)
        self.rows = rows
        c = self.case
        rng = np.random.default_rng(wl.BASE_SEED + rows)
        q32 = rng.standard_normal((len(c.seq_lens), rows, cfg.q_heads, cfg.head_dim)).astype(np.float32)
        self.q = _to_dev(q32 if cfg.q_dtype == wl.F32 else wl.to_bf16_bits(q32), cfg.q_dtype, "cuda")
        self.out = self.q.new_empty(self.q.shape)
        self.lse = self.lse.new_empty((len(c.seq_lens), rows, cfg.q_heads))
        self.bytes = accounting.gqa_bytes(c.seq_lens, cfg.page_size, cfg.q_heads, cfg.kv_heads, cfg.head_dim,
                                          cfg.q_dtype, cfg.kv_dtype, rows)
        self.flops = accounting.gqa_flops(c.seq_lens, cfg.q_heads, cfg.head_dim, rows)

    def step(self):
        import paged_kv_cache_471_amd as da
        kv = self.kvs[self.i % len(self.kvs)]
        self.i += 1
        da.decode_attn_paged_rows(self.q, kv, self.pt, self.sl, self.case.scale, self.out, self.lse,
                                  k_scale=self.ks, v_scale=self.vs)

    @property
    def batch(self):
        return self.rows * len(self.case.seq_lens)       # tokens decoded per step


class MlaRowsRunner(MlaRunner):
    """The MLA workload with several query rows per request (multi-token
    prediction): q [B][rows][H][576], out [B][rows][H][512]."""

    def __init__(self, cfg, rows, sets=2):
        import numpy as np
        import workloads as wl
        from workloads import accounting
        super().__init__(cfg, sets)
        self.rows = rows
        c = self.case
        B, H = c.q.shape[:2]
        rng = np.random.default_rng(wl.BASE_SEED + rows)
        q32 = (cfg.value_std * rng.standard_normal((B, rows, H, cfg.latent_dim))).astype(np.float32)
        self.q = _to_dev(wl.to_bf16_bits(q32), wl.BF16, "cuda")
        self.out = self.out.new_empty((B, rows, H, cfg.v_dim))
        self.lse = self.lse.new_empty((B, rows, H))
        self.bytes = accounting.mla_bytes(c.seq_lens, cfg.page_size, H, cfg.latent_dim, cfg.v_dim, rows)
        self.flops = accounting.mla_flops(c.seq_lens, H, cfg.latent_dim, cfg.v_dim, rows)

    def step(self):
        import paged_kv_cache_471_amd as da
        kv = self.kvs[self.i % len(self.kvs)]
        self.i += 1
        da.decode_attn_mla_rows(self.q, kv, self.pt, self.sl, self.case.scale, self.cfg.v_dim, self.out, self.lse)

    @property
    def batch(self):
        return self.rows * len(self.case.seq_lens)       # tokens decoded per step


# secondary workloads with several query rows per request: name -> (workload, rows)
ROWS_WORKLOADS = {"llama8b-mtp2": ("llama8b", 2), "mla-mtp2": ("mla", 2)}


def rows_runner(cfg, rows):
    import workloads as wl
    return MlaRowsRunner(cfg, rows) if isinstance(cfg, wl.MLAConfig) else RowsRunner(cfg, rows)


# ---------------------------------------------------------------- latency model

# Slot traces for the calibration: prompts and decode lifetimes per slot; the
# batch at a decode step far into the traces holds each slot's stationary load.
CALIB = {
    "gqa": dict(shape=dict(q_heads=32, kv_heads=8, head_dim=128, page_size=16), slots=(16, 32, 64, 128, 256),
                p_law="lognormal:1024:0.8:16:16384", d_law="geometric:512"),
    "mla": dict(shape=dict(heads=128, page_size=64), slots=(32, 64, 96, 128, 192),
                p_law="lognormal:2048:0.8:64:32768", d_law="geometric:512"),
}


# bytes of K/V pages the calibration steps cycle through: twice the 256 MB
# last-level cache and more, so that no step finds its pages left in it by
# the steps before
CALIB_ROTATE_BYTES = 640 * 10 ** 6


class CalibRunner:
    """One decode step over a batch of stationary slot loads, on a K/V buffer
    filled on the device (values do not change the time).  Consecutive steps
    cycle through `sets` page tables over disjoint random pages of the buffer."""

    def __init__(self, kind, lens, kv, gen, sets=1):
        import numpy as np
        import torch
        c = CALIB[kind]["shape"]
        self.kind = kind
        B = len(lens)
        P = c["page_size"]
        npg = (lens + P - 1) // P
        need = int(npg.sum())
        if sets * need > kv.shape[0]:
            raise ValueError(f"{sets} page sets of {need} pages do not fit {kv.shape[0]} pages")
        width = int(npg.max())
        perm = np.random.default_rng(int(lens.sum())).permutation(kv.shape[0]).astype(np.int32)
        self.pts = []
        at = 0
        for _ in range(sets):
            table = np.full((B, width), -1, dtype=np.int32)
            for b in range(B):
                table[b, :npg[b]] = perm[at:at + npg[b]]
                at += int(npg[b])
            self.pts.append(torch.from_numpy(table).cuda())
        self.i = 0
        self.sl = torch.from_numpy(lens.astype(np.int32)).cuda()
        self.kv = kv
        if kind == "gqa":
            self.q = torch.randn((B, c["q_heads"], c["head_dim"]), generator=gen, device="cuda").to(torch.bfloat16)
            self.scale = c["head_dim"] ** -0.5
        else:
            self.q = (0.5 * torch.randn((B, c["heads"], 576), generator=gen, device="cuda")).to(torch.bfloat16)
            self.scale = 576 ** -0.5
        self.out = self.lse = None

    def step(self):
        import paged_kv_cache_471_amd as da
        pt = self.pts[self.i % len(self.pts)]
        self.i += 1
        if self.kind == "gqa":
            self.out, self.lse = da.decode_attn_paged(self.q, self.kv, pt, self.sl, self.scale, self.out, self.lse)
        else:
            self.out, self.lse = da.decode_attn_mla(self.q, self.kv, pt, self.sl, self.scale, 512, self.out,
                                                    self.lse)


def calibrate_latency(kind, steps=20, warmup=5):
    """Fit t_A(T) = alpha_A T + beta_A for one head shape from the kernel's own
    time and the whole step's, over batches of stationary slot loads."""
    import numpy as np
    import torch
    import workloads as wl
    import workloads.slots as slots
    from paged_kv_cache_471_amd import provision
    c = CALIB[kind]
    Bmax = max(c["slots"])
    Pt, Dt = slots.draw_slot_traces(Bmax, 400, c["p_law"], c["d_law"], k=1 if kind == "gqa" else 2)
    theta, q2, nu2 = provision.trace_moments(Pt.ravel(), Dt.ravel())
    step_at = 40 * int(Dt.mean())                   # many lifetimes into every slot's trace
    loads = provision.slot_loads(Pt, Dt, step_at)
    sh = c["shape"]
    P = sh["page_size"]
    per_token = 2 * sh["kv_heads"] * sh["head_dim"] * 2 if kind == "gqa" else 576 * 2
    plans = []
    for B in c["slots"]:
        lens = loads[:B].astype(np.int64)
        need = int(((lens + P - 1) // P).sum())
        plans.append((B, lens, need, max(2, math.ceil(CALIB_ROTATE_BYTES / (need * P * per_token)))))
    pages = max(need * sets for _, _, need, sets in plans)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl.BASE_SEED + 7)
    if kind == "gqa":
        kv = torch.randn((pages, 2, sh["kv_heads"], P, sh["head_dim"]), generator=gen, device="cuda").to(torch.bfloat16)
    else:
        kv = (0.5 * torch.randn((pages, P, 576), generator=gen, device="cuda")).to(torch.bfloat16)
    pts = []
    for B, lens, need, sets in plans:
        r = CalibRunner(kind, lens, kv, gen, sets)
        ms, kms, _ = time_runner(r, steps, warmup, warm_s=0.1)
        pts.append(dict(slots=B, T=int(lens.sum()), step_us=round(ms * 1e3, 2), kernel_us=round(kms * 1e3, 2),
                        page_sets=sets, rotated_MB=round(sets * need * P * per_token / 1e6, 1)))
        del r
    T = [p["T"] for p in pts]
    ak, bk, r2k = provision.fit_latency(T, [p["kernel_us"] * 1e-6 for p in pts])
    a_s, b_s, r2s = provision.fit_latency(T, [p["step_us"] * 1e-6 for p in pts])
    del kv
    torch.cuda.empty_cache()
    return {
        "shape": sh, "bytes_per_token": per_token,
        "slot_traces": {"prompt": c["p_law"], "lifetime": c["d_law"], "theta_hat": round(theta, 1),
                        "nu_hat": round(math.sqrt(nu2), 1), "mean_load_at_step": round(float(loads.mean()), 1)},
        "points": pts,
        "kernel": {"alpha_ns_per_token": round(ak * 1e9, 5), "beta_us": round(bk * 1e6, 2), "r2": round(r2k, 5),
                   "effective_GBps": round(per_token / ak / 1e9, 1)},
        "step": {"alpha_ns_per_token": round(a_s * 1e9, 5), "beta_us": round(b_s * 1e6, 2), "r2": round(r2s, 5),
                 "effective_GBps": round(per_token / a_s / 1e9, 1)},
    }


def oracle_sample(cfg, case, budget_s, per_call=4):
    """Time the float64 oracle on the workload's requests, `per_call` requests
    per oracle call, taken in order and cycling over the batch, until the
    budget is spent.  Returns seconds, requests, tokens and algorithmic bytes
    of the requests done."""
    import numpy as np
    import oracle
    import workloads as wl
    from workloads import accounting
    c = case
    B = len(c.seq_lens)
    done = []
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        reqs = [(len(done) + k) % B for k in range(min(per_call, B))]
        if isinstance(cfg, wl.MLAConfig):
            oracle.mla_decode_attention(c.q, c.kv, c.page_table, c.seq_lens, cfg.page_size, c.scale, cfg.v_dim,
                                        requests=reqs)
        else:
            oracle.paged_decode_attention(c.q, cfg.q_dtype, c.kv, cfg.kv_dtype, c.page_table, c.seq_lens,
                                          cfg.page_size, c.scale, c.k_scale, c.v_scale, requests=reqs)
        done.extend(reqs)
    dt = time.perf_counter() - t0
    lens = c.seq_lens[done]
    if isinstance(cfg, wl.MLAConfig):
        by = accounting.mla_bytes(lens, cfg.page_size, c.q.shape[1], cfg.latent_dim, cfg.v_dim)
    else:
        by = accounting.gqa_bytes(lens, cfg.page_size, cfg.q_heads, cfg.kv_heads, cfg.head_dim, cfg.q_dtype,
                                  cfg.kv_dtype)
    return dict(seconds=dt, requests=len(done), tokens=int(lens.astype(np.int64).sum()), bytes=by)


def host_cores():
    """Threads the CPU baseline uses: the cores this process may run on,
    capped by OMP_NUM_THREADS when the environment sets it."""
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return n


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cases, headline, budget_s):
    """The oracle, as it stands, on the host cores: a figure per workload
    (the median of three samples for the tiny and the headline workload),
    algorithmic GB/s and KV tokens/s."""
    import statistics
    import threadpoolctl
    cores = host_cores()
    per = {}
    with threadpoolctl.threadpool_limits(cores):
        for name, (cfg, case) in cases.items():
            reps = 3 if name in ("tiny", headline) else 1
            share = budget_s * (0.3 if name == headline else 0.15 if name != "tiny" else 0.05)
            per_call = max(1, min(4, len(case.seq_lens) // 32))
            runs = [oracle_sample(cfg, case, share / reps, per_call) for _ in range(reps)]
            gbs = [r["bytes"] / r["seconds"] / 1e9 for r in runs]
            med = sorted(range(reps), key=lambda i: gbs[i])[reps // 2]
            r = runs[med]
            per[name] = {"value": round(gbs[med], 4), "unit": "GB/s",
                         "tokens_per_s": round(r["tokens"] / r["seconds"], 1),
                         "samples": reps, "spread_GBps": [round(min(gbs), 4), round(max(gbs), 4)],
                         "sample": f"{r['requests']} requests ({r['tokens']} tokens) in {r['seconds']:.2f} s"}
    h = per[headline]
    return {
        "value": h["value"], "unit": "GB/s", "cores": cores, "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": f"median of 3 samples of the {headline} workload's requests taken in order, cycling over the "
                  f"batch ({h['sample']} for the median); float64 numpy with BLAS on "
                  f"{cores} threads",
        "tokens_per_s": h["tokens_per_s"],
        "per_config": per,
    }


def make_runner(cfg):
    import workloads as wl
    return MlaRunner(cfg) if isinstance(cfg, wl.MLAConfig) else GqaRunner(cfg)


def _to_dev(x, dtype, dev):
    import numpy as np
    import torch
    import workloads as wl
    if dtype == wl.F32:
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)
    if dtype == wl.BF16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).to(dev).view(torch.float8_e4m3fn)


SETTLE_S = 0.3                  # untimed stepping before a workload's warmup steps (see time_runner)


def time_runner(runner, steps, warmup, kernel_timer=True, warm_s=0.0):
    """Settle, run `warmup` untimed steps, then time exactly `steps` steps.

    Settling (if warm_s > 0) steps the workload untimed for warm_s seconds
    first: the inputs were just generated on the host with the GPU idle, and a
    decode server steps back to back, so the timed steps should see the clock
    the GPU settles at under this load, not its ramp from idle.

    The timed steps run uninstrumented.  With kernel_timer, a second pass of
    `steps` steps then launches the attention kernel with start/stop events
    (hipExtLaunchKernelGGL) to read its own average duration; those events
    lengthen a step by a few microseconds, so that pass is not the step time."""
    import torch
    import paged_kv_cache_471_amd as da
    if warm_s > 0:
        t_end = time.perf_counter() + warm_s
        while time.perf_counter() < t_end:
            for _ in range(8):
                runner.step()
            torch.cuda.synchronize()
    for _ in range(warmup):
        runner.step()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        runner.step()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(stop) / steps
    kms = None
    if kernel_timer:
        da.timer_begin(steps)
        for _ in range(steps):
            runner.step()
        torch.cuda.synchronize()
        tot, n = da.timer_end()
        kms = tot / n if n else None
    return ms, kms, wall


def step_percentiles(runner, calls):
    """Per-call latency of `calls` steps, each bracketed by its own pair of
    events (a separate pass after the timed steps): p10 / p50 / p90 in us."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        e0.record()
        runner.step()
        e1.record()
    torch.cuda.synchronize()
    us = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)
    pick = lambda f: round(us[min(len(us) - 1, int(f * len(us)))], 2)
    return {"calls": calls, "p10_us": pick(0.10), "p50_us": pick(0.50), "p90_us": pick(0.90)}


def copy_bandwidth(mb=1024, steps=20):
    """Device-to-device copy of an mb-MiB fp32 buffer: bytes read plus written per second."""
    import torch
    n = mb * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * n * 4 / (ms * 1e-3) / 1e9


def device_info():
    import torch
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
            "hbm_GiB": round(p.total_memory / 2 ** 30, 1)}


def copy_probe(mb, steps):
    """Plain device copy of known size (reference for counter scaling and bandwidth)."""
    import torch
    n = mb * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    moved = 2 * n * 4
    print(json.dumps({"mode": "copy", "bytes_read_per_copy": n * 4, "bytes_written_per_copy": n * 4,
                      "ms_per_copy": ms, "GBps_read_plus_write": moved / ms / 1e6}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama8b")
    ap.add_argument("--heads", type=int, default=0,
                    help="query heads of the headline workload instead of its own (e.g. an MLA model's heads "
                         "on one GPU of a tensor-parallel group); 0 keeps the workload's")
    ap.add_argument("--kv-heads", type=int, default=0,
                    help="KV heads of a GQA headline workload instead of its own; 0 keeps the workload's")
    ap.add_argument("--secondary", default="tiny,skewed,mla,longfp8,llama8b-mtp2,mla-mtp2",
                    help="comma list of other workloads to report beside the headline ('' for none)")
    ap.add_argument("--cpu-budget", type=float, default=30.0,
                    help="seconds of oracle time for the CPU baseline, over all workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-latency-model", action="store_true", help="skip the t_A(T) calibration")
    ap.add_argument("--mode", choices=["bench", "copy", "step", "append", "calibrate"], default="bench",
                    help="copy: time a plain device copy; step: run the headline step only; append: run the "
                         "workload's KV append only (both for profilers)")
    ap.add_argument("--copy-mb", type=int, default=1024)
    ap.add_argument("--gqa-kernel", choices=["auto", "vector"], default="auto",
                    help="vector: run GQA groups of up to 8 members on the vector kernel (profiling)")
    args = ap.parse_args()
    if args.gqa_kernel == "vector":
        os.environ["DA_GQA_VECTOR"] = "1"      # read by the library at its first GQA call

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not offered "
              "(across GPUs the path would shard by request or by KV head with no exchange inside attention, "
              "or by sequence with one exchange of partial outputs before the merge).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import workloads as wl
    import paged_kv_cache_471_amd as da   # fails loudly if the HIP library is missing

    torch.cuda.set_device(0)
    if args.mode == "copy":
        copy_probe(args.copy_mb, args.steps)
        return
    if args.mode == "calibrate":
        print(json.dumps({"mode": "calibrate", "latency_model": {k: calibrate_latency(k) for k in CALIB}}))
        return

    if args.workload in ROWS_WORKLOADS:
        base_name, rows = ROWS_WORKLOADS[args.workload]
        cfg = wl.CONFIGS[base_name]
        runner = rows_runner(cfg, rows)
    else:
        cfg = wl.CONFIGS[args.workload]
        if args.heads or args.kv_heads:
            import dataclasses
            if args.heads:
                cfg = dataclasses.replace(cfg, q_heads=args.heads)
            if args.kv_heads:
                cfg = dataclasses.replace(cfg, kv_heads=args.kv_heads)
        runner = make_runner(cfg)
    print(f"# headline {cfg.name}: inputs generated in {runner.gen_s:.1f}s, "
          f"sum L = {runner.tokens}, {runner.bytes / 1e6:.1f} MB", file=sys.stderr, flush=True)
    if args.mode == "step":
        ms, kms, _ = time_runner(runner, args.steps, args.warmup, kernel_timer=False, warm_s=SETTLE_S)
        print(json.dumps({"mode": "step", "workload": cfg.name, "ms_per_step": ms}))
        return
    if args.mode == "append":
        ms, kms, _ = time_runner(AppendRunner(runner), args.steps, args.warmup, kernel_timer=False, warm_s=0.1)
        print(json.dumps({"mode": "append", "workload": cfg.name, "ms_per_call": ms}))
        return

    ms, kms, wall = time_runner(runner, args.steps, args.warmup, warm_s=SETTLE_S)
    per_call = step_percentiles(runner, max(100, args.steps))
    appends = {cfg.name: time_append(runner, args.steps, args.warmup, ms)}
    gbs = runner.bytes / (ms * 1e-3) / 1e9
    kern_gbs = runner.bytes / (kms * 1e-3) / 1e9 if kms else None
    rows_h = ROWS_WORKLOADS[args.workload][1] if args.workload in ROWS_WORKLOADS else 1
    kname, ksrc, kpmc = headline_kernel(cfg, rows_h, not (args.heads or args.kv_heads))
    traffic = traffic_from_profiles(kpmc, ksrc) if kpmc else None

    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if isinstance(cfg, wl.MLAConfig) else wl.DTYPE_NAMES[cfg.kv_dtype],
        "data": "synthetic",
        "config": config_fields(cfg, runner),
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "decode_tokens_per_s": runner.batch / (ms * 1e-3),
        "kv_tokens_per_s": runner.tokens / (ms * 1e-3),
        "algorithmic_bytes_per_step": runner.bytes,
        "roofline": {
            "bound": "hbm",
            "kernel": kname,
            "achieved": round(kern_gbs, 2) if kern_gbs else None,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(kern_gbs / HBM_PEAK_GBS, 4) if kern_gbs else None,
            "traffic": traffic,
            "kernel_ms": kms,
            "kernel_source_hash": kernel_hash(ksrc) if ksrc else None,
        },
    }

    secondary = {}
    host_cases = {cfg.name: (cfg, runner.case)}
    for name in [s for s in args.secondary.split(",") if s]:
        rows = 1
        if name in ROWS_WORKLOADS:
            base_name, rows = ROWS_WORKLOADS[name]
            scfg = wl.CONFIGS[base_name]
        else:
            scfg = wl.CONFIGS[name]
        del runner
        torch.cuda.empty_cache()
        runner2 = rows_runner(scfg, rows) if rows > 1 else make_runner(scfg)
        print(f"# secondary {name}: sum L = {runner2.tokens}, {runner2.bytes / 1e6:.1f} MB", file=sys.stderr,
              flush=True)
        sms, skms, _ = time_runner(runner2, max(10, args.steps // 2), max(3, args.warmup // 2), warm_s=SETTLE_S)
        sg = runner2.bytes / (sms * 1e-3) / 1e9
        desc = workload_desc(scfg) + (f", {rows} query rows per request (MTP depth {rows - 1})" if rows > 1 else "")
        entry = {"workload": desc, "ms_per_step": sms, "GBps": round(sg, 2),
                 "pct_hbm_peak": round(100 * sg / HBM_PEAK_GBS, 2),
                 "kernel_ms": skms,
                 "kernel_GBps": round(runner2.bytes / (skms * 1e-3) / 1e9, 2) if skms else None,
                 "decode_tokens_per_s": runner2.batch / (sms * 1e-3),
                 "kv_tokens_per_s": runner2.tokens / (sms * 1e-3),
                 "algorithmic_bytes_per_step": runner2.bytes}
        if isinstance(scfg, wl.MLAConfig):
            entry["algorithmic_flops_per_step"] = runner2.flops
            entry["mfma_TFLOPs"] = round(runner2.flops / (sms * 1e-3) / 1e12, 1)
            entry["pct_mfma_bf16_peak"] = round(100 * runner2.flops / (sms * 1e-3) / MFMA_BF16_PEAK, 2)
            if name == "mla" and skms:
                kg = runner2.bytes / (skms * 1e-3) / 1e9
                kf = runner2.flops / (skms * 1e-3)
                entry["roofline"] = {
                    "bound": "hbm", "kernel": "mla_wave_kernel",
                    "achieved": round(kg, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(kg / HBM_PEAK_GBS, 4),
                    "mfma": {"achieved_TFLOPs": round(kf / 1e12, 1), "peak_TFLOPs": MFMA_BF16_PEAK / 1e12,
                             "frac": round(kf / MFMA_BF16_PEAK, 4)},
                    "traffic": traffic_from_profiles(MLA_PMC_FILE, MLA_KERNEL_SOURCES),
                    "counters": counters_from_profiles(os.path.join(ROOT, "profiles", "mla_sq_counters.md"),
                                                       MLA_KERNEL_SOURCES),
                    "kernel_ms": skms,
                    "kernel_source_hash": kernel_hash(MLA_KERNEL_SOURCES),
                }
        if rows == 1:
            host_cases[name] = (scfg, runner2.case)
        secondary[name] = entry
        if name in ("mla", "longfp8"):
            appends[name] = time_append(runner2, max(10, args.steps // 2), max(3, args.warmup // 2), sms)
        runner = runner2
    if secondary:
        result["secondary"] = secondary
    result["kv_append"] = appends
    del runner
    torch.cuda.empty_cache()
    copy_gbs = copy_bandwidth()
    result["step_latency"] = per_call
    result["device"] = device_info()
    result["copy_GBps"] = round(copy_gbs, 1)
    result["pct_of_copy_GBps"] = round(100.0 * gbs / copy_gbs, 2)
    if not args.no_latency_model:
        result["latency_model"] = {k: calibrate_latency(k) for k in CALIB}

    if not args.no_cpu_baseline:
        order = [n for n in ("tiny", "llama8b", "skewed", "mla", "longfp8") if n in host_cases]
        order += [n for n in host_cases if n not in order]
        result["cpu_baseline"] = cpu_baseline({n: host_cases[n] for n in order}, cfg.name, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
