"""Throughput of the MLA hot path on one MI355X.

Headline (one JSON line on stdout): decode of 64 sequences x 4096 cached
tokens + 1 new token each, DeepSeek-V3 MLA heads (n_h = 128, d_c = 512,
d_h^R = 64, 576 bf16 values cached per token, 64-token pages with a shuffled
block table).  A step is one mla_decode call: absorption of W^UK into the
queries, the split-context latent attention, the merge and W^UV.  `value` is
latent-cache bytes per second (the cache is read once per step; 302,063,616 B).

Also measured and reported in the same line:
  * roofline of the dominant kernel (the latent-attention kernel), timed with
    HIP events recorded around that kernel alone on its launch stream;
  * the causal prefill workload (B = 1, L = 8192, d = 7168, all projections,
    cache append and attention) in TFLOP/s, with its attention kernel's roofline;
  * the float64 oracle on the host cores for a bounded sample (cpu_baseline).

Inputs are seeded synthetic tensors (mla_inputs), resident in HBM before the
timed region.  Four copies of the 302 MB cache are rotated so the 256 MB
last-level cache cannot serve a step from the previous one.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import head_latent_attention_06_amd as mla  # noqa: E402
import mla_inputs as mi  # noqa: E402

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
METRIC = "MLA decode latent-KV GB/s + prefill TFLOP/s, % of MI355X roofline"
# YaRN settings of the pages' long-context extension (used with --yarn)
YARN = dict(yarn_s=40.0, yarn_alpha=1.0, yarn_beta=32.0, yarn_orig_ctx=4096)
CFG_EXTRA: dict = {}


class HipEvents:
    """Raw hipEvent_t pairs (the library records them on its launch stream)."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.ev = []
        for _ in range(2 * n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            self.ev.append(e)

    def pair(self, i):
        return self.ev[2 * i], self.ev[2 * i + 1]

    def elapsed_ms(self, i) -> float:
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), self.ev[2 * i], self.ev[2 * i + 1]) == 0
        return ms.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)


def settle(step, min_ms: float = 150.0) -> float:
    """Run `step` untimed until at least min_ms of wall time has passed: from
    idle the GPU needs some tens of milliseconds of sustained load before its
    clock settles, whatever the caller's warm-up count.  Returns the time spent."""
    t0 = time.perf_counter()
    n = 0
    while True:
        step(n)
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
            el = (time.perf_counter() - t0) * 1e3
            if el >= min_ms:
                return el


def _up(a, dtype=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda").to(dtype)


def decode_workload(copies: int, fp8: bool = False):
    inp = mi.decode_inputs(2, mi.V3, mi.config_context_lens(2), 1)
    cfg = mla.Config(kv_fp8=fp8, **CFG_EXTRA)
    bt, npages = mi.block_table(2, inp.kv_lens, cfg.page_size, shuffle=True)
    btd = torch.from_numpy(bt).cuda()
    if fp8:
        # the FP8 rows are written by the library's append, from the drawn rows
        # taken as raw c^KV and k^R (unit RMSNorm gains)
        pool = torch.empty((npages, cfg.page_size, cfg.row_bytes), dtype=torch.uint8, device="cuda")
        rows = _up(inp.rows)
        seq = np.repeat(np.arange(len(inp.kv_lens)), inp.kv_lens).astype(np.int32)
        pos = np.concatenate([np.arange(n) for n in inp.kv_lens]).astype(np.int32)
        mla.mla_cache_append(cfg, mla.PagedCache(pool, btd), rows[:, :cfg.d_c].contiguous(),
                             rows[:, cfg.d_c:].contiguous(), torch.ones(cfg.d_c, dtype=torch.bfloat16, device="cuda"),
                             torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda())
    else:
        pool = torch.empty((npages, cfg.page_size, cfg.row), dtype=torch.bfloat16, device="cuda")
        flat = pool.view(-1, cfg.row)
        for b in range(len(inp.kv_lens)):
            n = int(inp.kv_lens[b])
            pos = np.arange(n)
            idx = torch.from_numpy(bt[b, pos // cfg.page_size].astype(np.int64) * cfg.page_size + pos % cfg.page_size)
            flat[idx.cuda()] = _up(inp.seq_rows(b))
    caches = [mla.PagedCache(pool if i == 0 else pool.clone(), btd) for i in range(copies)]
    t = dict(q_nope=_up(inp.q_nope), q_pe=_up(inp.q_pe), w_uk=_up(inp.w_uk), w_uv=_up(inp.w_uv),
             kv_lens=torch.from_numpy(inp.kv_lens).cuda())
    return inp, cfg, caches, t


def run_decode_bench(steps: int, warmup: int, fp8: bool = False):
    inp, cfg, caches, t = decode_workload(4, fp8)
    B, max_kv = len(inp.kv_lens), int(inp.kv_lens.max())
    out = torch.empty((B, 1, cfg.n_heads, cfg.d_head), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mla.mla_decode_workspace_size(cfg, B, 1, max_kv), dtype=torch.uint8, device="cuda")
    ev = HipEvents(steps)

    def step(i, evs=None):
        mla.mla_decode(cfg, caches[i % len(caches)], t["kv_lens"], max_kv, t["q_nope"], t["q_pe"], t["w_uk"],
                       t["w_uv"], out, ws=ws, attn_events=evs)

    settle_ms = settle(step)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the attention kernel alone: the same steps again, with HIP events recorded
    # around it (kept out of the timed loop above, where they would add gaps)
    for i in range(steps):
        step(i, ev.pair(i))
    torch.cuda.synchronize()
    attn_list = [ev.elapsed_ms(i) for i in range(steps)]
    ev.close()
    latent_bytes = int(inp.kv_lens.sum()) * cfg.row_bytes
    flops = int(inp.kv_lens.sum()) * cfg.n_heads * (cfg.row + cfg.d_c) * 2
    return dict(inp=inp, wall=wall, attn_ms=float(np.mean(attn_list)), attn_list=attn_list,
                latent_bytes=latent_bytes, attn_flops=flops, settle_ms=settle_ms)


def run_fp8_summary(steps: int, warmup: int, bf16_attn_ms: float) -> dict:
    """The decode workload over an FP8 latent cache (656-byte rows)."""
    d = run_decode_bench(steps, warmup, fp8=True)
    ms = d["wall"] / steps * 1e3
    gbs = d["latent_bytes"] / (d["attn_ms"] * 1e-3) / 1e9
    return {"workload": "MLA decode step over an FP8 latent cache (E4M3 c^KV, 1x128 power-of-two scales, bf16 "
                        "k^R: 656 B/token), B=64 x 4097 tokens, n_h=128, 64-token pages",
            "ms_per_step": round(ms, 4), "cache_bytes": d["latent_bytes"],
            "cache_gbs_step": round(d["latent_bytes"] / (ms * 1e-3) / 1e9, 1),
            "roofline": {"bound": "hbm", "kernel": "attn_bf16_kernel<fp8>", "kernel_ms": round(d["attn_ms"], 5),
                         "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "mfma_tflops": round(d["attn_flops"] / (d["attn_ms"] * 1e-3) / 1e12, 1)},
            "attn_time_vs_bf16_cache": round(d["attn_ms"] / bf16_attn_ms, 3)}


def prefill_flops(s: mi.Shape, L: int, explicit: bool) -> dict:
    """FLOPs one prefill executes in the given attention form."""
    T = L
    pairs = L * (L + 1) // 2
    H, dh, dr, dc, dcq, d = s.n_heads, s.d_head, s.d_rope, s.d_c, s.d_cq, s.d_model
    f = {
        "kv_down_proj": 2 * T * (dc + dr) * d,
        "q_down_proj": 2 * T * dcq * d,
        "q_up_proj": 2 * T * H * dh * dcq,
        "q_rope_proj": 2 * T * H * dr * dcq,
    }
    if explicit:  # k^C, v^C materialised per head; d_qk = 192, d_v = 128
        f["k_up_proj"] = 2 * T * H * dh * dc
        f["v_up_proj"] = 2 * T * H * dh * dc
        f["attention"] = 2 * pairs * H * (dh + dr + dh)
    else:         # W^UK folded into the query, W^UV after the latent sum
        f["absorb_w_uk"] = 2 * T * H * dh * dc
        f["attention"] = 2 * pairs * H * (dc + dr + dc)
        f["w_uv"] = 2 * T * H * dc * dh
    f["total"] = sum(f.values())
    return f


def run_prefill_bench(steps: int, warmup: int, form: int, L: int = 8192):
    s = mi.V3
    cfg = mla.Config(prefill_form=form, **CFG_EXTRA)
    w = {k: _up(v) for k, v in mi.weights(3, s).items()}
    h = _up(mi.hidden(3, s, 1, L))
    bt, npages = mi.block_table(3, [L], s.page_size, shuffle=True)
    cache = mla.PagedCache(torch.zeros((npages, s.page_size, cfg.row), dtype=torch.bfloat16, device="cuda"),
                           torch.from_numpy(bt).cuda())
    out = torch.empty((1, L, s.n_heads, s.d_head), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mla.mla_prefill_workspace_size(cfg, 1, L), dtype=torch.uint8, device="cuda")
    ev = HipEvents(steps)
    settle(lambda i: mla.mla_prefill(cfg, cache, w, h, out, ws=ws), 100.0)
    for _ in range(warmup):
        mla.mla_prefill(cfg, cache, w, h, out, ws=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        mla.mla_prefill(cfg, cache, w, h, out, ws=ws, attn_events=ev.pair(i))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    attn_ms = float(np.mean([ev.elapsed_ms(i) for i in range(steps)]))
    ev.close()
    del ws, cache, out
    torch.cuda.empty_cache()
    return dict(wall=wall, attn_ms=attn_ms, flops=prefill_flops(s, L, form == mla.PREFILL_EXPLICIT), L=L)


def run_output_projection_bench(steps: int, warmup: int) -> dict:
    """u = W^O o for the decode workload's 64 rows (W^O: 7168 x 16384 bf16,
    235 MB), and the folded W^O' (7168 x 65536, 940 MB) on the latent sums
    instead: the fold removes the W^UV GEMM but reads 4x the weight bytes."""
    s = mi.V3
    cfg = mla.Config(**CFG_EXTRA)
    T = 64
    res = {"workload": "output projection of one decode step: 64 rows, d=7168, n_h*d_h=16384 (W^O) or "
                       "n_h*d_c=65536 (folded W^O' = [W_i^O W_i^UV])"}
    for name, width in (("w_o", s.n_heads * s.d_head), ("folded_w_o", s.n_heads * s.d_c)):
        x = torch.randn((T, width), device="cuda").bfloat16()
        w = (torch.randn((s.d_model, width), device="cuda") * width ** -0.5).bfloat16()
        u = torch.empty((T, s.d_model), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(max(mla.mla_output_projection_workspace_size(cfg, T, width), 256), dtype=torch.uint8,
                         device="cuda")
        settle(lambda i: mla.mla_output_projection(cfg, x, w, u, ws=ws), 100.0)
        for _ in range(warmup):
            mla.mla_output_projection(cfg, x, w, u, ws=ws)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            mla.mla_output_projection(cfg, x, w, u, ws=ws)
        torch.cuda.synchronize()
        us = (time.perf_counter() - t0) / steps * 1e6
        wbytes = s.d_model * width * 2
        res[name] = {"us": round(us, 2), "weight_bytes": wbytes, "weight_gbs": round(wbytes / (us * 1e-6) / 1e9, 1),
                     "frac_hbm": round(wbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        del x, w, u, ws
    torch.cuda.empty_cache()
    return res


def run_down_projection_bench(steps: int, warmup: int) -> dict:
    """[W^DKV ; W^KR] h at the prefill workload's size (B=1, L=8192, d=7168 ->
    576 columns), through mla_project_kv: the GEMM, then the RMSNorm / RoPE /
    append of the 8192 new cache rows.  Inputs drawn on the device (seeded
    N(0,1) h, W ~ N(0, 1/d), unit gain); the rate counts the GEMM's FLOPs over
    the whole call."""
    s = mi.V3
    cfg = mla.Config(**CFG_EXTRA)
    L = 8192
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    h = torch.randn((1, L, s.d_model), device="cuda", generator=g).bfloat16()
    w = {"w_dkv": (torch.randn((s.d_c, s.d_model), device="cuda", generator=g) * s.d_model ** -0.5).bfloat16(),
         "w_kr": (torch.randn((s.d_rope, s.d_model), device="cuda", generator=g) * s.d_model ** -0.5).bfloat16(),
         "g_kv": torch.ones((s.d_c,), device="cuda").bfloat16()}
    bt, npages = mi.block_table(3, [L], s.page_size, shuffle=True)
    cache = mla.PagedCache(torch.zeros((npages, s.page_size, cfg.row), dtype=torch.bfloat16, device="cuda"),
                           torch.from_numpy(bt).cuda())
    ws = torch.empty(max(mla.mla_project_kv_workspace_size(cfg, 1, L), 256), dtype=torch.uint8, device="cuda")
    settle(lambda i: mla.mla_project_kv(cfg, cache, w, h, ws=ws), 100.0)
    for _ in range(warmup):
        mla.mla_project_kv(cfg, cache, w, h, ws=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        mla.mla_project_kv(cfg, cache, w, h, ws=ws)
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) / steps * 1e6
    flops = 2 * L * (s.d_c + s.d_rope) * s.d_model
    del h, w, cache, ws
    torch.cuda.empty_cache()
    return {"workload": "down-projection + append, B=1, L=8192, d=7168 -> 576 (c^KV 512 + k^R 64), bf16",
            "us": round(us, 1), "gemm_flops": flops, "tflops": round(flops / (us * 1e-6) / 1e12, 1),
            "frac_mfma": round(flops / (us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)}


def run_other_decode(steps: int, warmup: int) -> dict:
    """The long-context (B=4 x 131072) and ragged (B=128, context ~ U{1..32768},
    s_q=2) decode workloads.  Cache, queries and weights are drawn on the device
    (seeded torch generator, N(0,1), W ~ N(0, 1/d_c)); lengths and the
    shuffled block tables come from mla_inputs."""
    s = mi.V3
    cfg = mla.Config(**CFG_EXTRA)
    res = {}
    for cid, name, s_q, desc in (
            (4, "long_context_b4_131072", 1, "MLA decode step, B=4 sequences x (131072 cached + 1 new) tokens, "
                                             "s_q=1, V3 heads, 64-token pages, shuffled block table"),
            (5, "ragged_b128_u1_32768_sq2", 2, "MLA decode step, B=128 sequences, context ~ U{1..32768} + 2 new "
                                               "tokens (causal pair), V3 heads, 64-token pages, shuffled block table")):
        ctx = mi.config_context_lens(cid)
        kv = (ctx + s_q).astype(np.int32)
        B, max_kv = len(kv), int(kv.max())
        bt, npages = mi.block_table(cid, kv, s.page_size, shuffle=True)
        g = torch.Generator(device="cuda")
        g.manual_seed(cid)
        pool = torch.randn((npages, s.page_size, cfg.row), generator=g, device="cuda").bfloat16()
        cache = mla.PagedCache(pool, torch.from_numpy(bt).cuda())
        q_nope = torch.randn((B, s_q, s.n_heads, s.d_head), generator=g, device="cuda").bfloat16()
        q_pe = torch.randn((B, s_q, s.n_heads, s.d_rope), generator=g, device="cuda").bfloat16()
        w_uk = (torch.randn((s.n_heads * s.d_head, s.d_c), generator=g, device="cuda") * s.d_c ** -0.5).bfloat16()
        w_uv = (torch.randn((s.n_heads * s.d_head, s.d_c), generator=g, device="cuda") * s.d_c ** -0.5).bfloat16()
        kvd = torch.from_numpy(kv).cuda()
        out = torch.empty((B, s_q, s.n_heads, s.d_head), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(mla.mla_decode_workspace_size(cfg, B, s_q, max_kv), dtype=torch.uint8, device="cuda")
        ev = HipEvents(steps)

        def step(i, evs=None):
            mla.mla_decode(cfg, cache, kvd, max_kv, q_nope, q_pe, w_uk, w_uv, out, ws=ws, attn_events=evs)

        settle(step, 100.0)
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / steps * 1e3
        for i in range(steps):
            step(i, ev.pair(i))
        torch.cuda.synchronize()
        kms = float(np.mean([ev.elapsed_ms(i) for i in range(steps)]))
        ev.close()
        nbytes = int(kv.sum()) * cfg.row * 2
        # keys each query sees (causal within the s_q new tokens)
        pairs = int(sum(int(k) - s_q + i + 1 for k in kv for i in range(s_q)))
        flops = pairs * s.n_heads * (cfg.row + cfg.d_c) * 2
        # the binding roof: bytes at the HBM peak or FLOPs at the MFMA peak, whichever takes longer
        t_hbm, t_mfma = nbytes / (HBM_PEAK_GBS * 1e9), flops / (BF16_PEAK_TFLOPS * 1e12)
        if t_hbm >= t_mfma:
            roof = {"bound": "hbm", "achieved": round(nbytes / (kms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s"}
        else:
            roof = {"bound": "mfma", "achieved": round(flops / (kms * 1e-3) / 1e12, 1), "peak": BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s"}
        roof.update(frac=round(roof["achieved"] / roof["peak"], 4), kernel="attn_bf16_kernel",
                    kernel_ms=round(kms, 5), t_roof_ms=round(max(t_hbm, t_mfma) * 1e3, 5))
        res[name] = {"workload": desc, "ms_per_step": round(ms, 4), "latent_bytes": nbytes, "attn_flops": flops,
                     "gbs_step": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "tflops_step": round(flops / (ms * 1e-3) / 1e12, 1),
                     "frac_roof_step": round(max(t_hbm, t_mfma) * 1e3 / ms, 4), "roofline": roof}
        del pool, cache, out, ws
        torch.cuda.empty_cache()
    return res


def cpu_baseline(inp, min_seconds: float):
    """The float64 oracle on whole sequences of the decode workload (all 128
    heads, every cached row), one after another until min_seconds have passed."""
    from oracle import mla_oracle as om
    s = inp.shape
    t0 = time.perf_counter()
    n = 0
    while n < len(inp.kv_lens) and (n == 0 or time.perf_counter() - t0 < min_seconds):
        om.decode([inp.seq_rows(n)], inp.kv_lens[n:n + 1], 1, inp.q_nope[n:n + 1], inp.q_pe[n:n + 1], inp.w_uk,
                  inp.w_uv, s.d_c, s.scale)
        n += 1
    dt = time.perf_counter() - t0
    rows = int(inp.kv_lens[:n].sum())
    threads = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count())
    return dict(value=rows * s.row * 2 / dt / 1e9, unit="GB/s", cores=threads, kind="oracle",
                sample=f"float64 explicit-form MLA (numpy, {threads} BLAS threads) on sequences 0..{n - 1} of the "
                       f"decode workload ({rows} cached rows, all 128 heads), {dt:.1f} s; value = their latent-row "
                       f"bytes / time")


def copy_calibration(n_bytes: int = 1 << 30, reps: int = 5):
    """A plain device copy of known size, for scaling HBM byte counters."""
    src = torch.ones(n_bytes // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": n_bytes, "bytes_written": n_bytes, "launches": reps}}))


def run_prefill_summary(args) -> dict:
    """Both attention forms on the same workload; the explicit form (what
    mla_prefill picks by itself here) is the main entry, the absorbed form is
    reported beside it."""
    steps = max(2, min(args.steps // 4, 10))  # prefill steps are milliseconds long
    res = {"workload": "MLA causal prefill, B=1, L=8192, d=7168, all projections + append + attention"}
    for form, name, kernel in ((mla.PREFILL_EXPLICIT, "explicit", "fa_bf16_kernel"),
                               (mla.PREFILL_ABSORBED, "absorbed", "attn_bf16_kernel")):
        p = run_prefill_bench(steps, max(2, min(args.warmup // 2, 10)), form)
        pms = p["wall"] / steps * 1e3
        f = p["flops"]
        achieved = f["attention"] / (p["attn_ms"] * 1e-3) / 1e12
        r = {
            "ms_per_step": round(pms, 3), "tflops_executed": round(f["total"] / (pms * 1e-3) / 1e12, 1),
            "tokens_per_s": round(p["L"] / (pms * 1e-3), 1),
            "roofline": {"bound": "mfma", "kernel": kernel, "kernel_ms": round(p["attn_ms"], 4),
                         "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "flops_per_launch": f["attention"]},
        }
        if name == "explicit":
            res.update(r)
            res["form"] = "explicit"
        else:
            res["absorbed_form"] = r
    return res


def measured_traffic(path: str = os.path.join(ROOT, "profiles", "attn_bf16_decode_b64_ctx4096_traffic.md")):
    """HBM bytes per attention launch from the committed counter summary, or
    None when it is missing or the kernel's sources changed after it was taken."""
    try:
        kv = dict(l.split(":", 1) for l in open(path).read().splitlines() if l.startswith(("traffic_", "source_")))
    except OSError:
        return None
    if attention_sources_sha256() != kv.get("source_sha256", "").strip():
        return None
    return int(kv["traffic_bytes_per_launch"].strip())


def attention_sources_sha256() -> str:
    """One hash over the sources the decode attention kernel is built from."""
    import hashlib
    h = hashlib.sha256()
    for f in ("mla_attn.hip", "mla_plan.h", "mla_device.h", "mla_kernels.h"):
        h.update(open(os.path.join(ROOT, "head_latent_attention_06_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def run_ceilings(steps: int = 20) -> dict:
    """Measured ceilings on this GPU: a plain streaming read of 4 GiB (the
    library's own read kernel), the library's large-tile bf16 GEMM at
    8192 x 8192 x 8192 (through the output-projection entry point), a stream
    of independent MFMAs on random operands (both instruction shapes), and the
    vendor GEMM library on the same product."""
    res = {}
    src = torch.ones(1 << 31, dtype=torch.int16, device="cuda")  # 4 GiB
    nbytes = src.numel() * 2
    settle(lambda i: mla.mla_stream_read(src), 100.0)
    ev = HipEvents(steps)
    hip_stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for i in range(steps):
        ev.hip.hipEventRecord(ev.ev[2 * i], hip_stream)
        mla.mla_stream_read(src)
        ev.hip.hipEventRecord(ev.ev[2 * i + 1], hip_stream)
    torch.cuda.synchronize()
    ms = float(np.median([ev.elapsed_ms(i) for i in range(steps)]))
    ev.close()
    res["hbm_read"] = {"kernel": "stream_read_kernel", "bytes": nbytes, "ms": round(ms, 4),
                       "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                       "frac_of_spec": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del src
    n = 8192
    cfg = mla.Config(d_model=n, **CFG_EXTRA)
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    x = torch.randn((n, n), device="cuda", generator=g).bfloat16()
    w = (torch.randn((n, n), device="cuda", generator=g) * n ** -0.5).bfloat16()
    u = torch.empty((n, n), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(mla.mla_output_projection_workspace_size(cfg, n, n), 256), dtype=torch.uint8, device="cuda")
    settle(lambda i: mla.mla_output_projection(cfg, x, w, u, ws=ws), 100.0)
    ev = HipEvents(steps)
    for i in range(steps):
        ev.hip.hipEventRecord(ev.ev[2 * i], hip_stream)
        mla.mla_output_projection(cfg, x, w, u, ws=ws)
        ev.hip.hipEventRecord(ev.ev[2 * i + 1], hip_stream)
    torch.cuda.synchronize()
    ms = float(np.median([ev.elapsed_ms(i) for i in range(steps)]))
    ev.close()
    flops = 2 * n ** 3
    res["gemm_bf16"] = {"kernel": "gemm_big_kernel", "shape": [n, n, n], "operands": "N(0,1) x N(0,1/n), bf16",
                        "ms": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                        "frac_of_spec": round(flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
    del u, ws
    # The matrix cores alone: independent MFMAs on random bf16 operands (the
    # library's mfma_rate_kernel), both instruction shapes.
    ops = torch.randn(1 << 20, device="cuda", generator=g).bfloat16()
    mf = {"kernel": "mfma_rate_kernel", "operands": "N(0,1) bf16"}
    for shape in (16, 32):
        iters = 2000
        settle(lambda i: mla.mla_mfma_rate(ops, iters, shape), 100.0)
        ev = HipEvents(steps)
        hip_stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for i in range(steps):
            ev.hip.hipEventRecord(ev.ev[2 * i], hip_stream)
            mla.mla_mfma_rate(ops, iters, shape)
            ev.hip.hipEventRecord(ev.ev[2 * i + 1], hip_stream)
        torch.cuda.synchronize()
        ms_m = float(np.median([ev.elapsed_ms(i) for i in range(steps)]))
        ev.close()
        # the core clock under the stream (s_memtime cycles per 100 MHz tick)
        clk = torch.zeros(2, dtype=torch.int64, device="cuda")
        mla.mla_mfma_rate(ops, iters, shape, clocks=clk)
        cyc, ticks = (int(v) for v in clk.tolist())
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        tf = cus * 4 * iters * 2 ** 20 / (ms_m * 1e-3) / 1e12
        mf[f"tflops_{shape}x{shape}"] = round(tf, 1)
        mf[f"frac_of_spec_{shape}x{shape}"] = round(tf / BF16_PEAK_TFLOPS, 4)
        mf[f"clock_ghz_{shape}x{shape}"] = round(0.1 * cyc / ticks, 3) if ticks > 0 else None
    res["mfma_bf16"] = mf
    del ops
    # The vendor GEMM library (torch.mm) on the same operands and layout
    # (x times the transpose of w [N, K]), timed the same way (back-to-back
    # launches after the settle phase, an event pair around each): a second
    # reference for what the matrix cores sustain.  Measurement only, never
    # on the library's path.
    settle(lambda i: torch.mm(x, w.t()), 100.0)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in evs:
        e0.record()
        torch.mm(x, w.t())
        e1.record()
    torch.cuda.synchronize()
    ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in evs]))
    res["gemm_bf16_vendor"] = {"kernel": "torch.mm (vendor GEMM library)", "shape": [n, n, n],
                               "operands": "N(0,1) x N(0,1/n), bf16", "ms": round(ms, 4),
                               "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                               "frac_of_spec": round(flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
    del x, w
    torch.cuda.empty_cache()
    return res


def _vs_measured(roof: dict, ceil: dict) -> None:
    """Add the fraction of the measured ceiling of the same unit to a roofline."""
    if roof.get("unit") == "GB/s" and "hbm_read" in ceil:
        roof["frac_of_measured"] = round(roof["achieved"] / ceil["hbm_read"]["gbs"], 4)
    elif roof.get("unit") == "TFLOP/s" and "gemm_bf16" in ceil:
        # against the highest measured matrix-core rate: the MFMA stream, or a
        # GEMM if one ever ran faster
        best = max(ceil["gemm_bf16"]["tflops"], ceil.get("gemm_bf16_vendor", {}).get("tflops", 0.0),
                   ceil.get("mfma_bf16", {}).get("tflops_16x16", 0.0), ceil.get("mfma_bf16", {}).get("tflops_32x32", 0.0))
        roof["frac_of_measured"] = round(roof["achieved"] / best, 4)


LEGS = ("decode", "output_projection", "fp8", "other_decode", "prefill", "down_projection", "ceilings", "cpu")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # Every leg first runs its step untimed for at least 100-150 ms (settle()),
    # so the GPU clock has settled whatever the warm-up count.
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--legs", default=",".join(LEGS),
                    help="comma-separated subset of " + ",".join(LEGS) + " (the headline decode always runs "
                         "unless --prefill-only)")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--prefill-only", action="store_true", help="time only the prefill workload (for profiling)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--yarn", action="store_true",
                    help="run both workloads with the YaRN long-context settings (s=40, alpha=1, beta=32, 4K window)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}): decode sequences shard across GPUs "
              "with no exchange, so N GPUs run N independent copies of this step", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.yarn:
        CFG_EXTRA.update(YARN)
    legs = set(args.legs.split(","))
    unknown = legs - set(LEGS)
    if unknown:
        ap.error(f"unknown legs {sorted(unknown)}")
    if args.no_prefill:
        legs -= {"prefill", "down_projection"}
    if args.no_cpu_baseline:
        legs -= {"cpu"}

    if args.prefill_only:
        print(json.dumps({"prefill": run_prefill_summary(args)}), flush=True)
        return
    d = run_decode_bench(args.steps, args.warmup)
    ms = d["wall"] / args.steps * 1e3
    value = d["latent_bytes"] / (ms * 1e-3) / 1e9
    attn_gbs = d["latent_bytes"] / (d["attn_ms"] * 1e-3) / 1e9
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "MLA decode step, B=64 sequences x (4096 cached + 1 new) tokens, s_q=1, "
                               "n_h=128, d_h=128, d_c=512, d_h^R=64, 64-token pages, shuffled block table",
                   "global_batch": 64, "seq_len": 4097, "parallelism": "none (1 GPU)",
                   "yarn": bool(CFG_EXTRA)},
        "settle_ms": round(d["settle_ms"], 1),
        "roofline": {"bound": "hbm", "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(attn_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "kernel": "attn_bf16_kernel", "kernel_ms": round(d["attn_ms"], 5),
                     "algorithmic_bytes": d["latent_bytes"],
                     "mfma_tflops": round(d["attn_flops"] / (d["attn_ms"] * 1e-3) / 1e12, 1)},
    }
    if "output_projection" in legs:
        res["output_projection"] = run_output_projection_bench(args.steps, args.warmup)
    if "fp8" in legs:
        res["fp8_cache"] = run_fp8_summary(max(20, args.steps // 2), max(20, args.warmup // 2), d["attn_ms"])
    if "other_decode" in legs:
        res["other_decode"] = run_other_decode(max(10, args.steps // 4), max(10, args.warmup // 2))
    if "prefill" in legs:
        res["prefill"] = run_prefill_summary(args)
    if "down_projection" in legs:
        res["down_projection"] = run_down_projection_bench(20, 10)
    if "ceilings" in legs:
        ceil = run_ceilings()
        res["measured_ceilings"] = ceil
        _vs_measured(res["roofline"], ceil)
        for sub in ("fp8_cache", "prefill"):
            if sub in res:
                _vs_measured(res[sub]["roofline"], ceil)
        if "prefill" in res:
            _vs_measured(res["prefill"]["absorbed_form"]["roofline"], ceil)
        for r in res.get("other_decode", {}).values():
            _vs_measured(r["roofline"], ceil)
    if "cpu" in legs:
        res["cpu_baseline"] = cpu_baseline(d["inp"], args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
