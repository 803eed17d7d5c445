"""Shapes beside the DeepSeek-V3 defaults, against the float64 oracle.

* Head counts other than 128 (any multiple of 32 is served): one workgroup
  covers 128 heads, so 32 and 96 heads leave waves without heads and 160
  heads take a second, partly filled head group.
* Head widths d_h = 64 and 256 (any multiple of 64 up to 512 is served): the
  separate merge and W^UV GEMM in decode, the absorbed form in prefill.
* Pages of 96 (not a power of two) and 256 tokens.

Decode over bf16 and FP8 caches, prefill in both forms where served."""
import dataclasses

import numpy as np
import pytest
import torch

import head_latent_attention_06_amd as mla
import mla_inputs as mi
from mla_testutil import BF16_TOL, config, decode_setup, dev, host, oracle_decode, paged_cache, rel_l2, run_decode
from oracle import mla_oracle as om

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("H", [32, 96, 160])
def test_decode_head_counts_bf16(H):
    s = dataclasses.replace(mi.V3, n_heads=H)
    print(f"[decode heads] H={H}", flush=True)
    inp = mi.decode_inputs(121, s, [5, 300, 2047], 1)
    cfg, cache, bt, t = decode_setup(inp, config_id=121)
    out = run_decode(cfg, cache, t, int(inp.kv_lens.max()))
    torch.cuda.synchronize()
    assert int(cache.err_flags.item()) == 0
    got, ref = host(out), oracle_decode(inp)
    for b in range(3):
        assert rel_l2(got[b], ref[b]) <= BF16_TOL


@pytest.mark.parametrize("H", [32, 160])
def test_decode_head_counts_fp8(H):
    s = dataclasses.replace(mi.V3, n_heads=H)
    print(f"[decode heads fp8] H={H}", flush=True)
    cfg = config(s)
    cfg.kv_fp8 = True
    inp = mi.decode_inputs(122, s, [5, 300, 2047], 1)
    bt, npages = mi.block_table(122, inp.kv_lens, s.page_size, shuffle=True)
    pool = torch.full((npages, s.page_size, cfg.row_bytes), 0xFF, dtype=torch.uint8, device="cuda")
    cache = mla.PagedCache(pool, torch.from_numpy(bt).cuda(), torch.zeros(1, dtype=torch.int32, device="cuda"))
    raws = [inp.seq_rows(b) for b in range(3)]
    g = np.ones(s.d_c, np.float32)
    ckv = np.concatenate([r[:, :s.d_c] for r in raws])
    kr = np.concatenate([r[:, s.d_c:] for r in raws])
    seq = np.concatenate([np.full(len(r), b, np.int32) for b, r in enumerate(raws)])
    pos = np.concatenate([np.arange(len(r), dtype=np.int32) for r in raws])
    mla.mla_cache_append(cfg, cache, dev(ckv), dev(kr), dev(g), torch.from_numpy(seq).cuda(),
                         torch.from_numpy(pos).cuda())
    out = torch.empty((3, 1, H, s.d_head), dtype=torch.bfloat16, device="cuda")
    mla.mla_decode(cfg, cache, torch.from_numpy(inp.kv_lens).cuda(), int(inp.kv_lens.max()), dev(inp.q_nope),
                   dev(inp.q_pe), dev(inp.w_uk), dev(inp.w_uv), out)
    torch.cuda.synchronize()
    assert int(cache.err_flags.item()) == 0
    rows = [om.cache_row_fp8(r[:, :s.d_c], r[:, s.d_c:], g, np.arange(len(r)), s.rms_eps, s.rope_base)[3]
            for r in raws]
    ref = om.decode(rows, inp.kv_lens, 1, inp.q_nope, inp.q_pe, inp.w_uk, inp.w_uv, s.d_c, s.scale)
    got = host(out)
    for b in range(3):
        assert rel_l2(got[b], ref[b]) <= BF16_TOL


@pytest.mark.parametrize("form", [pytest.param(mla.PREFILL_ABSORBED, id="absorbed"),
                                  pytest.param(mla.PREFILL_EXPLICIT, id="explicit")])
def test_prefill_96_heads(form):
    s = dataclasses.replace(mi.V3, n_heads=96)
    print(f"[prefill heads] H=96 form={form}", flush=True)
    cfg = config(s)
    cfg.prefill_form = form
    L = 130
    w = mi.weights(123, s)
    h = mi.hidden(123, s, 1, L)
    bt, npages = mi.block_table(123, [L], s.page_size, shuffle=True)
    cache = paged_cache(cfg, npages, bt)
    out = torch.empty((1, L, 96, s.d_head), dtype=torch.bfloat16, device="cuda")
    mla.mla_prefill(cfg, cache, {k: dev(v) for k, v in w.items()}, dev(h), out)
    torch.cuda.synchronize()
    assert int(cache.err_flags.item()) == 0
    ref, _ = om.prefill(h[0], w, 96, s.rms_eps, s.rope_base, s.scale)
    err = rel_l2(host(out)[0], ref)
    print(f"rel_l2={err:.3e}")
    assert err <= BF16_TOL


@pytest.mark.parametrize("dh", [64, 256])
def test_decode_head_widths(dh):
    """d_h = 64 and 256: the absorption GEMM with K = d_h and, since the fused
    merge + W^UV kernel is written for d_h = 128, the separate merge followed
    by the batched W^UV GEMM."""
    s = dataclasses.replace(mi.V3, d_head=dh)
    print(f"[decode d_h] {dh}", flush=True)
    inp = mi.decode_inputs(124, s, [5, 300, 2047], 2)
    cfg, cache, bt, t = decode_setup(inp, config_id=124)
    out = run_decode(cfg, cache, t, int(inp.kv_lens.max()))
    torch.cuda.synchronize()
    assert int(cache.err_flags.item()) == 0
    got, ref = host(out), oracle_decode(inp)
    for b in range(3):
        err = rel_l2(got[b], ref[b])
        print(f"b={b} rel_l2={err:.3e}")
        assert err <= BF16_TOL


@pytest.mark.parametrize("dh", [64, 256])
def test_prefill_head_widths_absorbed(dh):
    """Prefill at d_h = 64 and 256 (the absorbed form; the explicit form is
    built for d_h = 128 and is refused for other widths)."""
    s = dataclasses.replace(mi.V3, d_head=dh)
    print(f"[prefill d_h] {dh}", flush=True)
    cfg = config(s)
    L = 200
    w = mi.weights(125, s)
    h = mi.hidden(125, s, 1, L)
    bt, npages = mi.block_table(125, [L], s.page_size, shuffle=True)
    cache = paged_cache(cfg, npages, bt)
    out = torch.empty((1, L, s.n_heads, dh), dtype=torch.bfloat16, device="cuda")
    wd = {k: dev(v) for k, v in w.items()}
    cfg.prefill_form = mla.PREFILL_EXPLICIT
    with pytest.raises(mla.MLAError):
        mla.mla_prefill(cfg, cache, wd, dev(h), out)
    cfg.prefill_form = mla.PREFILL_AUTO
    mla.mla_prefill(cfg, cache, wd, dev(h), out)
    torch.cuda.synchronize()
    assert int(cache.err_flags.item()) == 0
    toks = np.array([0, 1, 63, 64, 127, 199])
    ref, _ = om.prefill(h[0], w, s.n_heads, s.rms_eps, s.rope_base, s.scale, tokens=toks, heads=[0, 77, 127])
    err = rel_l2(host(out)[0][toks][:, [0, 77, 127]], ref)
    print(f"rel_l2={err:.3e}")
    assert err <= BF16_TOL


@pytest.mark.parametrize("page_size", [96, 256])
@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_decode_page_sizes_96_256(page_size, fp8):
    """Pages of 96 tokens (a multiple of 32 that is not a power of two: tiles
    wrap to the next page at 3 tiles) and 256 tokens, shuffled tables."""
    s = dataclasses.replace(mi.V3, page_size=page_size)
    print(f"[decode page_size] {page_size} fp8={fp8}", flush=True)
    inp = mi.decode_inputs(126, s, [0, 95, 96, 97, 700, 3000], 1)
    if not fp8:
        cfg, cache, bt, t = decode_setup(inp, config_id=126)
        out = run_decode(cfg, cache, t, int(inp.kv_lens.max()))
        ref = oracle_decode(inp)
    else:
        cfg = config(s)
        cfg.kv_fp8 = True
        bt, npages = mi.block_table(126, inp.kv_lens, page_size, shuffle=True)
        pool = torch.full((npages, page_size, cfg.row_bytes), 0xFF, dtype=torch.uint8, device="cuda")
        cache = mla.PagedCache(pool, torch.from_numpy(bt).cuda(), torch.zeros(1, dtype=torch.int32, device="cuda"))
        raws = [inp.seq_rows(b) for b in range(len(inp.kv_lens))]
        g = np.ones(s.d_c, np.float32)
        seq = np.concatenate([np.full(len(r), b, np.int32) for b, r in enumerate(raws)])
        pos = np.concatenate([np.arange(len(r), dtype=np.int32) for r in raws])
        mla.mla_cache_append(cfg, cache, dev(np.concatenate([r[:, :s.d_c] for r in raws])),
                             dev(np.concatenate([r[:, s.d_c:] for r in raws])), dev(g),
                             torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda())
        out = torch.empty((len(raws), 1, s.n_heads, s.d_head), dtype=torch.bfloat16, device="cuda")
        mla.mla_decode(cfg, cache, torch.from_numpy(inp.kv_lens).cuda(), int(inp.kv_lens.max()), dev(inp.q_nope),
                       dev(inp.q_pe), dev(inp.w_uk), dev(inp.w_uv), out)
        rows = [om.cache_row_fp8(r[:, :s.d_c], r[:, s.d_c:], g, np.arange(len(r)), s.rms_eps, s.rope_base)[3]
                for r in raws]
        ref = om.decode(rows, inp.kv_lens, 1, inp.q_nope, inp.q_pe, inp.w_uk, inp.w_uv, s.d_c, s.scale)
    torch.cuda.synchronize()
    assert int(cache.err_flags.item()) == 0
    got = host(out)
    for b in range(len(inp.kv_lens)):
        assert rel_l2(got[b], ref[b]) <= BF16_TOL


@pytest.mark.parametrize("form", [pytest.param(mla.PREFILL_ABSORBED, id="absorbed"),
                                  pytest.param(mla.PREFILL_EXPLICIT, id="explicit")])
def test_prefill_page_size_96_after_prefix(form):
    s = dataclasses.replace(mi.V3, page_size=96)
    print(f"[prefill page_size 96] form={form}", flush=True)
    cfg = config(s)
    cfg.prefill_form = form
    w = mi.weights(127, s)
    h = mi.hidden(127, s, 1, 400)
    bt, npages = mi.block_table(127, [400], 96, shuffle=True)
    cache = paged_cache(cfg, npages, bt)
    wd = {k: dev(v) for k, v in w.items()}
    for lo, L in ((0, 250), (250, 150)):
        out = torch.empty((1, L, s.n_heads, s.d_head), dtype=torch.bfloat16, device="cuda")
        mla.mla_prefill(cfg, cache, wd, dev(np.ascontiguousarray(h[:, lo:lo + L])), out, start_pos=lo)
    torch.cuda.synchronize()
    assert int(cache.err_flags.item()) == 0
    toks = np.array([0, 1, 95, 96, 149])
    ref, rows = om.prefill(h[0], w, s.n_heads, s.rms_eps, s.rope_base, s.scale, tokens=250 + toks,
                           heads=[0, 77, 127])
    assert rel_l2(host(out)[0][toks][:, [0, 77, 127]], ref) <= BF16_TOL
    gathered = om.paged_gather(host(cache.pool), bt, 0, 400, 96)
    assert rel_l2(gathered, rows) <= BF16_TOL
