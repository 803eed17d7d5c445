"""Prefill parity (all ten steps: projections, RMSNorm, RoPE, cache append,
causal attention in the absorbed form and in the explicit form) against the
float64 explicit oracle."""
import numpy as np
import pytest
import torch

import head_latent_attention_06_amd as mla
import mla_inputs as mi
from mla_testutil import BF16_TOL, F32_TOL, config, dev, host, paged_cache, rel_l2
from oracle import mla_oracle as om

pytestmark = pytest.mark.gpu

WNAMES = ("w_dq", "g_q", "w_uq", "w_qr", "w_dkv", "g_kv", "w_kr", "w_uk", "w_uv")


FORMS = [pytest.param(mla.PREFILL_ABSORBED, id="absorbed"), pytest.param(mla.PREFILL_EXPLICIT, id="explicit")]


def _prefill(shape, dtype, config_id, B, L, start_pos=0, gain_spread=0.0, shuffle=True, cache=None, w=None,
             h=None, form=mla.PREFILL_AUTO):
    bf16 = dtype == torch.bfloat16
    cfg = config(shape, dtype)
    cfg.prefill_form = form
    if w is None:
        w = mi.weights(config_id, shape, bf16=bf16, gain_spread=gain_spread)
    if h is None:
        h = mi.hidden(config_id, shape, B, L, bf16=bf16)
    if cache is None:
        kv_end = start_pos + L
        bt, npages = mi.block_table(config_id, [kv_end] * B, shape.page_size, shuffle=shuffle)
        cache = paged_cache(cfg, npages, bt)
    wd = {k: dev(v, dtype) for k, v in w.items()}
    out = torch.empty((B, L, shape.n_heads, shape.d_head), dtype=dtype, device="cuda")
    mla.mla_prefill(cfg, cache, wd, dev(h, dtype), out, start_pos=start_pos)
    torch.cuda.synchronize()
    return cfg, cache, w, h, out


def test_prefill_tiny_fp32_full():
    """B=1, L=64 tiny layer in fp32 (d=64, n_h=4, d_h=16, d_h^R=8, d_c=32, d_c'=48)."""
    s = mi.TINY
    cfg, cache, w, h, out = _prefill(s, torch.float32, 1, 1, 64)
    ref, rows = om.prefill(h[0], w, s.n_heads, s.rms_eps, s.rope_base, s.scale)
    got = host(out)[0]
    err = rel_l2(got, ref)
    print(f"tiny fp32 rel_l2={err:.3e}")
    assert err <= F32_TOL
    # the appended cache rows, read back through the block table
    bt = cache.block_table.cpu().numpy()
    pool = host(cache.pool)
    gathered = om.paged_gather(pool, bt, 0, 64, s.page_size)
    assert rel_l2(gathered, rows) <= F32_TOL
    assert int(cache.err_flags.item()) == 0


def test_prefill_tiny_fp32_gains_and_batch():
    """Non-unit RMSNorm gains (pins the gain reading) and two sequences."""
    s = mi.TINY
    cfg, cache, w, h, out = _prefill(s, torch.float32, 11, 2, 40, gain_spread=0.5)
    for b in range(2):
        ref, _ = om.prefill(h[b], w, s.n_heads, s.rms_eps, s.rope_base, s.scale)
        assert rel_l2(host(out)[b], ref) <= F32_TOL


def test_prefill_chunked_matches_whole_fp32():
    """Prefill of 64 tokens == prefill of 40 then 24 more at start_pos=40."""
    s = mi.TINY
    w = mi.weights(13, s, bf16=False, gain_spread=0.3)
    h = mi.hidden(13, s, 1, 64, bf16=False)
    cfg, cache, _, _, out_all = _prefill(s, torch.float32, 13, 1, 64, w=w, h=h)
    bt, npages = mi.block_table(14, [64], s.page_size, shuffle=True)
    cache2 = paged_cache(cfg, npages, bt)
    _prefill(s, torch.float32, 13, 1, 40, w=w, h=h[:, :40], cache=cache2)
    _, _, _, _, out_tail = _prefill(s, torch.float32, 13, 1, 24, start_pos=40, w=w, h=h[:, 40:], cache=cache2)
    assert rel_l2(host(out_tail)[0], host(out_all)[0, 40:]) <= F32_TOL
    ref, _ = om.prefill(h[0, 40:], w, s.n_heads, s.rms_eps, s.rope_base, s.scale, start_pos=40,
                        past_rows=om.prefill(h[0, :40], w, s.n_heads, s.rms_eps, s.rope_base, s.scale)[1])
    assert rel_l2(host(out_tail)[0], ref) <= F32_TOL


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("L", [96, 300])
def test_prefill_v3_small_bf16_full(form, L):
    """DeepSeek-V3 shapes, B=2: L=96 spans several 32-key tiles with a ragged
    tail; L=300 spans two 256-query groups and five 64-key tiles."""
    s = mi.V3
    cfg, cache, w, h, out = _prefill(s, torch.bfloat16, 31, 2, L, form=form)
    got = host(out)
    assert np.isfinite(got).all()
    for b in range(2):
        ref, rows = om.prefill(h[b], w, s.n_heads, s.rms_eps, s.rope_base, s.scale)
        err = rel_l2(got[b], ref)
        print(f"b={b} rel_l2={err:.3e}")
        assert err <= BF16_TOL
        gathered = om.paged_gather(host(cache.pool), cache.block_table.cpu().numpy(), b, L, s.page_size)
        assert rel_l2(gathered, rows) <= BF16_TOL
    assert int(cache.err_flags.item()) == 0


@pytest.mark.parametrize("form", FORMS)
def test_prefill_v3_8192_sampled(form):
    """B=1, L=8192 causal prefill at DeepSeek-V3 shapes; oracle on sampled (token, head)."""
    s = mi.V3
    L = 8192
    cfg, cache, w, h, out = _prefill(s, torch.bfloat16, 3, 1, L, form=form)
    got = host(out)[0]
    assert np.isfinite(got).all()
    tokens = np.array([0, 1, 31, 32, 1000, 4095, 4096, 8190, 8191])
    heads = [0, 63, 127]
    ref, rows = om.prefill(h[0], w, s.n_heads, s.rms_eps, s.rope_base, s.scale, tokens=tokens, heads=heads)
    err = rel_l2(got[tokens][:, heads], ref)
    print(f"rel_l2(sampled)={err:.3e}")
    assert err <= BF16_TOL
    gathered = om.paged_gather(host(cache.pool), cache.block_table.cpu().numpy(), 0, L, s.page_size)
    assert rel_l2(gathered, rows) <= BF16_TOL
    assert int(cache.err_flags.item()) == 0


@pytest.mark.parametrize("form", FORMS)
def test_prefill_bf16_chunked_matches_whole(form):
    """V3 shapes: prefill of 160 tokens == 96 tokens, then 64 more at start_pos=96."""
    s = mi.V3
    w = mi.weights(32, s)
    h = mi.hidden(32, s, 1, 160)
    cfg, cache, _, _, out_all = _prefill(s, torch.bfloat16, 32, 1, 160, w=w, h=h, form=form)
    bt, npages = mi.block_table(33, [160], s.page_size, shuffle=True)
    cache2 = paged_cache(cfg, npages, bt)
    _prefill(s, torch.bfloat16, 32, 1, 96, w=w, h=h[:, :96], cache=cache2, form=form)
    _, _, _, _, out_tail = _prefill(s, torch.bfloat16, 32, 1, 64, start_pos=96, w=w, h=h[:, 96:], cache=cache2,
                                    form=form)
    ref, _ = om.prefill(h[0], w, s.n_heads, s.rms_eps, s.rope_base, s.scale, tokens=np.arange(96, 160))
    assert rel_l2(host(out_tail)[0], ref) <= BF16_TOL
    assert rel_l2(host(out_tail)[0], host(out_all)[0, 96:]) <= 5e-3


@pytest.mark.parametrize("form", FORMS)
def test_prefill_bf16_two_sequences_after_prefix(form):
    """B=2, 200 cached tokens, then 300 new ones (two 256-query groups, the
    diagonal off every tile boundary); checked on sampled tokens."""
    s = mi.V3
    w = mi.weights(35, s)
    h = mi.hidden(35, s, 2, 500)
    bt, npages = mi.block_table(36, [500, 500], s.page_size, shuffle=True)
    cfg = config(s, torch.bfloat16)
    cfg.prefill_form = form
    cache = paged_cache(cfg, npages, bt)
    _prefill(s, torch.bfloat16, 35, 2, 200, w=w, h=h[:, :200], cache=cache, form=form)
    _, _, _, _, out = _prefill(s, torch.bfloat16, 35, 2, 300, start_pos=200, w=w, h=h[:, 200:], cache=cache,
                               form=form)
    toks = np.array([0, 1, 55, 56, 255, 256, 299])
    for b in range(2):
        ref, _ = om.prefill(h[b], w, s.n_heads, s.rms_eps, s.rope_base, s.scale, tokens=200 + toks,
                            heads=[0, 64, 127])
        err = rel_l2(host(out)[b][toks][:, [0, 64, 127]], ref)
        print(f"b={b} rel_l2={err:.3e}")
        assert err <= BF16_TOL
    assert int(cache.err_flags.item()) == 0


def test_prefill_bf16_12000_tokens_large_projection_tiles():
    """B=2 x 6000 tokens: enough rows for the 256-row GEMM tiles on every
    projection, including [W^DKV ; W^KR] h, whose weight comes in two
    segments split at row 512 inside a tile (checked through the appended
    cache rows), and a ragged last row tile (12000 = 46 x 256 + 224)."""
    s = mi.V3
    B, L = 2, 6000
    cfg, cache, w, h, out = _prefill(s, torch.bfloat16, 37, B, L)
    got = host(out)
    toks = np.array([0, 255, 256, 4095, 5999])
    heads = [0, 64, 127]
    pool = host(cache.pool)
    bt = cache.block_table.cpu().numpy()
    for b in range(B):
        ref, rows = om.prefill(h[b], w, s.n_heads, s.rms_eps, s.rope_base, s.scale, tokens=toks, heads=heads)
        err = rel_l2(got[b][toks][:, heads], ref)
        rerr = rel_l2(om.paged_gather(pool, bt, b, L, s.page_size), rows)
        print(f"b={b} out rel_l2={err:.3e} rows rel_l2={rerr:.3e}")
        assert err <= BF16_TOL
        assert rerr <= BF16_TOL
    assert int(cache.err_flags.item()) == 0


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("page_size", [32, 128])
def test_prefill_bf16_other_page_sizes(form, page_size):
    """B=2, 200 cached tokens then 130 more, with 32- or 128-token pages."""
    import dataclasses
    s = dataclasses.replace(mi.V3, page_size=page_size)
    w = mi.weights(38, s)
    h = mi.hidden(38, s, 2, 330)
    bt, npages = mi.block_table(39, [330, 330], page_size, shuffle=True)
    cfg = config(s, torch.bfloat16)
    cfg.prefill_form = form
    cache = paged_cache(cfg, npages, bt)
    _prefill(s, torch.bfloat16, 38, 2, 200, w=w, h=h[:, :200], cache=cache, form=form)
    _, _, _, _, out = _prefill(s, torch.bfloat16, 38, 2, 130, start_pos=200, w=w, h=h[:, 200:], cache=cache,
                               form=form)
    toks = np.array([0, 31, 32, 63, 64, 127, 129])
    pool = host(cache.pool)
    for b in range(2):
        ref, rows = om.prefill(h[b], w, s.n_heads, s.rms_eps, s.rope_base, s.scale, tokens=200 + toks,
                               heads=[0, 77, 127])
        err = rel_l2(host(out)[b][toks][:, [0, 77, 127]], ref)
        rerr = rel_l2(om.paged_gather(pool, cache.block_table.cpu().numpy(), b, 330, page_size), rows)
        print(f"page_size={page_size} b={b} rel_l2={err:.3e} rows={rerr:.3e}", flush=True)
        assert err <= BF16_TOL
        assert rerr <= BF16_TOL
    assert int(cache.err_flags.item()) == 0
