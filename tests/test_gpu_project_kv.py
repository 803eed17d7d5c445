"""The W^DKV || W^KR down-projection GEMM with its append epilogue, against the
oracle's latent rows (steps (5) and (7) of the complete MLA computation)."""
import numpy as np
import pytest
import torch

import head_latent_attention_06_amd as mla
import mla_inputs as mi
from mla_testutil import BF16_TOL, F32_TOL, config, dev, host, paged_cache, rel_l2
from oracle import mla_oracle as om

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,L,start", [(1, 200, 0), (3, 77, 64), (2, 130, 1000)])
def test_project_kv_bf16(B, L, start):
    s = mi.V3
    cfg = config(s)
    w = mi.weights(51, s)
    h = mi.hidden(51 + B, s, B, L)
    bt, npages = mi.block_table(51, [start + L] * B, s.page_size, shuffle=True)
    cache = paged_cache(cfg, npages, bt)
    wd = {k: dev(w[k]) for k in ("w_dkv", "w_kr", "g_kv")}
    mla.mla_project_kv(cfg, cache, wd, dev(h), start_pos=start)
    torch.cuda.synchronize()
    assert int(cache.err_flags.item()) == 0
    pool = host(cache.pool)
    for b in range(B):
        c, kr = om.latent_rows(h[b], w["w_dkv"], w["g_kv"], w["w_kr"], start + np.arange(L), s.rms_eps, s.rope_base)
        rows = np.stack([pool[om.paged_slot(bt, b, start + t, s.page_size)] for t in range(L)])
        assert rel_l2(rows[:, :s.d_c], c) <= BF16_TOL
        assert rel_l2(rows[:, s.d_c:], kr) <= BF16_TOL
        if start:  # rows before start_pos are untouched
            assert np.isnan(pool[om.paged_slot(bt, b, start - 1, s.page_size)]).all()


def test_project_kv_f32_tiny():
    s = mi.TINY
    cfg = config(s, torch.float32)
    w = mi.weights(52, s, bf16=False, gain_spread=0.4)
    h = mi.hidden(52, s, 2, 50, bf16=False)
    bt, npages = mi.block_table(52, [50, 50], s.page_size)
    cache = paged_cache(cfg, npages, bt)
    mla.mla_project_kv(cfg, cache, {k: dev(w[k], torch.float32) for k in ("w_dkv", "w_kr", "g_kv")},
                       dev(h, torch.float32))
    torch.cuda.synchronize()
    pool = host(cache.pool)
    for b in range(2):
        c, kr = om.latent_rows(h[b], w["w_dkv"], w["g_kv"], w["w_kr"], np.arange(50), s.rms_eps, s.rope_base)
        rows = om.paged_gather(pool, bt, b, 50, s.page_size)
        assert rel_l2(rows, np.concatenate([c, kr], 1)) <= F32_TOL


@pytest.mark.parametrize("B,L", [(1, 255), (1, 300), (2, 4096), (1, 20224), (1, 20225)])
def test_project_kv_bf16_large(B, L):
    """Token counts around the forms of the down-projection GEMM: below 256
    tokens the 128 x 128 kernel; from 256 tokens while there are fewer row
    tiles of 256 than the 80 workgroup groups of the stream-K form (up to
    20,224 tokens) that form, whose partial sums the append adds (300 tokens:
    8 groups, up to four partials per row tile; 8192: 80 groups, up to
    three); past that one plain launch (20,225).  Sampled rows include tile
    edges and the ragged last tile."""
    s = mi.V3
    cfg = config(s)
    w = mi.weights(53, s)
    h = mi.hidden(53 + L, s, B, L)
    bt, npages = mi.block_table(53, [L] * B, s.page_size, shuffle=True)
    cache = paged_cache(cfg, npages, bt)
    wd = {k: dev(w[k]) for k in ("w_dkv", "w_kr", "g_kv")}
    print(f"project_kv B={B} L={L}", flush=True)
    mla.mla_project_kv(cfg, cache, wd, dev(h))
    torch.cuda.synchronize()
    assert int(cache.err_flags.item()) == 0
    pool = host(cache.pool)
    toks = np.unique(np.array([0, 1, 255, 256, 4095, L // 2, L - 257, L - 256, L - 2, L - 1]) % L)
    for b in range(B):
        c, kr = om.latent_rows(h[b][toks], w["w_dkv"], w["g_kv"], w["w_kr"], toks, s.rms_eps, s.rope_base)
        rows = np.stack([pool[om.paged_slot(bt, b, int(t), s.page_size)] for t in toks])
        assert rel_l2(rows[:, :s.d_c], c) <= BF16_TOL
        assert rel_l2(rows[:, s.d_c:], kr) <= BF16_TOL
