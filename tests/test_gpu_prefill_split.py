"""Absorbed-form prefill over contexts longer than one attention split.

A query row whose visible keys exceed what one workgroup stages (98,240 keys
with a bf16 cache and 64-token pages, 32,704 with the FP8 cache) is cut into
chunks whose partials are merged: fused with W^UV for up to 256 query rows,
else a separate merge and a W^UV GEMM.  These cases append a long prefix with
mla_cache_append and prefill a short chunk after it, checked against the
float64 oracle over the same prefix rows (the oracle's own rows of the same
raw inputs; its own FP8 rows for the FP8 cache).
"""
import numpy as np
import pytest
import torch

import head_latent_attention_06_amd as mla
import mla_inputs as mi
from mla_testutil import BF16_TOL, config, dev, host, paged_cache, rel_l2
from oracle import mla_oracle as om

pytestmark = pytest.mark.gpu

S = mi.V3
HEADS = [0, 45, 127]


def _case(config_id, B, start_pos, L, fp8, toks):
    print(f"[prefill split] B={B} start_pos={start_pos} L={L} fp8={fp8}", flush=True)
    cfg = config(S)
    cfg.prefill_form = mla.PREFILL_ABSORBED
    cfg.kv_fp8 = fp8
    kv_end = start_pos + L
    bt, npages = mi.block_table(config_id, [kv_end] * B, S.page_size, shuffle=True)
    if fp8:
        pool = torch.full((npages, S.page_size, cfg.row_bytes), 0xFF, dtype=torch.uint8, device="cuda")
        cache = mla.PagedCache(pool, torch.from_numpy(bt).to("cuda"), torch.zeros(1, dtype=torch.int32,
                                                                                     device="cuda"))
    else:
        cache = paged_cache(cfg, npages, bt)
    # the prefix: raw rows appended by the library
    ckv, kr = mi.append_inputs(config_id, S, B * start_pos)
    g_kv = np.ones(S.d_c, np.float32)
    seq = np.repeat(np.arange(B, dtype=np.int32), start_pos)
    pos = np.tile(np.arange(start_pos, dtype=np.int32), B)
    mla.mla_cache_append(cfg, cache, dev(ckv), dev(kr), dev(g_kv), torch.from_numpy(seq).to("cuda"),
                         torch.from_numpy(pos).to("cuda"))
    w = mi.weights(config_id, S)
    h = mi.hidden(config_id, S, B, L)
    out = torch.empty((B, L, S.n_heads, S.d_head), dtype=torch.bfloat16, device="cuda")
    mla.mla_prefill(cfg, cache, {k: dev(v) for k, v in w.items()}, dev(h), out, start_pos=start_pos)
    torch.cuda.synchronize()
    assert int(cache.err_flags.item()) == 0
    got = host(out)
    assert np.isfinite(got).all()
    for b in range(B):
        sl = slice(b * start_pos, (b + 1) * start_pos)
        if fp8:
            past = om.cache_row_fp8(ckv[sl], kr[sl], g_kv, np.arange(start_pos), S.rms_eps, S.rope_base)[3]
        else:
            past = om.cache_row(ckv[sl], kr[sl], g_kv, np.arange(start_pos), S.rms_eps, S.rope_base)
        ref, _ = om.prefill(h[b], w, S.n_heads, S.rms_eps, S.rope_base, S.scale, start_pos=start_pos,
                            past_rows=past, tokens=np.asarray(toks), heads=HEADS, kv_fp8=fp8)
        err = rel_l2(got[b][toks][:, HEADS], ref)
        print(f"b={b} rel_l2={err:.3e}", flush=True)
        assert err <= BF16_TOL


def test_prefill_split_fp8_fused_merge():
    """FP8 cache, 40,000 cached tokens (two chunks of at most 511 pages), 64 new
    ones: 64 query rows, so the merge runs fused with W^UV."""
    assert 40000 + 64 > 511 * 64
    _case(301, 1, 40000, 64, True, [0, 1, 31, 32, 63])


def test_prefill_split_bf16_fused_merge():
    """bf16 cache, 100,000 cached tokens (past the 98,240 keys of one chunk), 64 new."""
    assert 100000 + 64 > 1535 * 64
    _case(302, 1, 100000, 64, False, [0, 17, 63])


def test_prefill_split_bf16_separate_merge_and_wuv():
    """B = 2 x 160 new tokens after 100,000 cached ones: 320 query rows, so the
    merge and the W^UV GEMM run as separate launches."""
    _case(303, 2, 100000, 160, False, [0, 100, 159])
