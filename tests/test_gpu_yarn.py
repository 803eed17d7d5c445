"""YaRN long-context extension (the page's s = 40, alpha = 1, beta = 32 over a
4K window): RoPE frequencies in the cache append and the prefill query path,
and the logit factor in prefill and decode, against the float64 oracle."""
import numpy as np
import pytest
import torch

import head_latent_attention_06_amd as mla
import mla_inputs as mi
from mla_testutil import BF16_TOL, F32_TOL, config, decode_setup, dev, host, oracle_decode, paged_cache, rel_l2, \
    run_decode
from oracle import mla_oracle as om

pytestmark = pytest.mark.gpu

YARN = dict(s=40.0, alpha=1.0, beta=32.0, orig_ctx=4096)


def _yarn_cfg(shape, dtype, form=mla.PREFILL_AUTO):
    cfg = config(shape, dtype)
    cfg.prefill_form = form
    cfg.yarn_s, cfg.yarn_alpha, cfg.yarn_beta, cfg.yarn_orig_ctx = YARN["s"], YARN["alpha"], YARN["beta"], \
        YARN["orig_ctx"]
    return cfg


@pytest.mark.parametrize("dtype,tol", [(torch.bfloat16, 4e-3), (torch.float32, F32_TOL)])
def test_yarn_append_large_positions(dtype, tol):
    s = mi.V3
    pos = np.array([0, 1, 4095, 4096, 32767, 65536, 131070, 131071])
    n = len(pos)
    ckv, kr = mi.append_inputs(61, s, n)
    g = np.ones(s.d_c, np.float32)
    bt = np.arange(131072 // 64, dtype=np.int32)[None, :]
    cfg = _yarn_cfg(s, dtype)
    cache = paged_cache(cfg, bt.shape[1], bt)
    mla.mla_cache_append(cfg, cache, dev(ckv, dtype), dev(kr, dtype), dev(g, dtype),
                         torch.zeros(n, dtype=torch.int32, device="cuda"),
                         torch.from_numpy(pos.astype(np.int32)).cuda())
    torch.cuda.synchronize()
    pool = host(cache.pool)
    for i in range(n):
        ref = om.cache_row(ckv[i], kr[i], g, int(pos[i]), s.rms_eps, s.rope_base, yarn=YARN)
        plain = om.cache_row(ckv[i], kr[i], g, int(pos[i]), s.rms_eps, s.rope_base)
        got = pool[om.paged_slot(bt, 0, int(pos[i]), 64)]
        err = rel_l2(got[s.d_c:], ref[s.d_c:])
        assert err <= tol, (int(pos[i]), err)
        if pos[i] >= 4096:  # far enough for the YaRN rotation to differ from the plain one
            assert rel_l2(ref[s.d_c:], plain[s.d_c:]) > 10 * tol
    assert int(cache.err_flags.item()) == 0


def _prefill(cfg, shape, config_id, B, L, dtype, w=None, h=None, cache=None, start_pos=0):
    bf16 = dtype == torch.bfloat16
    w = mi.weights(config_id, shape, bf16=bf16) if w is None else w
    h = mi.hidden(config_id, shape, B, L, bf16=bf16) if h is None else h
    if cache is None:
        bt, npages = mi.block_table(config_id, [start_pos + L] * B, shape.page_size, shuffle=True)
        cache = paged_cache(cfg, npages, bt)
    out = torch.empty((B, L, shape.n_heads, shape.d_head), dtype=dtype, device="cuda")
    mla.mla_prefill(cfg, cache, {k: dev(v, dtype) for k, v in w.items()}, dev(h, dtype), out, start_pos=start_pos)
    torch.cuda.synchronize()
    return w, h, cache, out


def test_yarn_prefill_tiny_fp32_chunked():
    """Tiny layer (d_h^R = 8: its four pairs turn ~652, 65, 6.5 and 0.65 times
    over 4K, so all three YaRN regimes occur); 40 tokens, then 24 more."""
    s = mi.TINY
    cfg = _yarn_cfg(s, torch.float32)
    w = mi.weights(62, s, bf16=False, gain_spread=0.3)
    h = mi.hidden(62, s, 1, 64, bf16=False)
    _, _, cache, out_a = _prefill(cfg, s, 62, 1, 40, torch.float32, w=w, h=h[:, :40])
    _, _, _, out_b = _prefill(cfg, s, 62, 1, 24, torch.float32, w=w, h=h[:, 40:], cache=cache, start_pos=40)
    ref, _ = om.prefill(h[0], w, s.n_heads, s.rms_eps, s.rope_base, s.scale, yarn=YARN)
    assert rel_l2(host(out_a)[0], ref[:40]) <= F32_TOL
    assert rel_l2(host(out_b)[0], ref[40:]) <= F32_TOL
    plain, _ = om.prefill(h[0], w, s.n_heads, s.rms_eps, s.rope_base, s.scale)
    assert rel_l2(plain, ref) > 100 * F32_TOL


@pytest.mark.parametrize("form", [pytest.param(mla.PREFILL_ABSORBED, id="absorbed"),
                                  pytest.param(mla.PREFILL_EXPLICIT, id="explicit")])
def test_yarn_prefill_v3_bf16(form):
    s = mi.V3
    cfg = _yarn_cfg(s, torch.bfloat16, form)
    w, h, cache, out = _prefill(cfg, s, 63, 1, 96, torch.bfloat16)
    ref, rows = om.prefill(h[0], w, s.n_heads, s.rms_eps, s.rope_base, s.scale, yarn=YARN)
    err = rel_l2(host(out)[0], ref)
    print(f"yarn prefill rel_l2={err:.3e}")
    assert err <= BF16_TOL
    gathered = om.paged_gather(host(cache.pool), cache.block_table.cpu().numpy(), 0, 96, s.page_size)
    assert rel_l2(gathered, rows) <= BF16_TOL


def test_yarn_decode_logit_factor():
    """Decode takes q^R already rotated, so YaRN there is the logit factor."""
    inp = mi.decode_inputs(64, mi.V3, [0, 70, 300, 1000], 2)
    cfg, cache, bt, t = decode_setup(inp)
    cfg.yarn_s, cfg.yarn_alpha, cfg.yarn_beta, cfg.yarn_orig_ctx = 40.0, 1.0, 32.0, 4096
    out = run_decode(cfg, cache, t, int(inp.kv_lens.max()))
    torch.cuda.synchronize()
    s = inp.shape
    rows = [inp.seq_rows(b) for b in range(len(inp.kv_lens))]
    ref = om.decode(rows, inp.kv_lens, inp.s_q, inp.q_nope, inp.q_pe, inp.w_uk, inp.w_uv, s.d_c,
                    s.scale * om.yarn_logit_factor(40.0))
    err = rel_l2(host(out), ref)
    print(f"yarn decode rel_l2={err:.3e}")
    assert err <= BF16_TOL
    assert rel_l2(oracle_decode(inp), ref) > 5 * BF16_TOL


@pytest.mark.parametrize("form", [pytest.param(mla.PREFILL_ABSORBED, id="absorbed"),
                                  pytest.param(mla.PREFILL_EXPLICIT, id="explicit")])
def test_yarn_prefill_v3_fp8_cache(form):
    """YaRN with the FP8 latent cache: the FP8 append rotates k^R with YaRN's
    frequencies (kept in bf16) and both attention forms read the FP8 rows."""
    s = mi.V3
    cfg = _yarn_cfg(s, torch.bfloat16, form)
    cfg.kv_fp8 = True
    L = 300
    w = mi.weights(63, s)
    h = mi.hidden(63, s, 1, L)
    bt, npages = mi.block_table(63, [L], s.page_size, shuffle=True)
    pool = torch.full((npages, s.page_size, cfg.row_bytes), 0xFF, dtype=torch.uint8, device="cuda")
    cache = mla.PagedCache(pool, torch.from_numpy(bt).cuda(), torch.zeros(1, dtype=torch.int32, device="cuda"))
    out = torch.empty((1, L, s.n_heads, s.d_head), dtype=torch.bfloat16, device="cuda")
    mla.mla_prefill(cfg, cache, {k: dev(v) for k, v in w.items()}, dev(h), out)
    torch.cuda.synchronize()
    assert int(cache.err_flags.item()) == 0
    ref, rows = om.prefill(h[0], w, s.n_heads, s.rms_eps, s.rope_base, s.scale, yarn=YARN, kv_fp8=True)
    err = rel_l2(host(out)[0], ref)
    p = om.paged_gather(pool.cpu().numpy(), bt, 0, L, s.page_size)
    kr = (p[:, 512:640].copy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    print(f"rel_l2={err:.3e} k^R rel_l2={rel_l2(kr, rows[:, 512:]):.3e}", flush=True)
    assert err <= BF16_TOL
    assert rel_l2(kr, rows[:, 512:]) <= BF16_TOL
