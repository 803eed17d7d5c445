"""Output projection u = W^O [o_1; ...; o_n_h] and the folded W^O' = [W_i^O W_i^UV]
applied to the latent sums, against the float64 oracle."""
import numpy as np
import pytest
import torch

import head_latent_attention_06_amd as mla
import mla_inputs as mi
from mla_testutil import BF16_TOL, F32_TOL, config, dev, host, paged_cache, rel_l2
from oracle import mla_oracle as om

pytestmark = pytest.mark.gpu


def _rand(seed, shape, std=1.0):
    return mi.round_to_bf16((mi.rng(seed, 1).standard_normal(shape) * std).astype(np.float32))


def _project(cfg, x, w_o, dtype):
    T = x.shape[0]
    u = torch.empty((T, w_o.shape[0]), dtype=dtype, device="cuda")
    mla.mla_output_projection(cfg, dev(x.reshape(T, -1), dtype), dev(w_o, dtype), u)
    torch.cuda.synchronize()
    return host(u)


@pytest.mark.parametrize("T", [64, 300])
def test_output_projection_v3_split(T):
    """Decode-sized rows: the 16384-wide reduction is split over workgroups."""
    s = mi.V3
    cfg = config(s)
    x = _rand(71 + T, (T, s.n_heads * s.d_head))
    w_o = _rand(72, (s.d_model, s.n_heads * s.d_head), std=(s.n_heads * s.d_head) ** -0.5)
    got = _project(cfg, x, w_o, torch.bfloat16)
    ref = om.output_projection(x.reshape(T, s.n_heads, s.d_head), w_o)
    err = rel_l2(got, ref)
    print(f"T={T} rel_l2={err:.3e}")
    assert err <= BF16_TOL


def test_output_projection_v3_long_rows_sampled():
    """Prefill-sized rows: one GEMM straight into u; rows checked on a sample."""
    s = mi.V3
    T = 2048
    cfg = config(s)
    x = _rand(73, (T, s.n_heads * s.d_head))
    w_o = _rand(74, (s.d_model, s.n_heads * s.d_head), std=(s.n_heads * s.d_head) ** -0.5)
    got = _project(cfg, x, w_o, torch.bfloat16)
    rows = np.array([0, 1, 127, 128, 1000, 2047])
    ref = om.output_projection(x[rows].reshape(len(rows), s.n_heads, s.d_head), w_o)
    assert rel_l2(got[rows], ref) <= BF16_TOL


def test_output_projection_ragged_tiles_several_rounds():
    """More 256 x 256 tiles than one round of workgroups (396) with both a
    partial last row tile (3000 rows: 184 in the last) and a partial last
    column tile (8256 columns: 64 in the last).  Rows sampled from every row
    tile, every column checked."""
    s = mi.V3
    T, d, H = 3000, 8256, 32
    cfg = config(s)
    cfg.d_model = d
    cfg.n_heads = H
    x = _rand(79, (T, H * s.d_head))
    w_o = _rand(80, (d, H * s.d_head), std=(H * s.d_head) ** -0.5)
    got = _project(cfg, x, w_o, torch.bfloat16)
    rows = np.array([0, 1, 255, 256, 700, 1500, 2047, 2815, 2816, 2999])
    ref = om.output_projection(x[rows].reshape(len(rows), H, s.d_head), w_o)
    err = rel_l2(got[rows], ref)
    print(f"rel_l2={err:.3e}")
    assert err <= BF16_TOL
    assert np.isfinite(got).all()


def test_folded_output_projection():
    """W^O' applied to the latent sums equals W^O applied to the heads'
    outputs (d_model reduced to 1024 to keep the float64 oracle quick)."""
    s = mi.V3
    d, T = 1024, 64
    cfg = config(s)
    cfg.d_model = d
    o_lat = _rand(75, (T, s.n_heads, s.d_c))
    w_uv = _rand(76, (s.n_heads * s.d_head, s.d_c), std=s.d_c ** -0.5)
    w_o = _rand(77, (d, s.n_heads * s.d_head), std=(s.n_heads * s.d_head) ** -0.5)
    w_fold = mi.round_to_bf16(om.fold_output(w_o, w_uv, s.n_heads).astype(np.float32))
    got = _project(cfg, o_lat, w_fold, torch.bfloat16)
    o = np.stack([o_lat[:, i] @ w_uv[i * s.d_head:(i + 1) * s.d_head].astype(np.float64).T for i in range(s.n_heads)],
                 axis=1)
    ref = om.output_projection(o, w_o)
    err = rel_l2(got, ref)
    print(f"folded rel_l2={err:.3e}")
    assert err <= BF16_TOL


def test_output_projection_tiny_fp32_after_prefill():
    """Tiny fp32 layer end to end: prefill, then u = W^O o."""
    s = mi.TINY
    cfg = config(s, torch.float32)
    w = mi.weights(78, s, bf16=False)
    h = mi.hidden(78, s, 1, 40, bf16=False)
    bt, npages = mi.block_table(78, [40], s.page_size)
    cache = paged_cache(cfg, npages, bt)
    out = torch.empty((1, 40, s.n_heads, s.d_head), device="cuda")
    mla.mla_prefill(cfg, cache, {k: dev(v, torch.float32) for k, v in w.items()}, dev(h, torch.float32), out)
    w_o = (mi.rng(78, 5).standard_normal((s.d_model, s.n_heads * s.d_head)) / 8.0).astype(np.float32)
    u = torch.empty((40, s.d_model), device="cuda")
    mla.mla_output_projection(cfg, out.view(40, -1), dev(w_o, torch.float32), u)
    torch.cuda.synchronize()
    o_ref, _ = om.prefill(h[0], w, s.n_heads, s.rms_eps, s.rope_base, s.scale)
    assert rel_l2(host(u), om.output_projection(o_ref, w_o)) <= F32_TOL
