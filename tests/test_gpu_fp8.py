"""FP8 latent cache: the append's codes, scales and k^R against the oracle's
own quantisation of the same raw rows, and decode / prefill over an FP8 cache
against the float64 oracle reading the oracle's FP8 rows.

The GPU cache is filled only by the library (mla_cache_append, mla_prefill);
the oracle quantises the same seeded raw rows itself.  Codes are decided on
float32 values on both sides; the GPU's float32 RMSNorm differs from the
oracle's rounded float64 one by a few ulps, so a code may differ where the
value sits on a rounding midpoint (or a tile maximum on a scale boundary):
those cases are checked to be exactly such, and rare.
"""
import dataclasses

import numpy as np
import pytest
import torch

import head_latent_attention_06_amd as mla
import mla_inputs as mi
from mla_testutil import BF16_TOL, config, dev, host, rel_l2
from oracle import mla_oracle as om

pytestmark = pytest.mark.gpu

S = mi.V3


def _shape(page_size=64):
    return dataclasses.replace(S, page_size=page_size)


def _cfg(shape):
    cfg = config(shape)
    cfg.kv_fp8 = True
    return cfg


def _cache(cfg, npages, bt):
    pool = torch.full((npages, cfg.page_size, cfg.row_bytes), 0xFF, dtype=torch.uint8, device="cuda")
    return mla.PagedCache(pool, torch.from_numpy(np.ascontiguousarray(bt, np.int32)).to("cuda"),
                          torch.zeros(1, dtype=torch.int32, device="cuda"))


def _gains(seed):
    return mi.round_to_bf16(1.0 + 0.25 * mi.rng(seed, 97).standard_normal(S.d_c)).astype(np.float32)


def _split(rows_u8):
    """[..., 656] bytes -> codes [..., 512], k^R [..., 64] (float), scales [..., 4]."""
    r = np.ascontiguousarray(rows_u8)
    codes = r[..., :512]
    kr = (r[..., 512:640].copy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    sc = r[..., 640:656].copy().view(np.float32)
    return codes, kr, sc


def _append(cfg, cache, raw_by_seq, g):
    ckv = np.concatenate([r[:, :S.d_c] for r in raw_by_seq])
    kr = np.concatenate([r[:, S.d_c:] for r in raw_by_seq])
    seq = np.concatenate([np.full(len(r), b, np.int32) for b, r in enumerate(raw_by_seq)])
    pos = np.concatenate([np.arange(len(r), dtype=np.int32) for r in raw_by_seq])
    mla.mla_cache_append(cfg, cache, dev(ckv), dev(kr), dev(g), torch.from_numpy(seq).to("cuda"),
                         torch.from_numpy(pos).to("cuda"))


def _oracle_rows(raw, g, shape=S):
    return om.cache_row_fp8(raw[:, :shape.d_c], raw[:, shape.d_c:], g, np.arange(len(raw)), shape.rms_eps,
                            shape.rope_base)


def test_fp8_append_codes_scales_and_rope():
    """3000 tokens of one sequence (46 full pages and a ragged one), rows scaled
    by 2^-8 .. 2^8 so the tile exponents vary, one row with an all-zero tile."""
    shape = _shape()
    cfg = _cfg(shape)
    n = 3000
    ckv, kr = mi.append_inputs(71, shape, n)
    ckv = ckv * np.exp2(mi.rng(71, 98).integers(-8, 9, (n, 1))).astype(np.float32)
    ckv[5, 128:256] = 0.0
    g = _gains(71)
    bt, npages = mi.block_table(71, [n], shape.page_size, shuffle=True)
    cache = _cache(cfg, npages, bt)
    _append(cfg, cache, [np.concatenate([ckv, kr], 1)], g)
    torch.cuda.synchronize()
    assert int(cache.err_flags.item()) == 0
    pool = cache.pool.cpu().numpy()
    rows = np.stack([pool[om.paged_slot(bt, 0, p, shape.page_size)] for p in range(n)])
    codes, kr_g, sc = _split(rows)
    codes_o, e_o, kr_o, _ = om.cache_row_fp8(ckv, kr, g, np.arange(n), shape.rms_eps, shape.rope_base)

    assert rel_l2(kr_g, kr_o) <= BF16_TOL
    y32 = om.rms_norm(ckv, g, shape.rms_eps).astype(np.float32).astype(np.float64)
    # scales: 2^e exactly; a different e only where the tile max sits on 448 * 2^e
    amax = np.abs(y32).reshape(n, 4, 128).max(-1)
    sc_o = np.exp2(e_o.astype(np.float64))
    diff = sc != sc_o
    ratio = amax[diff] / 448.0
    assert np.all(np.abs(ratio / np.exp2(np.round(np.log2(ratio))) - 1) < 1e-5), "scale differs off a boundary"
    assert diff.mean() < 1e-3
    assert sc[5, 1] == 1.0 and np.all(codes[5, 128:256] == 0)
    # codes: equal values, except adjacent codes around a rounding midpoint
    same = np.repeat(~diff, 128, axis=1)
    vg, vo = om.e4m3_value(codes), om.e4m3_value(codes_o)
    x = y32 / np.repeat(sc_o, 128, axis=1)
    off = same & (vg != vo)
    mid = (vg[off] + vo[off]) / 2
    assert np.all(np.abs(x[off] - mid) <= 1e-5 * np.abs(x[off])), "a code differs away from a midpoint"
    assert np.all(np.abs(codes[off].astype(int) - codes_o[off].astype(int)) == 1)
    assert off.mean() < 1e-3
    print(f"scale diffs {diff.sum()}, code diffs {off.sum()} of {same.sum()}")
    # the ragged last page keeps its untouched slots
    last = bt[0, (n - 1) // shape.page_size]
    assert np.all(pool[last, n % shape.page_size:] == 0xFF)


def _decode_case(seed, contexts, s_q, page_size, heads=None):
    shape = _shape(page_size)
    cfg = _cfg(shape)
    inp = mi.decode_inputs(seed, shape, contexts, s_q)
    g = _gains(seed)
    bt, npages = mi.block_table(seed, inp.kv_lens, page_size, shuffle=True)
    cache = _cache(cfg, npages, bt)
    raws = [inp.seq_rows(b) for b in range(len(contexts))]
    _append(cfg, cache, raws, g)
    out = torch.empty((len(contexts), s_q, shape.n_heads, shape.d_head), dtype=torch.bfloat16, device="cuda")
    mla.mla_decode(cfg, cache, torch.from_numpy(inp.kv_lens).to("cuda"), int(inp.kv_lens.max()), dev(inp.q_nope),
                   dev(inp.q_pe), dev(inp.w_uk), dev(inp.w_uv), out)
    torch.cuda.synchronize()
    assert int(cache.err_flags.item()) == 0
    got = host(out)
    assert np.isfinite(got).all()
    rows8 = [_oracle_rows(r, g, shape)[3] for r in raws]
    ref = om.decode(rows8, inp.kv_lens, s_q, inp.q_nope, inp.q_pe, inp.w_uk, inp.w_uv, shape.d_c, shape.scale,
                    heads=heads)
    return inp, raws, g, got if heads is None else got[:, :, heads], ref


@pytest.mark.parametrize("contexts,s_q,page_size", [
    ([0, 1, 31, 32, 33, 63, 64, 65, 100, 300], 1, 64),  # ragged tails around tile and page edges
    ([0, 5, 127, 129, 700], 2, 64),                      # two causal queries per sequence
    ([2047, 3000], 1, 32),                               # 32-token pages, many tiles per chunk
    ([500, 4096], 1, 128),                               # 128-token pages
])
def test_fp8_decode(contexts, s_q, page_size):
    print(f"[fp8 decode] contexts={contexts} s_q={s_q} page_size={page_size}", flush=True)
    inp, raws, g, got, ref = _decode_case(111, contexts, s_q, page_size)
    for b in range(len(contexts)):
        err = rel_l2(got[b], ref[b])
        print(f"b={b} rel_l2={err:.3e}")
        assert err <= BF16_TOL
    # what FP8 storage itself costs: the same step over the unquantised rows
    exact = om.decode([om.cache_row(r[:, :S.d_c], r[:, S.d_c:], g, np.arange(len(r)), S.rms_eps, S.rope_base)
                       for r in raws], inp.kv_lens, s_q, inp.q_nope, inp.q_pe, inp.w_uk, inp.w_uv, S.d_c, S.scale)
    print(f"fp8 cache vs exact rows: rel_l2={rel_l2(ref, exact):.3e}")


def test_fp8_decode_long_rows_split():
    """40,001 and 70,001 keys: more than one FP8 split (at most 511 pages of
    64 keys each), merged; checked on three heads."""
    heads = [0, 77, 127]
    print("[fp8 decode long] contexts=[40000, 70000]", flush=True)
    _, _, _, got, ref = _decode_case(112, [40000, 70000], 1, 64, heads=heads)
    for b in range(2):
        err = rel_l2(got[b], ref[b])
        print(f"b={b} rel_l2={err:.3e}")
        assert err <= BF16_TOL


FORMS = [pytest.param(mla.PREFILL_ABSORBED, id="absorbed"), pytest.param(mla.PREFILL_EXPLICIT, id="explicit")]


def _deq(rows_u8):
    codes, kr, sc = _split(rows_u8)
    return np.concatenate([om.e4m3_value(codes) * np.repeat(sc, 128, axis=-1), kr], axis=-1)


@pytest.mark.parametrize("form", FORMS)
def test_fp8_prefill_after_prefix(form):
    """B=2: 200 tokens, then 130 more at start_pos = 200, over an FP8 cache."""
    shape = S
    cfg = _cfg(shape)
    cfg.prefill_form = form
    w = mi.weights(113, shape)
    h = mi.hidden(113, shape, 2, 330)
    bt, npages = mi.block_table(113, [330, 330], shape.page_size, shuffle=True)
    cache = _cache(cfg, npages, bt)
    wd = {k: dev(v) for k, v in w.items()}
    for lo, L in ((0, 200), (200, 130)):
        out = torch.empty((2, L, shape.n_heads, shape.d_head), dtype=torch.bfloat16, device="cuda")
        mla.mla_prefill(cfg, cache, wd, dev(np.ascontiguousarray(h[:, lo:lo + L])), out, start_pos=lo)
    torch.cuda.synchronize()
    assert int(cache.err_flags.item()) == 0
    got = host(out)
    pool = cache.pool.cpu().numpy()
    toks = np.array([0, 1, 31, 32, 63, 64, 127, 129])
    for b in range(2):
        ref, rows = om.prefill(h[b], w, shape.n_heads, shape.rms_eps, shape.rope_base, shape.scale,
                               tokens=200 + toks, heads=[0, 64, 127], kv_fp8=True)
        err = rel_l2(got[b][toks][:, [0, 64, 127]], ref)
        rerr = rel_l2(_deq(om.paged_gather(pool, bt, b, 330, shape.page_size)), rows)
        print(f"b={b} rel_l2={err:.3e} rows={rerr:.3e}", flush=True)
        assert err <= BF16_TOL
        assert rerr <= BF16_TOL


@pytest.mark.parametrize("form", FORMS)
def test_fp8_prefill_8192_sampled(form):
    """B=1, L=8192 over an FP8 cache; sampled (token, head) and every cached row."""
    shape = S
    cfg = _cfg(shape)
    cfg.prefill_form = form
    L = 8192
    w = mi.weights(114, shape)
    h = mi.hidden(114, shape, 1, L)
    bt, npages = mi.block_table(114, [L], shape.page_size, shuffle=True)
    cache = _cache(cfg, npages, bt)
    out = torch.empty((1, L, shape.n_heads, shape.d_head), dtype=torch.bfloat16, device="cuda")
    print(f"[fp8 prefill 8192] form={form}", flush=True)
    mla.mla_prefill(cfg, cache, {k: dev(v) for k, v in w.items()}, dev(h), out)
    torch.cuda.synchronize()
    assert int(cache.err_flags.item()) == 0
    toks = np.array([0, 1, 31, 32, 1000, 4095, 4096, 8190, 8191])
    ref, rows = om.prefill(h[0], w, shape.n_heads, shape.rms_eps, shape.rope_base, shape.scale, tokens=toks,
                           heads=[0, 63, 127], kv_fp8=True)
    err = rel_l2(host(out)[0][toks][:, [0, 63, 127]], ref)
    rerr = rel_l2(_deq(om.paged_gather(cache.pool.cpu().numpy(), bt, 0, L, shape.page_size)), rows)
    print(f"rel_l2={err:.3e} rows={rerr:.3e}")
    assert err <= BF16_TOL
    assert rerr <= BF16_TOL


def test_fp8_decode_bench_workload_sampled():
    """The timed FP8 decode workload: B=64 sequences x 4097 tokens, s_q=1,
    64-token shuffled pages, the full step (all 64 x 128 outputs computed);
    the oracle checks three sequences on three heads."""
    seqs, heads = [0, 31, 63], [0, 77, 127]
    shape = _shape(64)
    cfg = _cfg(shape)
    inp = mi.decode_inputs(2, shape, mi.config_context_lens(2), 1)
    g = _gains(2)
    bt, npages = mi.block_table(2, inp.kv_lens, 64, shuffle=True)
    cache = _cache(cfg, npages, bt)
    raws = [inp.seq_rows(b) for b in range(len(inp.kv_lens))]
    print("[fp8 decode B=64 x 4097]", flush=True)
    _append(cfg, cache, raws, g)
    out = torch.empty((64, 1, shape.n_heads, shape.d_head), dtype=torch.bfloat16, device="cuda")
    mla.mla_decode(cfg, cache, torch.from_numpy(inp.kv_lens).to("cuda"), int(inp.kv_lens.max()), dev(inp.q_nope),
                   dev(inp.q_pe), dev(inp.w_uk), dev(inp.w_uv), out)
    torch.cuda.synchronize()
    assert int(cache.err_flags.item()) == 0
    got = host(out)
    assert np.isfinite(got).all()
    rows8 = [_oracle_rows(raws[b], g, shape)[3] if b in seqs else None for b in range(len(raws))]
    ref = om.decode(rows8, inp.kv_lens, 1, inp.q_nope, inp.q_pe, inp.w_uk, inp.w_uv, shape.d_c, shape.scale,
                    seqs=seqs, heads=heads)
    for k, b in enumerate(seqs):
        err = rel_l2(got[b][:, heads], ref[k])
        print(f"b={b} rel_l2={err:.3e}")
        assert err <= BF16_TOL


def test_fp8_decode_bad_page_and_length_are_flagged():
    """With an FP8 cache, a block-table entry outside the pool and a length
    past the bound are reported in err_flags and skipped; the valid row is
    unaffected and the invalid one is written as zeros."""
    shape = _shape(64)
    cfg = _cfg(shape)
    inp = mi.decode_inputs(115, shape, [100, 100], 1)
    g = _gains(115)
    bt, npages = mi.block_table(115, inp.kv_lens, 64, shuffle=True)
    cache = _cache(cfg, npages, bt)
    raws = [inp.seq_rows(b) for b in range(2)]
    _append(cfg, cache, raws, g)
    out = torch.empty((2, 1, shape.n_heads, shape.d_head), dtype=torch.bfloat16, device="cuda")
    args = (dev(inp.q_nope), dev(inp.q_pe), dev(inp.w_uk), dev(inp.w_uv), out)
    bad = cache.block_table.clone()
    bad[0, 1] = npages + 5  # page id past the pool
    mla.mla_decode(cfg, mla.PagedCache(cache.pool, bad, cache.err_flags),
                   torch.from_numpy(inp.kv_lens).to("cuda"), 101, *args)
    torch.cuda.synchronize()
    assert int(cache.err_flags.item()) & mla.MLA_FLAG_BAD_PAGE
    cache.err_flags.zero_()
    mla.mla_decode(cfg, cache, torch.tensor([101, 500], dtype=torch.int32, device="cuda"), 101, *args)
    torch.cuda.synchronize()
    assert int(cache.err_flags.item()) & mla.MLA_FLAG_BAD_LEN
    assert torch.all(out[1].float() == 0)
    ref = om.decode([_oracle_rows(raws[0], g, shape)[3]], inp.kv_lens[:1], 1, inp.q_nope[:1], inp.q_pe[:1],
                    inp.w_uk, inp.w_uv, shape.d_c, shape.scale)
    assert rel_l2(host(out)[0:1], ref) <= BF16_TOL


def test_fp8_decode_hip_graph_replay_matches_eager():
    """The FP8 decode step captured in a HIP graph replays bit-identically to
    eager launches, with eager work between replays."""
    shape = _shape(64)
    cfg = _cfg(shape)
    inp = mi.decode_inputs(116, shape, [40, 300, 1000, 2047], 1)
    bt, npages = mi.block_table(116, inp.kv_lens, 64, shuffle=True)
    cache = _cache(cfg, npages, bt)
    _append(cfg, cache, [inp.seq_rows(b) for b in range(4)], _gains(116))
    max_kv = int(inp.kv_lens.max())
    out = torch.empty((4, 1, shape.n_heads, shape.d_head), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mla.mla_decode_workspace_size(cfg, 4, 1, max_kv), dtype=torch.uint8, device="cuda")
    t = [torch.from_numpy(inp.kv_lens).to("cuda"), dev(inp.q_nope), dev(inp.q_pe), dev(inp.w_uk), dev(inp.w_uv)]

    def step():
        mla.mla_decode(cfg, cache, t[0], max_kv, t[1], t[2], t[3], t[4], out, ws=ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for i in range(3):
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs"
        step()  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("L", [300, 20224, 20225])
def test_fp8_project_kv_both_sides_of_the_stream_k_form(L):
    """[W^DKV ; W^KR] h then the FP8 append, where the projection runs in the
    stream-K form and the append adds its partial sums (300 and 20,224
    tokens, the last count with fewer 256-row tiles than stream-K groups) and
    where it runs as one plain launch (20,225); sampled rows against the
    oracle's FP8 rows."""
    shape = S
    cfg = _cfg(shape)
    w = mi.weights(117, shape)
    h = mi.hidden(117 + L, shape, 1, L)
    bt, npages = mi.block_table(117, [L], shape.page_size, shuffle=True)
    cache = _cache(cfg, npages, bt)
    print(f"[fp8 project_kv] L={L}", flush=True)
    mla.mla_project_kv(cfg, cache, {k: dev(w[k]) for k in ("w_dkv", "w_kr", "g_kv")}, dev(h))
    torch.cuda.synchronize()
    assert int(cache.err_flags.item()) == 0
    pool = cache.pool.cpu().numpy()
    toks = np.unique(np.array([0, 1, 255, 256, 4095, L // 2, L - 257, L - 256, L - 2, L - 1]) % L)
    c, kr = om.latent_rows(h[0][toks], w["w_dkv"], w["g_kv"], w["w_kr"], toks, shape.rms_eps, shape.rope_base)
    ref = np.concatenate([om.quantize_latent_fp8(c)[2], kr], axis=1)
    got = _deq(np.stack([pool[om.paged_slot(bt, 0, int(t), shape.page_size)] for t in toks]))
    err = rel_l2(got, ref)
    print(f"rows rel_l2={err:.3e}")
    assert err <= BF16_TOL
