"""Decode parity: the HIP path through the C ABI against the float64 oracle.

Workloads are seeded synthetic inputs (``mla_inputs``) with the decode
configurations' shapes; the oracle materialises per-head k and v explicitly.
"""
import numpy as np
import pytest
import torch

import mla_inputs as mi
from mla_testutil import BF16_TOL, decode_setup, host, oracle_decode, rel_l2, run_decode

pytestmark = pytest.mark.gpu


def _case(config_id, contexts, s_q, shape=mi.V3):
    return mi.decode_inputs(config_id, shape, contexts, s_q)


@pytest.mark.parametrize("contexts,s_q", [
    ([0, 1, 31, 32, 33, 63, 64, 65, 100, 300], 1),   # ragged tails around tile/page edges
    ([0, 5, 127, 129, 700], 2),                       # two causal queries per sequence
    ([2047], 1),                                      # one long row, many chunks
])
def test_decode_small_full_compare(contexts, s_q):
    print(f"[decode small] contexts={contexts} s_q={s_q}", flush=True)
    inp = _case(101, contexts, s_q)
    cfg, cache, bt, t = decode_setup(inp)
    out = run_decode(cfg, cache, t, int(inp.kv_lens.max()))
    torch.cuda.synchronize()
    ref = oracle_decode(inp)
    got = host(out)
    assert np.isfinite(got).all()
    err = rel_l2(got, ref)
    print(f"rel_l2={err:.3e}")
    assert err <= BF16_TOL
    for b in range(len(contexts)):  # every sequence on its own, not just the batch
        assert rel_l2(got[b], ref[b]) <= BF16_TOL
    assert int(cache.err_flags.item()) == 0


def test_decode_paged_equals_contiguous():
    """Same rows through a shuffled and an identity block table: bit-identical."""
    inp = _case(102, [70, 200, 513], 1)
    outs = []
    for shuffle in (False, True):
        cfg, cache, bt, t = decode_setup(inp, shuffle=shuffle, config_id=7)
        outs.append(run_decode(cfg, cache, t, int(inp.kv_lens.max())).view(torch.int16).cpu())
    assert torch.equal(outs[0], outs[1])


def test_decode_deterministic():
    inp = _case(103, [1000, 3], 2)
    cfg, cache, bt, t = decode_setup(inp)
    a = run_decode(cfg, cache, t, int(inp.kv_lens.max())).view(torch.int16).cpu()
    b = run_decode(cfg, cache, t, int(inp.kv_lens.max())).view(torch.int16).cpu()
    assert torch.equal(a, b)


def test_decode_split_invariance():
    """A sequence decoded alone or inside a larger batch is cut into different
    chunks by the device plan; the merged result must agree closely."""
    big = _case(104, [4000] + [4000] * 63, 1)
    cfg, cache, bt, t = decode_setup(big)
    out_big = host(run_decode(cfg, cache, t, 4001))
    alone = mi.decode_inputs(104, mi.V3, [4000] * 64, 1)
    # the first sequence alone: same rows and queries
    one = mi.DecodeInputs(alone.shape, alone.kv_lens[:1], 1, alone.rows[:4001], alone.row_offsets[:1],
                          alone.q_nope[:1], alone.q_pe[:1], alone.w_uk, alone.w_uv)
    cfg1, cache1, bt1, t1 = decode_setup(one)
    out_one = host(run_decode(cfg1, cache1, t1, 4001))
    assert rel_l2(out_one[0], out_big[0]) <= 5e-3


def test_decode_v3_batch64_context4096():
    """The B=64 x 4096-context decode workload; oracle on sampled (sequence, head) pairs."""
    ctx = mi.config_context_lens(2)
    inp = _case(2, ctx, 1)
    cfg, cache, bt, t = decode_setup(inp, config_id=2)
    out = run_decode(cfg, cache, t, int(inp.kv_lens.max()))
    got = host(out)
    assert np.isfinite(got).all()
    seqs, heads = [0, 17, 40, 63], [0, 31, 64, 127]
    ref = oracle_decode(inp, seqs=seqs, heads=heads)
    err = rel_l2(got[seqs][:, :, heads], ref)
    print(f"rel_l2(sampled)={err:.3e}")
    assert err <= BF16_TOL
    assert int(cache.err_flags.item()) == 0


def test_decode_long_context_131072():
    """B=4 sequences x 131072 cached tokens (+1 new): long split chains and merge."""
    ctx = mi.config_context_lens(4)
    inp = _case(4, ctx, 1)
    cfg, cache, bt, t = decode_setup(inp, config_id=4)
    got = host(run_decode(cfg, cache, t, int(inp.kv_lens.max())))
    assert np.isfinite(got).all()
    seqs, heads = [0, 3], [5, 100]
    ref = oracle_decode(inp, seqs=seqs, heads=heads)
    err = rel_l2(got[seqs][:, :, heads], ref)
    print(f"rel_l2(sampled)={err:.3e}")
    assert err <= BF16_TOL


def test_decode_ragged_paged_s_q2():
    """B=128, context ~ U{1..32768}, 2 causal queries per sequence, shuffled pages."""
    ctx = mi.config_context_lens(5)
    inp = _case(5, ctx, 2)
    cfg, cache, bt, t = decode_setup(inp, config_id=5)
    got = host(run_decode(cfg, cache, t, int(inp.kv_lens.max())))
    assert np.isfinite(got).all()
    order = np.argsort(inp.kv_lens)
    seqs = [int(order[0]), int(order[1]), int(order[64]), int(order[-1])]  # shortest, middle, longest
    heads = [0, 77]
    ref = oracle_decode(inp, seqs=seqs, heads=heads)
    err = rel_l2(got[seqs][:, :, heads], ref)
    print(f"kv_lens={inp.kv_lens[seqs]} rel_l2(sampled)={err:.3e}")
    assert err <= BF16_TOL
    assert int(cache.err_flags.item()) == 0


def test_decode_bad_page_and_length_are_flagged():
    """Block-table entries outside the pool and lengths past the bound are
    reported in err_flags; the kernels skip them (no access outside the pool)."""
    import head_latent_attention_06_amd as mla
    inp = _case(106, [100, 100], 1)
    cfg, cache, bt, t = decode_setup(inp, config_id=106)
    bad = cache.block_table.clone()
    bad[0, 1] = cache.pool.shape[0] + 5           # page id past the pool
    cache_bad = mla.PagedCache(cache.pool, bad, cache.err_flags)
    run_decode(cfg, cache_bad, t, 101)
    torch.cuda.synchronize()
    assert int(cache.err_flags.item()) & mla.MLA_FLAG_BAD_PAGE
    cache.err_flags.zero_()
    t2 = dict(t)
    t2["kv_lens"] = torch.tensor([101, 500], dtype=torch.int32, device="cuda")  # 500 > max_kv_len
    out = run_decode(cfg, cache, t2, 101)
    torch.cuda.synchronize()
    assert int(cache.err_flags.item()) & mla.MLA_FLAG_BAD_LEN
    assert torch.all(out[1].float() == 0)          # the invalid row is written as zeros
    ref = oracle_decode(inp, seqs=[0])
    assert rel_l2(host(out)[0:1], ref) <= BF16_TOL  # the valid row is unaffected


def test_decode_hip_graph_replay_matches_eager():
    """The decode step (absorption GEMM with the plan, attention, merge + W^UV)
    issues no memset, copy or synchronisation, so a caller can capture it in a
    HIP graph.  Every replay (with eager work and synchronisations between
    replays) must equal the eager result bit for bit, and a replay after the
    queries change in place must follow them."""
    import head_latent_attention_06_amd as mla
    from mla_testutil import dev
    inp = _case(111, [40, 300, 1000, 2047], 1)
    cfg, cache, bt, t = decode_setup(inp)
    max_kv = int(inp.kv_lens.max())
    B, s_q, H = t["q_nope"].shape[0], t["q_nope"].shape[1], cfg.n_heads
    out = torch.empty((B, s_q, H, cfg.d_head), dtype=cfg.dtype, device="cuda")
    ws = torch.empty(mla.mla_decode_workspace_size(cfg, B, s_q, max_kv), dtype=torch.uint8, device="cuda")

    def step():
        mla.mla_decode(cfg, cache, t["kv_lens"], max_kv, t["q_nope"], t["q_pe"], t["w_uk"], t["w_uv"], out, ws=ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    assert rel_l2(host(eager), oracle_decode(inp)) <= BF16_TOL
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        out.zero_()
        filler = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        print(f"replay {rep}: equal={torch.equal(out, eager)} filler={float(filler):.2f}", flush=True)
        assert torch.equal(out, eager)
    # new queries in the same buffers: the replay must use them
    inp2 = mi.decode_inputs(112, mi.V3, [40, 300, 1000, 2047], 1)
    t["q_nope"].copy_(dev(inp2.q_nope, torch.bfloat16))
    t["q_pe"].copy_(dev(inp2.q_pe, torch.bfloat16))
    step()
    torch.cuda.synchronize()
    eager2 = out.clone()
    assert not torch.equal(eager2, eager)
    out.zero_()
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, eager2)
    assert int(cache.err_flags.item()) == 0


@pytest.mark.parametrize("page_size", [32, 128])
def test_decode_other_page_sizes(page_size):
    """32- and 128-token pages (the tile/page walk with one and four tiles per
    page), lengths around tile and page edges, two causal queries."""
    import dataclasses
    s = dataclasses.replace(mi.V3, page_size=page_size)
    inp = mi.decode_inputs(121, s, [1, 31, 32, 33, 95, 96, 97, 127, 129, 500, 1100], 2)
    cfg, cache, bt, t = decode_setup(inp)
    assert cfg.page_size == page_size
    out = run_decode(cfg, cache, t, int(inp.kv_lens.max()))
    torch.cuda.synchronize()
    got = host(out)
    ref = oracle_decode(inp)
    err = rel_l2(got, ref)
    print(f"page_size={page_size} rel_l2={err:.3e}", flush=True)
    assert err <= BF16_TOL
    for b in range(len(inp.kv_lens)):
        assert rel_l2(got[b], ref[b]) <= BF16_TOL
    assert int(cache.err_flags.item()) == 0
