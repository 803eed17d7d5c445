"""mla_decode_noalloc: decode with the library's per-GPU scratch array as its
workspace, against mla_decode with a caller-allocated workspace.

Two calls in a row share the scratch array (the second with a smaller input,
so it runs over what the first left there).  Where both entry points make the
same split plan the results are bit-identical; where the scratch holds fewer
split slots than the usual workspace (a large ragged batch) the plan cuts
fewer, longer chunks and the results agree to the bf16 bar, and both match
the oracle.
"""
import numpy as np
import pytest
import torch

import head_latent_attention_06_amd as mla
import mla_inputs as mi
from mla_testutil import BF16_TOL, decode_setup, host, oracle_decode, rel_l2

pytestmark = pytest.mark.gpu


def _both(inp, config_id):
    cfg, cache, bt, t = decode_setup(inp, config_id=config_id)
    B, s_q = len(inp.kv_lens), inp.s_q
    max_kv = int(inp.kv_lens.max())
    ref = torch.empty((B, s_q, cfg.n_heads, cfg.d_head), dtype=torch.bfloat16, device="cuda")
    mla.mla_decode(cfg, cache, t["kv_lens"], max_kv, t["q_nope"], t["q_pe"], t["w_uk"], t["w_uv"], ref)
    got = torch.full_like(ref, float("nan"))
    print(f"[noalloc] B={B} s_q={s_q} max_kv={max_kv}", flush=True)
    mla.mla_decode_noalloc(cfg, cache, t["kv_lens"], max_kv, t["q_nope"], t["q_pe"], t["w_uk"], t["w_uv"], got)
    torch.cuda.synchronize()
    assert int(cache.err_flags.item()) == 0
    return got, ref


def test_noalloc_matches_decode_two_calls_second_smaller():
    # 1: the B = 64 x 4097 decode workload; its usual workspace (154 MiB) is
    # larger than the scratch, so fewer slots are carved, but a uniform batch
    # needs only 256 of them: the same plan, bit-identical output
    inp = mi.decode_inputs(501, mi.V3, [4096] * 64, 1)
    got, ref = _both(inp, 501)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    seqs, heads = [0, 63], [0, 127]
    assert rel_l2(host(got)[seqs][:, :, heads], oracle_decode(inp, seqs=seqs, heads=heads)) <= BF16_TOL
    # 2: smaller, ragged, two queries per sequence, over the scratch the first
    # call left behind
    inp = mi.decode_inputs(502, mi.V3, [0, 31, 64, 300, 2000], 2)
    got, ref = _both(inp, 502)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    assert rel_l2(host(got), oracle_decode(inp)) <= BF16_TOL


def test_noalloc_large_ragged_batch_fewer_slots():
    """B = 128 ragged with two queries (256 rows): the usual workspace is 226 MiB,
    the scratch 128 MiB, so the plan gets fewer slots; then a smaller call."""
    ctx = mi.config_context_lens(5)
    inp = mi.decode_inputs(5, mi.V3, ctx, 2)
    got, ref = _both(inp, 5)
    g, r = host(got), host(ref)
    assert np.isfinite(g).all()
    assert rel_l2(g, r) <= BF16_TOL
    order = np.argsort(inp.kv_lens)
    seqs, heads = [int(order[0]), int(order[64]), int(order[-1])], [3, 90]
    assert rel_l2(g[seqs][:, :, heads], oracle_decode(inp, seqs=seqs, heads=heads)) <= BF16_TOL
    inp = mi.decode_inputs(503, mi.V3, [5000, 70, 1], 2)
    got, ref = _both(inp, 503)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def test_noalloc_rejects_sizes_beyond_the_scratch():
    """1024 query rows need 256 MiB of absorbed queries and latents alone."""
    cfg = mla.Config()
    B = 1024
    pool = torch.zeros((B, 64, cfg.row), dtype=torch.bfloat16, device="cuda")
    cache = mla.PagedCache(pool, torch.arange(B, dtype=torch.int32, device="cuda").view(B, 1))
    q = torch.zeros((B, 1, 128, 128), dtype=torch.bfloat16, device="cuda")
    qp = torch.zeros((B, 1, 128, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((128 * 128, 512), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((B, 1, 128, 128), dtype=torch.bfloat16, device="cuda")
    lens = torch.full((B,), 10, dtype=torch.int32, device="cuda")
    with pytest.raises(mla.MLAError) as e:
        mla.mla_decode_noalloc(cfg, cache, lens, 10, q, qp, w, w, out)
    assert e.value.status == mla.MLA_ERR_WORKSPACE
