"""Cache append: indexing is bit-exact, values follow RMSNorm and RoPE."""
import numpy as np
import pytest
import torch

import head_latent_attention_06_amd as mla
import mla_inputs as mi
from mla_testutil import BF16_TOL, SENTINEL, config, dev, host, paged_cache, rel_l2
from oracle import mla_oracle as om

pytestmark = pytest.mark.gpu


def _append(shape, bt, npages, ckv, kr, g, seq, pos, dtype=torch.bfloat16):
    cfg = config(shape, dtype)
    cache = paged_cache(cfg, npages, bt)
    mla.mla_cache_append(cfg, cache, dev(ckv, dtype), dev(kr, dtype), dev(g, dtype),
                         torch.from_numpy(np.asarray(seq, np.int32)).cuda(),
                         torch.from_numpy(np.asarray(pos, np.int32)).cuda())
    torch.cuda.synchronize()
    return cache


def test_append_indexing_bit_exact_and_values():
    s = mi.V3
    kv = np.array([1, 64, 65, 200, 7])
    n = int(kv.sum())
    seq = np.repeat(np.arange(len(kv)), kv)
    pos = np.concatenate([np.arange(k) for k in kv])
    perm = mi.rng(41, 99).permutation(n)            # append in a scrambled order
    seq, pos = seq[perm], pos[perm]
    ckv, kr = mi.append_inputs(41, s, n)
    g = mi.round_to_bf16(mi.rng(41, 98).uniform(0.5, 1.5, s.d_c).astype(np.float32))
    bt_s, npages = mi.block_table(41, kv, s.page_size, shuffle=True, spare_pages=3)
    bt_i, _ = mi.block_table(41, kv, s.page_size, shuffle=False, spare_pages=3)
    c_s = _append(s, bt_s, npages, ckv, kr, g, seq, pos)
    c_i = _append(s, bt_i, npages, ckv, kr, g, seq, pos)
    assert int(c_s.err_flags.item()) == 0 and int(c_i.err_flags.item()) == 0
    ps = c_s.pool.view(torch.int16).cpu().numpy()
    pi = c_i.pool.view(torch.int16).cpu().numpy()
    touched = np.zeros(ps.shape[:2], bool)
    for b, k in enumerate(kv):
        for p in range(k):
            a = ps[om.paged_slot(bt_s, b, p, s.page_size)]
            c = pi[om.paged_slot(bt_i, b, p, s.page_size)]
            assert np.array_equal(a, c)              # same row through either table
            touched[om.paged_slot(bt_s, b, p, s.page_size)] = True
    sent = np.int16(SENTINEL - 65536)
    assert np.all(ps[~touched] == sent)              # untouched slots keep the sentinel
    # values: each written row against its token's oracle row
    pool = host(c_s.pool)
    for i in range(n):
        b, p = int(seq[i]), int(pos[i])
        ref = om.cache_row(ckv[i], kr[i], g, p, s.rms_eps, s.rope_base)
        got = pool[om.paged_slot(bt_s, b, p, s.page_size)]
        assert rel_l2(got, ref) <= 4e-3


def test_append_large_positions_rope():
    """Positions up to 131071: angles formed in double precision."""
    s = mi.V3
    n = 8
    pos = np.array([0, 1, 4095, 4096, 32767, 65536, 131070, 131071])
    seq = np.zeros(n, np.int32)
    ckv, kr = mi.append_inputs(42, s, n)
    g = np.ones(s.d_c, np.float32)
    bt = np.arange(131072 // 64, dtype=np.int32)[None, :]
    cache = _append(s, bt, bt.shape[1], ckv, kr, g, seq, pos)
    pool = host(cache.pool)
    for i in range(n):
        ref = om.cache_row(ckv[i], kr[i], g, int(pos[i]), s.rms_eps, s.rope_base)
        got = pool[om.paged_slot(bt, 0, int(pos[i]), 64)]
        assert rel_l2(got[s.d_c:], ref[s.d_c:]) <= 4e-3


def test_append_rejects_out_of_range_rows():
    s = mi.V3
    bt, npages = mi.block_table(43, [64], s.page_size)
    ckv, kr = mi.append_inputs(43, s, 3)
    g = np.ones(s.d_c, np.float32)
    cache = _append(s, bt, npages, ckv, kr, g, [0, 1, 0], [3, 3, 64])  # seq 1 missing, pos 64 past table
    flags = int(cache.err_flags.item())
    assert flags & mla.MLA_FLAG_BAD_SEQ and flags & mla.MLA_FLAG_BAD_POS
    written = (cache.pool.view(torch.int16) != np.int16(SENTINEL - 65536)).any(-1).cpu().numpy()
    assert written.sum() == 1                       # only (seq 0, pos 3)


def test_append_empty_is_noop():
    s = mi.V3
    bt, npages = mi.block_table(44, [10], s.page_size)
    cfg = config(s)
    cache = paged_cache(cfg, npages, bt)
    e = torch.empty((0, s.d_c), dtype=torch.bfloat16, device="cuda")
    mla.mla_cache_append(cfg, cache, e, torch.empty((0, s.d_rope), dtype=torch.bfloat16, device="cuda"),
                         torch.ones(s.d_c, dtype=torch.bfloat16, device="cuda"),
                         torch.empty(0, dtype=torch.int32, device="cuda"), torch.empty(0, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert (cache.pool.view(torch.int16) == np.int16(SENTINEL - 65536)).all()
