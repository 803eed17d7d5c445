"""Pins for the float64 oracle: checks against things other than the oracle itself.

Each test names what fixes the expected value: a closed form, an identity the
notes page derives, a library routine the method reduces to in a special case,
a brute-force loop written from the definitions, or a value the pages print
(``tests/golden``).  A plausible slip in the oracle -- a dropped RoPE term, a
wrong sign, a transposed per-head block, an off-by-one causal mask, a wrong
scale -- fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import mla_inputs as mi
from oracle import mla_oracle as om

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "v3_mla_constants.json")


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _rand_setup(seed, H=3, dh=4, dr=2, dc=6, dcq=5, d=7, L=6):
    r = np.random.default_rng(seed)
    w = {
        "w_dq": r.standard_normal((dcq, d)), "g_q": r.uniform(0.5, 1.5, dcq),
        "w_uq": r.standard_normal((H * dh, dcq)), "w_qr": r.standard_normal((H * dr, dcq)),
        "w_dkv": r.standard_normal((dc, d)), "g_kv": r.uniform(0.5, 1.5, dc),
        "w_kr": r.standard_normal((dr, d)),
        "w_uk": r.standard_normal((H * dh, dc)), "w_uv": r.standard_normal((H * dh, dc)),
    }
    h = r.standard_normal((L, d))
    return w, h


# ---------------------------------------------------------------------------
# Brute force (P4): scalar loops written straight from steps (1)-(10) of the
# notes page, no matrix library.  Tiny shapes only.
# ---------------------------------------------------------------------------
def _bf_matvec(W, x):
    return [sum(W[r][k] * x[k] for k in range(len(x))) for r in range(len(W))]


def _bf_rms(x, g, eps):
    ms = sum(v * v for v in x) / len(x)
    return [x[k] / math.sqrt(ms + eps) * g[k] for k in range(len(x))]


def _bf_theta(p, d, base, yarn=None):
    """Frequency of pair p.  With ``yarn`` (s, alpha, beta, orig_ctx): count the
    pair's turns over the original window, r = orig_ctx * theta / (2 pi); at
    r <= alpha the frequency is divided by s, at r >= beta it is kept, and in
    between the two are blended linearly in r."""
    th = base ** (-2.0 * p / d)
    if yarn is None:
        return th
    r = yarn["orig_ctx"] * th / (2.0 * math.pi)
    if r <= yarn["alpha"]:
        blend = 0.0
    elif r >= yarn["beta"]:
        blend = 1.0
    else:
        blend = (r - yarn["alpha"]) / (yarn["beta"] - yarn["alpha"])
    return blend * th + (1.0 - blend) * (th / yarn["s"])


def _bf_rope(x, pos, base, yarn=None):
    d = len(x)
    y = list(x)
    for p in range(d // 2):
        th = pos * _bf_theta(p, d, base, yarn)
        c, s = math.cos(th), math.sin(th)
        # R = [[c, -s], [s, c]] applied to the column (x_2p, x_2p+1)
        y[2 * p] = c * x[2 * p] - s * x[2 * p + 1]
        y[2 * p + 1] = s * x[2 * p] + c * x[2 * p + 1]
    return y


def _bf_fp8_latent(x):
    """c^KV as the FP8 cache holds it, one 128-value tile at a time: the
    tile's power of two 2^e (smallest e with max|x| <= 448 * 2^e), each value
    divided by it in float32, rounded by torch's float8_e4m3fn conversion and
    multiplied back."""
    out = []
    for t0 in range(0, len(x), 128):
        tile = [float(np.float32(v)) for v in x[t0:t0 + 128]]
        amax = max(abs(v) for v in tile)
        e = 0
        if amax > 0:
            while amax > 448.0 * 2.0 ** e:
                e += 1
            while amax <= 448.0 * 2.0 ** (e - 1):
                e -= 1
        q = torch.tensor([v / 2.0 ** e for v in tile], dtype=torch.float32).to(torch.float8_e4m3fn)
        out += [float(v) * 2.0 ** e for v in q.to(torch.float64).tolist()]
    return out


def _bf_prefill(h, w, H, eps, base, yarn=None, kv_fp8=False):
    """Steps (1)-(10) in scalar loops.  ``yarn``: YaRN frequencies on q^R and
    k^R, every logit times (0.1 ln s + 1)^2.  ``kv_fp8``: c^KV read back
    through the FP8 cache format (k^R untouched)."""
    W = {k: np.asarray(v).tolist() for k, v in w.items()}
    L = len(h)
    dh = len(W["w_uq"]) // H
    dr = len(W["w_kr"])
    hs = np.asarray(h).tolist()
    q, k, v = [], [], []
    for t in range(L):
        cq = _bf_rms(_bf_matvec(W["w_dq"], hs[t]), W["g_q"], eps)            # (1)
        qc = _bf_matvec(W["w_uq"], cq)                                       # (2)
        qr_all = _bf_matvec(W["w_qr"], cq)                                   # (3)
        ckv = _bf_rms(_bf_matvec(W["w_dkv"], hs[t]), W["g_kv"], eps)         # (5)
        if kv_fp8:
            ckv = _bf_fp8_latent(ckv)
        kc = _bf_matvec(W["w_uk"], ckv)                                      # (6)
        kr = _bf_rope(_bf_matvec(W["w_kr"], hs[t]), t, base, yarn)           # (7)
        vc = _bf_matvec(W["w_uv"], ckv)                                      # (9)
        q.append([qc[i * dh:(i + 1) * dh] + _bf_rope(qr_all[i * dr:(i + 1) * dr], t, base, yarn)
                  for i in range(H)])                                        # (4)
        k.append([kc[i * dh:(i + 1) * dh] + kr for i in range(H)])           # (8)
        v.append([vc[i * dh:(i + 1) * dh] for i in range(H)])
    scale = 1.0 / math.sqrt(dh + dr)
    if yarn is not None:
        scale *= (0.1 * math.log(yarn["s"]) + 1.0) ** 2
    out = np.zeros((L, H, dh))
    for t in range(L):                                                       # (10)
        for i in range(H):
            sc = [sum(a * b for a, b in zip(q[t][i], k[j][i])) * scale for j in range(t + 1)]
            m = max(sc)
            e = [math.exp(s - m) for s in sc]
            tot = sum(e)
            for j in range(t + 1):
                for a in range(dh):
                    out[t, i, a] += e[j] / tot * v[j][i][a]
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_p4_bruteforce_matches_oracle(seed):
    w, h = _rand_setup(seed)
    H, eps, base = 3, 1e-6, 10000.0
    ref = _bf_prefill(h, w, H, eps, base)
    o, _ = om.prefill(h, w, H, eps, base, scale=1.0 / math.sqrt(4 + 2))
    assert _rel(o, ref) <= 1e-13


def test_p4_bruteforce_tiny_base_large_angles():
    # a small RoPE base makes every pair rotate visibly, so a pairing slip shows
    w, h = _rand_setup(7, L=5)
    ref = _bf_prefill(h, w, 3, 1e-6, 3.0)
    o, _ = om.prefill(h, w, 3, 1e-6, 3.0, scale=1.0 / math.sqrt(6))
    assert _rel(o, ref) <= 1e-13


# ---------------------------------------------------------------------------
# P1: absorbed form == explicit form (【思考】 on absorption)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [0, 1])
def test_p1_absorbed_equals_explicit(seed):
    r = np.random.default_rng(100 + seed)
    H, dh, dr, dc, N, T = 4, 8, 4, 16, 23, 5
    q_c = r.standard_normal((T, H, dh))
    q_r = r.standard_normal((T, H, dr))
    c = r.standard_normal((N, dc))
    k_r = r.standard_normal((N, dr))
    w_uk = r.standard_normal((H * dh, dc)) / 4
    w_uv = r.standard_normal((H * dh, dc)) / 4
    q_pos = np.array([0, 5, 11, 17, 22])
    a = om.explicit_attention(q_c, q_r, c, k_r, w_uk, w_uv, q_pos, 0.3)
    b = om.absorbed_attention(q_c, q_r, c, k_r, w_uk, w_uv, q_pos, 0.3)
    assert _rel(b, a) <= 1e-12
    # a subset of heads, in another order, is those heads of the whole
    sub = om.absorbed_attention(q_c, q_r, c, k_r, w_uk, w_uv, q_pos, 0.3, heads=[3, 1])
    assert _rel(sub, a[:, [3, 1]]) <= 1e-12


# ---------------------------------------------------------------------------
# P2: with d_c = n_h d_h and identity up-projections MLA is textbook causal MHA,
# checked against torch's scaled_dot_product_attention in float64 on the CPU.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("zero_rope", [False, True])
def test_p2_reduces_to_mha(zero_rope):
    r = np.random.default_rng(5)
    H, dh, dr, L = 3, 4, 2, 9
    dc = H * dh
    q_c = r.standard_normal((L, H, dh))
    q_r = np.zeros((L, H, dr)) if zero_rope else r.standard_normal((L, H, dr))
    c = r.standard_normal((L, dc))
    k_r = np.zeros((L, dr)) if zero_rope else r.standard_normal((L, dr))
    eye = np.eye(dc)
    scale = 1.0 / math.sqrt(dh + dr)
    o = om.explicit_attention(q_c, q_r, c, k_r, eye, eye, np.arange(L), scale)
    # MHA: head i's key is [c_j block i ; k^R_j], value is c_j block i
    q = torch.from_numpy(np.concatenate([q_c, q_r], axis=2)).permute(1, 0, 2)          # [H, L, E]
    kb = np.stack([np.concatenate([c[:, i * dh:(i + 1) * dh], k_r], axis=1) for i in range(H)])
    vb = np.stack([c[:, i * dh:(i + 1) * dh] for i in range(H)])
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, torch.from_numpy(kb), torch.from_numpy(vb), is_causal=True, scale=scale)
    assert _rel(o, ref.permute(1, 0, 2).numpy()) <= 1e-12


def test_p2_permuted_up_projection_matches_mha():
    # a non-symmetric (permutation) W^UK catches a transposed per-head block
    r = np.random.default_rng(6)
    H, dh, dr, L = 2, 3, 2, 7
    dc = H * dh
    perm = r.permutation(dc)
    P = np.eye(dc)[perm]
    q_c = r.standard_normal((L, H, dh))
    q_r = r.standard_normal((L, H, dr))
    c = r.standard_normal((L, dc))
    k_r = r.standard_normal((L, dr))
    scale = 1.0 / math.sqrt(dh + dr)
    o = om.explicit_attention(q_c, q_r, c, k_r, P, np.eye(dc), np.arange(L), scale)
    pc = c[:, perm]                       # (P c_j) = c_j permuted
    q = torch.from_numpy(np.concatenate([q_c, q_r], axis=2)).permute(1, 0, 2)
    kb = np.stack([np.concatenate([pc[:, i * dh:(i + 1) * dh], k_r], axis=1) for i in range(H)])
    vb = np.stack([c[:, i * dh:(i + 1) * dh] for i in range(H)])
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, torch.from_numpy(kb), torch.from_numpy(vb), is_causal=True, scale=scale)
    assert _rel(o, ref.permute(1, 0, 2).numpy()) <= 1e-12


# ---------------------------------------------------------------------------
# P3: softmax weights are a distribution over the visible rows
# ---------------------------------------------------------------------------
def test_p3_weights_are_causal_distributions():
    r = np.random.default_rng(9)
    H, dh, dr, dc, N = 3, 4, 2, 8, 12
    q_pos = np.array([0, 3, 11])
    _, a = om.explicit_attention(r.standard_normal((3, H, dh)), r.standard_normal((3, H, dr)),
                                 r.standard_normal((N, dc)), r.standard_normal((N, dr)),
                                 r.standard_normal((H * dh, dc)), r.standard_normal((H * dh, dc)),
                                 q_pos, 0.5, return_weights=True)
    assert np.all(a >= 0)
    assert np.max(np.abs(a.sum(axis=2) - 1.0)) <= 1e-12
    for t, p in enumerate(q_pos):
        assert np.all(a[t, :, p + 1:] == 0.0)
        assert np.all(a[t, :, :p + 1] > 0.0)


# ---------------------------------------------------------------------------
# P5: RoPE
# ---------------------------------------------------------------------------
def test_p5_rope_matches_complex_rotation():
    r = np.random.default_rng(11)
    x = r.standard_normal((5, 8))
    pos = np.array([0, 1, 7, 100, 131072])
    y = om.rope(x, pos, 10000.0)
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * np.exp(1j * pos[:, None] * 10000.0 ** (-np.arange(4) * 2 / 8))
    assert np.max(np.abs(y[:, 0::2] - z.real)) <= 1e-12
    assert np.max(np.abs(y[:, 1::2] - z.imag)) <= 1e-12


def test_p5_rope_block_from_page():
    g = json.load(open(GOLDEN))["rope_block"]
    assert g["rotate_unit_x"] == "cos_sin"
    y = om.rope(np.array([1.0, 0.0]), 3, 10000.0)        # theta_0 = 1, angle 3
    assert np.allclose(y, [math.cos(3.0), math.sin(3.0)], atol=1e-15)


def test_p5_rope_identity_at_zero_and_norm_preserving():
    r = np.random.default_rng(12)
    x = r.standard_normal((4, 64))
    assert np.array_equal(om.rope(x, np.zeros(4), 10000.0), x)
    y = om.rope(x, np.array([1, 50, 4097, 32769]), 10000.0)
    for p in range(32):
        assert np.allclose(np.hypot(y[:, 2 * p], y[:, 2 * p + 1]), np.hypot(x[:, 2 * p], x[:, 2 * p + 1]),
                           rtol=1e-13)


def test_p5_scores_depend_only_on_relative_position():
    r = np.random.default_rng(13)
    H, dh, dr, dc, N = 2, 4, 6, 8, 10
    q_c = r.standard_normal((3, H, dh))
    q_raw = r.standard_normal((3, H, dr))
    c = r.standard_normal((N, dc))
    k_raw = r.standard_normal((N, dr))
    w_uk = r.standard_normal((H * dh, dc))
    w_uv = r.standard_normal((H * dh, dc))
    q_pos = np.array([2, 6, 9])
    outs = []
    for shift in [0, 17, 4093]:
        q_r = om.rope(q_raw, (q_pos + shift)[:, None], 10000.0)
        k_r = om.rope(k_raw, np.arange(N) + shift, 10000.0)
        outs.append(om.explicit_attention(q_c, q_r, c, k_r, w_uk, w_uv, q_pos, 0.4))
    assert _rel(outs[1], outs[0]) <= 1e-10 and _rel(outs[2], outs[0]) <= 1e-10


# ---------------------------------------------------------------------------
# RMSNorm
# ---------------------------------------------------------------------------
def test_rmsnorm_closed_forms():
    g = np.linspace(0.5, 1.5, 16)
    # a constant vector c*1 normalises to g * c / sqrt(c^2 + eps)
    y = om.rms_norm(np.full(16, 3.0), g, 1e-6)
    assert np.allclose(y, g * 3.0 / math.sqrt(9.0 + 1e-6), rtol=1e-15)
    r = np.random.default_rng(14)
    x = r.standard_normal((3, 16))
    y0 = om.rms_norm(x, np.ones(16), 0.0)
    assert np.allclose(np.mean(y0 * y0, axis=1), 1.0, rtol=1e-14)
    assert np.allclose(om.rms_norm(7.5 * x, np.ones(16), 0.0), y0, rtol=1e-14)
    assert np.allclose(om.rms_norm(x, g, 0.0), y0 * g, rtol=1e-14)


# ---------------------------------------------------------------------------
# P6: closed forms of attention
# ---------------------------------------------------------------------------
def test_p6_first_token_and_identical_keys():
    r = np.random.default_rng(15)
    H, dh, dr, dc, N = 3, 4, 2, 8, 9
    q_c = r.standard_normal((2, H, dh))
    q_r = r.standard_normal((2, H, dr))
    w_uk = r.standard_normal((H * dh, dc))
    w_uv = r.standard_normal((H * dh, dc))
    c = r.standard_normal((N, dc))
    k_r = r.standard_normal((N, dr))
    o = om.explicit_attention(q_c, q_r, c, k_r, w_uk, w_uv, np.array([0, 0]), 0.7)
    for i in range(H):
        assert np.allclose(o[:, i], (w_uv[i * dh:(i + 1) * dh] @ c[0])[None], rtol=1e-14)
    c_same = np.repeat(c[:1], N, axis=0)
    k_same = np.repeat(k_r[:1], N, axis=0)
    o = om.explicit_attention(q_c, q_r, c_same, k_same, w_uk, w_uv, np.array([N - 1, 4]), 0.7)
    for i in range(H):
        assert np.allclose(o[:, i], (w_uv[i * dh:(i + 1) * dh] @ c[0])[None], rtol=1e-13)


# ---------------------------------------------------------------------------
# P7: merging split partials equals the unsplit softmax
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cuts", [[0, 40], [0, 1, 40], [0, 13, 13, 27, 40], [0, 39, 40]])
def test_p7_merge_identity(cuts):
    r = np.random.default_rng(16)
    dc, dr, N = 12, 4, 40
    c = r.standard_normal((N, dc))
    k_r = r.standard_normal((N, dr))
    q_lat = r.standard_normal(dc) * 2
    q_r = r.standard_normal(dr)
    parts = [om.latent_partial(q_lat, q_r, c, k_r, 0.5, lo, hi) for lo, hi in zip(cuts[:-1], cuts[1:])]
    merged = om.merge_partials([p[0] for p in parts], [p[1] for p in parts], [p[2] for p in parts])
    s = (c @ q_lat + k_r @ q_r) * 0.5
    a = np.exp(s - s.max())
    a /= a.sum()
    assert _rel(merged, a @ c) <= 1e-12


# ---------------------------------------------------------------------------
# P8: layout constants printed on the pages
# ---------------------------------------------------------------------------
def test_p8_layout_constants():
    g = json.load(open(GOLDEN))
    hp = g["v3_hyperparameters"]
    s = mi.V3
    assert (s.n_heads, s.d_head, s.d_c, s.d_cq, s.d_rope, s.d_model) == \
        (hp["n_heads"], hp["d_head"], hp["d_c"], hp["d_cq"], hp["d_rope"], hp["d_model"])
    assert s.d_c == g["v2_ratios"]["d_c_over_d_head"] * s.d_head
    assert s.d_rope == g["v2_ratios"]["d_rope_over_d_head"] * s.d_head
    assert s.row == g["cache_elements_per_token_per_layer"]["mla"]
    assert 2 * s.n_heads * s.d_head == g["cache_elements_per_token_per_layer"]["mha"]
    assert s.d_head + s.d_rope == g["softmax_scale_denominator_squared"]["value"]
    lc = g["long_context_latent_bytes_per_sequence"]
    assert lc["tokens"] * s.row * 2 == lc["bytes"]
    assert round(lc["bytes"] / 1e6) == 151


# ---------------------------------------------------------------------------
# P10 (oracle side): paged placement is a bijection onto the pool
# ---------------------------------------------------------------------------
def test_p10_paged_slots_are_a_bijection():
    kv = np.array([1, 64, 65, 130, 7])
    bt, npages = mi.block_table(3, kv, 64, shuffle=True)
    seen = set()
    for b, n in enumerate(kv):
        for p in range(n):
            slot = om.paged_slot(bt, b, p, 64)
            assert 0 <= slot[0] < npages and 0 <= slot[1] < 64
            assert slot not in seen
            seen.add(slot)
    pool = np.zeros((npages, 64, 3))
    for b, n in enumerate(kv):
        for p in range(n):
            pool[om.paged_slot(bt, b, p, 64)] = (b, p, 1)
    for b, n in enumerate(kv):
        g = om.paged_gather(pool, bt, b, int(n), 64)
        assert np.array_equal(g[:, 0], np.full(n, b)) and np.array_equal(g[:, 1], np.arange(n))


def test_cache_row_is_norm_then_rope():
    r = np.random.default_rng(17)
    c_raw = r.standard_normal(32)
    k_raw = r.standard_normal(8)
    g = r.uniform(0.5, 1.5, 32)
    row = om.cache_row(c_raw, k_raw, g, 5, 1e-6, 10000.0)
    assert np.allclose(row[:32], _bf_rms(list(c_raw), list(g), 1e-6), rtol=1e-14)
    assert np.allclose(row[32:], _bf_rope(list(k_raw), 5, 10000.0), rtol=1e-14, atol=1e-15)


def test_decode_matches_prefill_last_rows():
    # a decode step over rows produced by a prefill gives that prefill's last outputs
    w, h = _rand_setup(21, L=8)
    H, eps, base, scale = 3, 1e-6, 10000.0, 1.0 / math.sqrt(6)
    o, rows = om.prefill(h, w, H, eps, base, scale)
    q_c, q_r = om.query_path(h[6:], w["w_dq"], w["g_q"], w["w_uq"], w["w_qr"], np.array([6, 7]), H, eps, base)
    od = om.decode([rows], [8], 2, q_c[None], q_r[None], w["w_uk"], w["w_uv"], rows.shape[1] - 2, scale)
    assert _rel(od[0], o[6:]) <= 1e-13


def test_prefill_with_past_rows_matches_whole():
    w, h = _rand_setup(22, L=9)
    H, eps, base, scale = 3, 1e-6, 10000.0, 1.0 / math.sqrt(6)
    o_all, rows_all = om.prefill(h, w, H, eps, base, scale)
    o2, rows2 = om.prefill(h[4:], w, H, eps, base, scale, start_pos=4, past_rows=rows_all[:4])
    assert _rel(rows2, rows_all[4:]) <= 1e-14
    assert _rel(o2, o_all[4:]) <= 1e-13


# ---------------------------------------------------------------------------
# YaRN (the long-context extension; frequencies and logit factor)
# ---------------------------------------------------------------------------
def _yarn_page():
    g = json.load(open(GOLDEN))["yarn_hyperparameters"]
    return dict(s=g["s"], alpha=g["alpha"], beta=g["beta"], orig_ctx=g["orig_ctx"]), g


def test_yarn_s1_is_plain_rope():
    y = dict(s=1.0, alpha=1.0, beta=32.0, orig_ctx=4096)
    assert np.allclose(om.yarn_frequencies(64, 10000.0, y), om.rope_frequencies(64, 10000.0), rtol=1e-15, atol=0)
    assert om.yarn_logit_factor(1.0) == 1.0
    r = np.random.default_rng(40)
    x = r.standard_normal((3, 64))
    assert np.allclose(om.rope(x, np.array([0, 5, 70000]), 10000.0, y), om.rope(x, np.array([0, 5, 70000]), 10000.0),
                       rtol=0, atol=1e-9)


def test_yarn_ramp_closed_forms():
    """One pair with theta = 1: its rotations over the original context are
    orig_ctx / (2 pi), so choosing orig_ctx puts it at alpha, beta or halfway."""
    s, a, b = 40.0, 1.0, 32.0
    for ctx, want in [(2 * math.pi * a, 1.0 / s), (2 * math.pi * b, 1.0), (2 * math.pi * (a + b) / 2, (1.0 / s + 1.0) / 2),
                      (2 * math.pi * 0.25, 1.0 / s), (2 * math.pi * 1000.0, 1.0)]:
        th = om.yarn_frequencies(2, 10000.0, dict(s=s, alpha=a, beta=b, orig_ctx=ctx))
        assert abs(th[0] - want) <= 1e-15, (ctx, th[0], want)


def test_yarn_page_values_limits_and_monotone():
    """With the page's values and the V3 RoPE width: the fastest pair (theta = 1,
    ~652 rotations over 4K) is unchanged, the slowest (< 1 rotation) is divided
    by s, and the ratio theta'/theta falls monotonically between."""
    y, _ = _yarn_page()
    base = om.rope_frequencies(64, 10000.0)
    th = om.yarn_frequencies(64, 10000.0, y)
    assert th[0] == base[0] == 1.0
    assert abs(th[31] - base[31] / y["s"]) <= 1e-18
    ratio = th / base
    assert np.all(np.diff(ratio) <= 1e-15) and ratio.min() >= 1.0 / y["s"] - 1e-15 and ratio.max() <= 1.0
    inner = (ratio > 1.0 / y["s"] + 1e-12) & (ratio < 1.0 - 1e-12)
    assert inner.sum() >= 3  # the ramp is populated


def test_yarn_low_frequency_pairs_interpolate_positions():
    """A pair left fully interpolated (g = 0) rotates at position s*m exactly as
    plain RoPE does at m: the context extension of YaRN's low frequencies."""
    y, _ = _yarn_page()
    base = om.rope_frequencies(64, 10000.0)
    th = om.yarn_frequencies(64, 10000.0, y)
    low = np.where(np.abs(th - base / y["s"]) <= 1e-18)[0]
    assert len(low) >= 4
    r = np.random.default_rng(41)
    x = r.standard_normal(64)
    m = np.array([3, 100, 4000])
    a = om.rope(np.tile(x, (3, 1)), m * y["s"], 10000.0, y)
    b = om.rope(np.tile(x, (3, 1)), m, 10000.0)
    for p in low:
        assert np.allclose(a[:, 2 * p:2 * p + 2], b[:, 2 * p:2 * p + 2], atol=1e-9)


def test_yarn_logit_factor_from_page():
    """The page prints sqrt(t) = 0.1 ln s + 1; the logits are multiplied by its
    square (YaRN applies that factor to both q and k)."""
    y, g = _yarn_page()
    c = g["factor_formula_coefficients"]
    sqrt_t = c["a"] * math.log(y["s"]) + c["b"]
    assert abs(om.yarn_logit_factor(y["s"]) - sqrt_t * sqrt_t) <= 1e-15
    assert 1.87 < om.yarn_logit_factor(40.0) < 1.88


def test_yarn_scores_depend_only_on_relative_position():
    y, _ = _yarn_page()
    r = np.random.default_rng(42)
    H, dh, dr, dc, N = 2, 4, 8, 8, 9
    q_c = r.standard_normal((3, H, dh))
    q_raw = r.standard_normal((3, H, dr))
    c = r.standard_normal((N, dc))
    k_raw = r.standard_normal((N, dr))
    w_uk = r.standard_normal((H * dh, dc))
    w_uv = r.standard_normal((H * dh, dc))
    q_pos = np.array([1, 5, 8])
    outs = []
    for shift in [0, 33, 90001]:
        q_r = om.rope(q_raw, (q_pos + shift)[:, None], 10000.0, y)
        k_r = om.rope(k_raw, np.arange(N) + shift, 10000.0, y)
        outs.append(om.explicit_attention(q_c, q_r, c, k_r, w_uk, w_uv, q_pos, 0.4))
    assert _rel(outs[1], outs[0]) <= 1e-9 and _rel(outs[2], outs[0]) <= 1e-9


def test_yarn_prefill_s1_equals_plain_prefill():
    s = mi.TINY
    w = mi.weights(43, s, bf16=False)
    h = mi.hidden(43, s, 1, 12, bf16=False)[0]
    a, ra = om.prefill(h, w, s.n_heads, s.rms_eps, s.rope_base, s.scale)
    b, rb = om.prefill(h, w, s.n_heads, s.rms_eps, s.rope_base, s.scale,
                       yarn=dict(s=1.0, alpha=1.0, beta=32.0, orig_ctx=4096))
    assert _rel(a, b) <= 1e-13 and _rel(ra, rb) <= 1e-13


def test_yarn_prefill_matches_bruteforce():
    """The whole prefill with YaRN at the page's s = 40, alpha = 1, beta = 32:
    scalar loops with the ramp written out pair by pair, the same frequencies
    on q^R and k^R and every logit times (0.1 ln s + 1)^2.  With d_h^R = 8,
    base 10000 and a 4096-token original window the four pairs make
    652, 65, 6.5 and 0.65 turns: two kept, one blended, one divided by s."""
    y, _ = _yarn_page()
    H, dr = 3, 8
    w, h = _rand_setup(11, H=H, dr=dr, L=8)
    turns = [y["orig_ctx"] * 10000.0 ** (-2.0 * p / dr) / (2 * math.pi) for p in range(dr // 2)]
    assert turns[0] > y["beta"] and turns[1] > y["beta"] and y["alpha"] < turns[2] < y["beta"] and turns[3] < y["alpha"]
    ref = _bf_prefill(h, w, H, 1e-6, 10000.0, yarn=y)
    o, _ = om.prefill(h, w, H, 1e-6, 10000.0, scale=1.0 / math.sqrt(4 + dr), yarn=y)
    assert _rel(o, ref) <= 1e-12
    # the pin can tell YaRN from plain RoPE: each of its two parts moves the output
    plain = _bf_prefill(h, w, H, 1e-6, 10000.0)
    assert _rel(plain, ref) > 1e-3


def test_yarn_prefill_parts_are_each_visible():
    """Each half of YaRN alone (frequencies without the logit factor, the
    factor without the frequencies) gives an output the brute force rejects,
    so the pin above fails if either is dropped."""
    y, _ = _yarn_page()
    H, dr = 2, 8
    w, h = _rand_setup(12, H=H, dr=dr, L=6)
    ref = _bf_prefill(h, w, H, 1e-6, 10000.0, yarn=y)
    sc = 1.0 / math.sqrt(4 + dr)
    freq_only, _ = om.prefill(h, w, H, 1e-6, 10000.0, scale=sc / om.yarn_logit_factor(y["s"]), yarn=y)
    factor_only, _ = om.prefill(h, w, H, 1e-6, 10000.0, scale=sc * om.yarn_logit_factor(y["s"]))
    assert _rel(freq_only, ref) > 1e-3 and _rel(factor_only, ref) > 1e-4


def test_fp8_prefill_matches_bruteforce():
    """Prefill over an FP8 cache: scalar loops that quantise c^KV tile by tile
    through torch's float8_e4m3fn with the power-of-two tile scale, leave k^R
    in full precision, and attend over the dequantised rows (the notes page,
    section 二(三): activations in FP8 with one scale per 1 x 128 tile)."""
    H, dc = 2, 128
    w, h = _rand_setup(13, H=H, dc=dc, L=5)
    ref = _bf_prefill(h, w, H, 1e-6, 10000.0, kv_fp8=True)
    o, rows = om.prefill(h, w, H, 1e-6, 10000.0, scale=1.0 / math.sqrt(4 + 2), kv_fp8=True)
    assert _rel(o, ref) <= 1e-12
    plain = _bf_prefill(h, w, H, 1e-6, 10000.0)
    assert _rel(plain, ref) > 1e-4  # the quantisation is visible at this bar
    # the cached k^R (last d_h^R values of each row) is not quantised
    pos = np.arange(5)
    kr = om.rope(np.asarray(h) @ np.asarray(w["w_kr"]).T, pos, 10000.0)
    assert np.array_equal(rows[:, dc:], kr)


def test_fp8_yarn_prefill_matches_bruteforce():
    """Both options together, as the library allows them together."""
    y, _ = _yarn_page()
    H, dr, dc = 2, 8, 128
    w, h = _rand_setup(14, H=H, dr=dr, dc=dc, L=5)
    ref = _bf_prefill(h, w, H, 1e-6, 10000.0, yarn=y, kv_fp8=True)
    o, _ = om.prefill(h, w, H, 1e-6, 10000.0, scale=1.0 / math.sqrt(4 + dr), yarn=y, kv_fp8=True)
    assert _rel(o, ref) <= 1e-12


# ---------------------------------------------------------------------------
# Output projection W^O and its fold with W^UV
# ---------------------------------------------------------------------------
def test_wo_fold_equals_unfolded():
    """The page's equation: W^O [W_1^UV s_1; ...] = W^O' [s_1; ...]."""
    r = np.random.default_rng(50)
    T, H, dh, dc, d = 3, 4, 5, 7, 6
    o_lat = r.standard_normal((T, H, dc))
    w_uv = r.standard_normal((H * dh, dc))
    w_o = r.standard_normal((d, H * dh))
    o = np.stack([o_lat[:, i] @ w_uv[i * dh:(i + 1) * dh].T for i in range(H)], axis=1)
    a = om.output_projection(o, w_o)
    b = om.folded_output(o_lat, om.fold_output(w_o, w_uv, H))
    assert _rel(b, a) <= 1e-13
    assert om.fold_output(w_o, w_uv, H).shape == (d, H * dc)


def test_wo_identity_concatenates_heads():
    r = np.random.default_rng(51)
    o = r.standard_normal((2, 3, 4))
    assert np.array_equal(om.output_projection(o, np.eye(12)), o.reshape(2, 12))


def test_wo_head_blocks():
    """W_i^O is the column block of head i: zeroing every other block leaves
    only head i's output in u."""
    r = np.random.default_rng(52)
    T, H, dh, d = 2, 3, 4, 5
    o = r.standard_normal((T, H, dh))
    w_o = r.standard_normal((d, H * dh))
    for i in range(H):
        w_i = np.zeros_like(w_o)
        w_i[:, i * dh:(i + 1) * dh] = w_o[:, i * dh:(i + 1) * dh]
        o2 = np.zeros_like(o)
        o2[:, i] = o[:, i]
        assert np.array_equal(om.output_projection(o, w_i), om.output_projection(o2, w_o))
