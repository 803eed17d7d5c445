"""Parity that single keys decide.

In these inputs one key per (sequence, head) outscores every other visible key
by a wide margin, so the softmax puts (almost) all weight on it and the output
is close to W_i^UV c_{j*}.  A kernel that drops that key, reads it from the
wrong page or tile, or lets a key the causal mask should hide into the sum is
then off by O(1), far past the bf16 bar (with random keys one misplaced key
moves the output by well under 1e-2).  The keys sit at the first and last
position of a 32-key tile, of a page and of a split chunk of the device plan,
and at future positions: the step's second new token for the first of two
decode queries (notes page, section 一(一)3, step (10): Softmax over j <= t).

Decode: heads are cut into four groups of 32 (one per wave of the attention
kernel); every head of group g gets q^R = u_g, and the group's key j*_g gets
k^R = lam * u_g, so its score lam |u_g|^2 / sqrt(192) ~ 37 beats the others'
(N(0, 1) scaled, and ~ N(0, 4.6^2) from the other groups' keys).
"""
import numpy as np
import pytest
import torch

import head_latent_attention_06_amd as mla
import mla_inputs as mi
from mla_testutil import BF16_TOL, config, decode_setup, dev, host, rel_l2
from oracle import mla_oracle as om

pytestmark = pytest.mark.gpu

S = mi.V3
LAM = 8.0
GROUPS = 4  # head groups of 32


def _plan_chunk(ws, n_rows):
    """Chunk (keys per split) the device plan chose: the decode workspace holds
    the absorbed queries and the merged latents ([rows, H, 512] bf16 each),
    then the plan, whose second int32 is the chunk."""
    off = 2 * n_rows * S.n_heads * S.d_c * 2
    return int(ws[off + 4:off + 8].view(torch.int32).item())


def _expected_chunk(vis, max_chunk_keys):
    """The plan's rule: about 256 items (1024 for ragged lengths), chunks a
    multiple of 32 keys in [256, max_chunk_keys]."""
    vis = np.asarray(vis, np.int64)
    T, M, n = int(vis.sum()), int(vis.max()), len(vis)
    tgt = 256 if 4 * T >= 3 * n * M else 1024
    c = -(-T // tgt)
    return int(min(max_chunk_keys, max(256, (c + 31) // 32 * 32)))


def _dominant_inputs(config_id, contexts, s_q, positions):
    """Decode inputs with q^R = u_g for the heads of group g and k^R = lam u_g
    at key positions[b][g] of sequence b (None: no dominant key for that group)."""
    inp = mi.decode_inputs(config_id, S, contexts, s_q)
    r = mi.rng(config_id, 90)
    u = [mi.round_to_bf16(r.standard_normal(S.d_rope).astype(np.float32)) for _ in range(GROUPS)]
    for g in range(GROUPS):
        inp.q_pe[:, :, 32 * g:32 * (g + 1), :] = u[g]
    for b, ps in enumerate(positions):
        ps = [p for p in ps if p is not None]
        assert len(set(ps)) == len(ps)
        for g, p in enumerate(positions[b]):
            if p is not None:
                assert 0 <= p < inp.kv_lens[b]
                inp.rows[int(inp.row_offsets[b]) + p, S.d_c:] = mi.round_to_bf16(LAM * u[g])
    return inp


def _check(inp, got, positions, must_dominate=True):
    """Every (sequence, query, head) against the oracle; and the inputs do what
    they claim: a visible dominant key carries the output, a hidden one would
    have moved it by O(1)."""
    s_q = inp.s_q
    worst = 0.0
    w_uk, w_uv = inp.w_uk.astype(np.float64), inp.w_uv.astype(np.float64)
    for b in range(len(inp.kv_lens)):
        rows = inp.seq_rows(b).astype(np.float64)
        kv = int(inp.kv_lens[b])
        q_pos = kv - s_q + np.arange(s_q)
        ref = om.absorbed_attention(inp.q_nope[b], inp.q_pe[b], rows[:, :S.d_c], rows[:, S.d_c:], w_uk, w_uv, q_pos,
                                    S.scale)
        for s in range(s_q):
            for hd in range(S.n_heads):
                e = rel_l2(got[b, s, hd], ref[s, hd])
                worst = max(worst, e)
                assert e <= BF16_TOL, (b, s, hd, e, positions[b])
            for g, p in enumerate(positions[b]):
                if p is None:
                    continue
                hd = 32 * g + 5
                alone = w_uv[hd * S.d_head:(hd + 1) * S.d_head] @ rows[p, :S.d_c]
                if p <= q_pos[s]:
                    if must_dominate:
                        assert rel_l2(ref[s, hd], alone) <= 1e-3, (b, s, g, p)
                else:
                    assert rel_l2(ref[s, hd], alone) > 0.3, (b, s, g, p)
    return worst


def _run(inp, cfg, cache, t):
    B, s_q = inp.q_nope.shape[0], inp.s_q
    max_kv = int(inp.kv_lens.max())
    ws = torch.empty(mla.mla_decode_workspace_size(cfg, B, s_q, max_kv), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, s_q, S.n_heads, S.d_head), dtype=torch.bfloat16, device="cuda")
    mla.mla_decode(cfg, cache, t["kv_lens"], max_kv, t["q_nope"], t["q_pe"], t["w_uk"], t["w_uv"], out, ws=ws)
    torch.cuda.synchronize()
    assert int(cache.err_flags.item()) == 0
    return host(out), ws


def _edge_positions(kv, chunk, page=64, tile=32):
    """First and last keys of tiles, pages and chunks, below kv."""
    ps = set()
    for step in (tile, page, chunk):
        for k in range(step, kv, step):
            ps.update((k - 1, k))
    ps.update((0, kv - 1))
    return sorted(p for p in ps if 0 <= p < kv)


def test_dominant_keys_decode_b64_ctx4096():
    """The benchmarked decode shape (B = 64 x 4097 keys, one query): the dominant
    keys of 64 sequences x 4 head groups cover every chunk edge, page and tile
    edges, and the new token itself."""
    contexts = [4096] * 64
    kv = 4097
    chunk = _expected_chunk([kv] * 64, 1535 * 64)
    edges = _edge_positions(kv, chunk)
    chunk_edges = [p for k in range(chunk, kv, chunk) for p in (k - 1, k)] + [0, kv - 1]
    r = mi.rng(201, 91)
    rest = [p for p in edges if p not in chunk_edges]
    order = chunk_edges + list(r.permutation(rest))
    positions = []
    for b in range(64):
        ps = []
        for g in range(GROUPS):
            p = order[(b * GROUPS + g) % len(order)]
            while p in ps:
                p = int(r.integers(0, kv))
            ps.append(int(p))
        positions.append(ps)
    inp = _dominant_inputs(201, contexts, 1, positions)
    cfg, cache, bt, t = decode_setup(inp, config_id=201)
    got, ws = _run(inp, cfg, cache, t)
    assert _plan_chunk(ws, 64) == chunk, "the test's chunk edges must be the plan's"
    print(f"chunk={chunk}, {len(set(sum(positions, [])))} distinct dominant positions", flush=True)
    worst = _check(inp, got, positions)
    print(f"worst per-head rel_l2={worst:.3e}", flush=True)


def test_dominant_keys_decode_long_context_131073():
    """B = 4 x 131073 keys: dominant keys at the last and first key of split
    chunks (mid-page and page-aligned chunk edges), the short last chunk, the
    first key and the new token."""
    kv = 131073
    chunk = _expected_chunk([kv] * 4, 1535 * 64)
    last = (kv - 1) // chunk * chunk
    positions = [[chunk - 1, chunk, 0, kv - 1],
                 [2 * chunk - 1, 2 * chunk, 17 * chunk - 1, 17 * chunk],
                 [last - 1, last, 64 * 1000, 64 * 1000 - 1],
                 [31 * chunk + 32, 31 * chunk - 33, kv - 2, 100003]]
    inp = _dominant_inputs(202, [kv - 1] * 4, 1, positions)
    cfg, cache, bt, t = decode_setup(inp, config_id=202)
    got, ws = _run(inp, cfg, cache, t)
    assert _plan_chunk(ws, 4) == chunk
    worst = _check(inp, got, positions)
    print(f"chunk={chunk} worst per-head rel_l2={worst:.3e}", flush=True)


def test_dominant_future_key_decode_s_q2():
    """Two queries per sequence (draft verification): group 0's dominant key is
    the step's second new token, which the first query must not see (it would
    take almost all of that query's weight) while the second query does.  The
    other groups' keys sit on tile, page and chunk edges.  Lengths are ragged,
    with the second new token alone in the last chunk of some sequences."""
    contexts = [31, 32, 63, 64, 255, 256, 511, 1023, 1024, 3000, 4094, 9000, 20000, 32767]
    kv = np.asarray(contexts) + 2
    vis = np.stack([kv - 1, kv], 1).reshape(-1)
    chunk = _expected_chunk(vis, 1535 * 64)
    positions = []
    for k in kv:
        ps = [int(k - 1)]
        for p in (chunk, chunk - 1, 64, 32, 31, 0, k - 2, 63):
            if len(ps) < GROUPS and p < k - 1 and p not in ps:
                ps.append(int(p))
        ps += [None] * (GROUPS - len(ps))
        positions.append(ps)
    inp = _dominant_inputs(203, contexts, 2, positions)
    cfg, cache, bt, t = decode_setup(inp, config_id=203)
    got, ws = _run(inp, cfg, cache, t)
    assert _plan_chunk(ws, 2 * len(contexts)) == chunk
    worst = _check(inp, got, positions)
    print(f"chunk={chunk} worst per-head rel_l2={worst:.3e}", flush=True)


def _inverse_rope(x, pos):
    """The raw k^R whose rotation at pos is x (rotation by -pos * theta_p)."""
    return om.rope(x, -np.asarray(pos, np.float64), S.rope_base)


def _fp8_case():
    """Inputs of the FP8 test: raw rows (c^KV before RMSNorm, k^R before RoPE)
    per sequence, the dominant positions, the plan's chunk, and the decode
    inputs over the oracle's own FP8 rows of those raw rows."""
    contexts = [4094, 4094, 40000, 300, 64, 1000]
    s_q = 2
    inp = mi.decode_inputs(204, S, contexts, s_q)
    kv = inp.kv_lens.astype(np.int64)
    vis = np.stack([kv - 1, kv], 1).reshape(-1)
    chunk = _expected_chunk(vis, 511 * 64)
    r = mi.rng(204, 90)
    u = [mi.round_to_bf16(r.standard_normal(S.d_rope).astype(np.float32)) for _ in range(GROUPS)]
    for g in range(GROUPS):
        inp.q_pe[:, :, 32 * g:32 * (g + 1), :] = u[g]
    positions = []
    for k in kv:
        cand = [int(k - 1), chunk - 1, chunk, 2 * chunk - 1, 2 * chunk, 31, 32, 0, 63, 64]
        ps = []
        for p in cand:
            if len(ps) < GROUPS and p < k and p not in ps:
                ps.append(p)
        positions.append(ps + [None] * (GROUPS - len(ps)))
    raws = [inp.seq_rows(b).copy() for b in range(len(contexts))]
    for b, ps in enumerate(positions):
        for g, p in enumerate(ps):
            if p is not None:
                raws[b][p, S.d_c:] = mi.round_to_bf16(_inverse_rope(LAM * u[g].astype(np.float64), p)
                                                      .astype(np.float32))
    g_kv = np.ones(S.d_c, np.float32)
    rows8 = [om.cache_row_fp8(x[:, :S.d_c], x[:, S.d_c:], g_kv, np.arange(len(x)), S.rms_eps, S.rope_base)[3]
             for x in raws]
    inp8 = mi.DecodeInputs(S, inp.kv_lens, s_q, np.concatenate(rows8), inp.row_offsets, inp.q_nope, inp.q_pe,
                           inp.w_uk, inp.w_uv)
    return inp, raws, positions, chunk, g_kv, inp8


def test_dominant_keys_decode_fp8_cache():
    """The same over an FP8 cache written by the library's append: the raw k^R
    of a dominant key is the inverse rotation of lam * u_g, so the appended
    (rotated, bf16) k^R is lam * u_g up to rounding; the oracle reads its own
    FP8 rows of the same raw inputs.  Splits of at most 511 pages, chunk edges
    at the FP8 plan's chunk, and a future key for s_q = 2."""
    inp, raws, positions, chunk, g_kv, inp8 = _fp8_case()
    cfg = config(S)
    cfg.kv_fp8 = True
    bt, npages = mi.block_table(204, inp.kv_lens, S.page_size, shuffle=True)
    pool = torch.full((npages, S.page_size, cfg.row_bytes), 0xFF, dtype=torch.uint8, device="cuda")
    cache = mla.PagedCache(pool, torch.from_numpy(bt).to("cuda"), torch.zeros(1, dtype=torch.int32, device="cuda"))
    seq = np.concatenate([np.full(len(x), b, np.int32) for b, x in enumerate(raws)])
    pos = np.concatenate([np.arange(len(x), dtype=np.int32) for x in raws])
    allr = np.concatenate(raws)
    mla.mla_cache_append(cfg, cache, dev(allr[:, :S.d_c]), dev(allr[:, S.d_c:]), dev(g_kv),
                         torch.from_numpy(seq).to("cuda"), torch.from_numpy(pos).to("cuda"))
    t = dict(q_nope=dev(inp.q_nope), q_pe=dev(inp.q_pe), w_uk=dev(inp.w_uk), w_uv=dev(inp.w_uv),
             kv_lens=torch.from_numpy(inp.kv_lens).to("cuda"))
    got, ws = _run(inp, cfg, cache, t)
    assert _plan_chunk(ws, inp.s_q * len(raws)) == chunk
    worst = _check(inp8, got, positions)
    print(f"chunk={chunk} worst per-head rel_l2={worst:.3e}", flush=True)


# ---------------------------------------------------------------------------
# Prefill: the keys come from h, so a dominant key is made through h.  For a
# target (query token t, key token j, head i) with j != t: q^R_{t,i} =
# RoPE(a, t) with a = W_i^QR c^Q_t, and k^R_j = RoPE(W^KR h_j, j), so their
# product is a . R_{j-t} (W^KR h_j).  Setting W^KR h_j = lam R_{t-j} a / |a|
# (h_j moved by the least-norm change) makes key j score lam |a| / sqrt(192)
# for that head: ~ 25 with lam = 40, |a| ~ 8.
# ---------------------------------------------------------------------------
P_LAM = 40.0


def _prefill_targets_inputs(config_id, L, targets):
    w = mi.weights(config_id, S)
    h = mi.hidden(config_id, S, 1, L)[0].astype(np.float64)
    keys = [j for _, j, _ in targets]
    queries = [t for t, _, _ in targets]
    assert len(set(keys)) == len(keys) and not set(keys) & set(queries)
    pos = np.arange(L)
    q_c, q_r = om.query_path(h[queries], w["w_dq"], w["g_q"], w["w_uq"], w["w_qr"], np.zeros(len(queries)),
                             S.n_heads, S.rms_eps, S.rope_base)  # position 0: a itself, unrotated
    wkr = w["w_kr"].astype(np.float64)
    pinv = np.linalg.pinv(wkr)
    for n, (t, j, hd) in enumerate(targets):
        a = q_r[n, hd]
        want = om.rope(P_LAM * a / np.linalg.norm(a), t - j, S.rope_base)
        h[j] = h[j] + pinv @ (want - wkr @ h[j])
    return w, mi.round_to_bf16(h.astype(np.float32))[None], pos


FORMS = [pytest.param(mla.PREFILL_ABSORBED, id="absorbed"), pytest.param(mla.PREFILL_EXPLICIT, id="explicit")]


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("L", [1024, 8192])
def test_dominant_keys_prefill(form, L):
    """Causal prefill, both attention forms: dominant past keys on tile,
    page and 256-query-group edges, and dominant FUTURE keys (key t+1 for
    query t, on and off the edges of the 64-key tiles of the explicit kernel
    and the 32-key tiles of the absorbed one), which the causal mask must give
    zero weight."""
    # (query token, key token, head); no key token is a query token of another target
    past = [(100, 63, 3), (200, 64, 40), (300, 255, 70), (400, 256, 127), (520, 31, 0), (700, 32, 96)]
    future = [(126, 127, 9), (191, 192, 33), (510, 511, 64), (767, 768, 100), (600, 601, 1), (95, 96, 120)]
    if L == 8192:
        past += [(8100, 4095, 17), (5000, 4096, 90), (8000, 3190, 66)]
        future += [(4093, 4094, 30), (8190, 8191, 77), (6143, 6144, 50)]
    targets = past + future
    w, h, pos = _prefill_targets_inputs(205 + L, L, targets)
    cfg = config(S)
    cfg.prefill_form = form
    bt, npages = mi.block_table(205, [L], S.page_size, shuffle=True)
    pool = torch.full((npages, S.page_size, cfg.row), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    cache = mla.PagedCache(pool, torch.from_numpy(bt).to("cuda"), torch.zeros(1, dtype=torch.int32, device="cuda"))
    out = torch.empty((1, L, S.n_heads, S.d_head), dtype=torch.bfloat16, device="cuda")
    mla.mla_prefill(cfg, cache, {k: dev(v) for k, v in w.items()}, dev(h), out)
    torch.cuda.synchronize()
    assert int(cache.err_flags.item()) == 0
    got = host(out)[0]
    toks = sorted({t for t, _, _ in targets})
    ref, rows = om.prefill(h[0], w, S.n_heads, S.rms_eps, S.rope_base, S.scale, tokens=np.array(toks))
    fails = []
    for t, j, hd in targets:
        n = toks.index(t)
        alone = w["w_uv"][hd * S.d_head:(hd + 1) * S.d_head].astype(np.float64) @ rows[j, :S.d_c]
        e_head = rel_l2(got[t, hd], ref[n, hd])
        e_tok = rel_l2(got[t], ref[n])  # all heads of the token
        if j <= t:
            # the key carries the output: (almost) W_i^UV c_j, one vector's rounding
            assert rel_l2(ref[n, hd], alone) <= 2e-2, (t, j, hd)
            ok = e_head <= BF16_TOL and e_tok <= BF16_TOL
        else:
            # hidden: the oracle is far from W_i^UV c_j, and so must the GPU be
            # (a leak would pull that head to it); the other keys of such a
            # row include the other targets' keys, whose large k^R make its
            # softmax peaky, so the bar is on all heads of the token
            assert rel_l2(ref[n, hd], alone) > 0.3, (t, j, hd)
            ok = rel_l2(got[t, hd], alone) > 0.3 and e_tok <= BF16_TOL
        print(f"target t={t} j={j} head={hd}: head rel_l2={e_head:.3e}, token rel_l2={e_tok:.3e}", flush=True)
        if not ok:
            fails.append((t, j, hd, e_head, e_tok))
    assert not fails, fails
    # every head of the target tokens together
    err = rel_l2(got[toks], ref)
    print(f"L={L} all heads of {len(toks)} tokens {err:.3e}", flush=True)
    assert err <= BF16_TOL
