"""Explicit Multi-head Latent Attention in float64 on the CPU: the oracle.

TEST INFRASTRUCTURE, NOT PART OF THE LIBRARY.  Only the tests, the smoke check
and the CPU-baseline leg of the benchmark may import this module.  It shares no
code with the HIP path and imports nothing from the library package.

What it follows.  The notes page "【论文解读】DeepSeek-V3" (wkq9411.github.io),
section 一(一) "多头潜在注意力MLA":
  * 1 "回顾多头注意力MHA": per-head softmax attention, Softmax_j over j = 1..t,
    heads are consecutive d_h-row blocks of the projections;
  * 2 "低秩KV联合压缩": c^KV = W^DKV h, k^C = W^UK c^KV, v^C = W^UV c^KV,
    c^Q = W^DQ h, q^C = W^UQ c^Q;
  * 【思考】 on absorption: per-head blocks W_i^UK, W_i^UV in R^{d_h x d_c};
    q^C_i . k^C_{j,i} = (W_i^UK^T q^C_i) . c_j and o_i = W_i^UV sum_j a_j c_j;
  * 3 "解耦RoPE": q^R = RoPE(W^QR c^Q) per head, k^R = RoPE(W^KR h) shared by
    all heads, q_i = [q^C_i; q^R_i], k_i = [k^C_i; k^R], scale 1/sqrt(d_h+d_h^R);
  * the ten-step "完整计算过程" list, steps (1)-(10);
  * section 二(二)1: "an additional RMSNorm after the compressed latent vectors".

The result has a plain definition (steps (1)-(10)), so the oracle is that
definition written out: it materialises every head's k and v and applies the
max-subtracted softmax, all in float64.  The absorbed form (used only by the
pins, to show the two forms agree) is a separate function.

Readings where the pages leave a step open:
  * RMSNorm: y = x / sqrt(mean(x^2) + eps) * g, applied to both c^KV and c^Q;
    k^R is not normalised (it is taken from h, not from a latent).
  * RoPE: rotation of adjacent pairs (x_2p, x_2p+1) by the 2x2 block
    [[cos, -sin], [sin, cos]] of section 一(一)3, angle pos * theta_p with
    theta_p = base^(-2p/d_rope) (the RoPE frequency formula quoted on the
    hnwysp.cn digest, section 4.3), base 10000, positions counted from 0.
  * Output stops at o = [o_1; ...; o_{n_h}]; W^O is applied separately
    (output_projection), as is its fold with W^UV (【思考】 on absorption:
    u_t = W^O [o_{t,1}; ...; o_{t,n_h}], W_i^O the d_h-column block of head i,
    W_i^O' = W_i^O W_i^UV, W^O' = [W_1^O' ... W_{n_h}^O']).
  * YaRN (optional, the long-context extension of the notes page, section
    三(二)3 "长上下文扩展": s = 40, alpha = 1, beta = 32, factor 0.1 ln s + 1,
    with the method's meaning taken from the YaRN paper the page points to):
    every RoPE frequency theta_p becomes (1 - g) theta_p / s + g theta_p,
    where g ramps from 0 to 1 as the pair's rotations over the original
    context, r_p = orig_ctx theta_p / (2 pi), go from alpha to beta; and every
    attention logit is multiplied by (0.1 ln s + 1)^2 (YaRN applies the square
    root of that temperature to both q and k).  The same frequencies rotate
    q^R and k^R, so scores still depend only on relative positions.
  * Decode: the step's s_q new tokens are already cached; query s of a
    sequence with kv_len cached rows sits at position kv_len - s_q + s and
    attends to rows j <= that position.
  * FP8 latent cache (optional; the notes page, section 二(三) "FP8训练",
    fixes only the granularity: activations are quantised per 1 x 128 tile,
    each tile with its own scale, and products accumulate in FP32).  The format is OCP E4M3 ("e4m3fn": 4 exponent bits,
    bias 7, 3 mantissa bits, largest finite 448, no infinities).  Each
    128-value tile of c^KV gets a power-of-two scale 2^e, e the smallest
    integer with max|x| <= 448 * 2^e, and codes round x / 2^e to the nearest
    E4M3 value, ties to even.  The decision is taken on the value rounded to
    float32.  k^R is not quantised.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=F64)


# ---------------------------------------------------------------------------
# Building blocks
# ---------------------------------------------------------------------------
def rms_norm(x, g, eps: float) -> np.ndarray:
    """RMSNorm over the last axis (section 二(二)1: RMSNorm after the latents)."""
    x = _f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * _f64(g)


def rope_frequencies(d_rope: int, base: float) -> np.ndarray:
    """theta_p = base^(-2p/d_rope), p = 0 .. d_rope/2 - 1."""
    p = np.arange(d_rope // 2, dtype=F64)
    return np.power(F64(base), -2.0 * p / d_rope)


def yarn_frequencies(d_rope: int, base: float, yarn) -> np.ndarray:
    """YaRN frequencies: theta'_p = (1 - g_p) theta_p / s + g_p theta_p.

    ``yarn`` = dict(s=..., alpha=..., beta=..., orig_ctx=...).  r_p =
    orig_ctx * theta_p / (2 pi) counts the pair's rotations over the original
    context; g_p = 0 for r_p < alpha (pure interpolation by s), 1 for
    r_p > beta (unchanged), linear in between.
    """
    theta = rope_frequencies(d_rope, base)
    r = F64(yarn["orig_ctx"]) * theta / (2.0 * np.pi)
    g = np.clip((r - F64(yarn["alpha"])) / (F64(yarn["beta"]) - F64(yarn["alpha"])), 0.0, 1.0)
    return (1.0 - g) * theta / F64(yarn["s"]) + g * theta


def yarn_logit_factor(s: float) -> float:
    """Multiplier of every attention logit under YaRN: (0.1 ln s + 1)^2."""
    return float((0.1 * np.log(F64(s)) + 1.0) ** 2)


def rope(x, pos, base: float, yarn=None) -> np.ndarray:
    """Rotate each adjacent pair of the last axis by pos * theta_p.

    Section 一(一)3 gives R_m as a block-diagonal matrix of 2x2 rotations
    [[cos m.theta, -sin m.theta], [sin m.theta, cos m.theta]].  ``x`` is
    [..., d_rope]; ``pos`` broadcasts against x's leading axes.  With ``yarn``
    the frequencies are the YaRN ones.
    """
    x = _f64(x)
    d = x.shape[-1]
    theta = rope_frequencies(d, base) if yarn is None else yarn_frequencies(d, base, yarn)
    ang = _f64(pos)[..., None] * theta            # [..., d/2]
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = c * x0 - s * x1
    out[..., 1::2] = s * x0 + c * x1
    return out


def split_heads(x, n_heads: int) -> np.ndarray:
    """[..., n_heads * w] -> [..., n_heads, w]: head i owns block i (section 一(一)1)."""
    x = _f64(x)
    return x.reshape(*x.shape[:-1], n_heads, x.shape[-1] // n_heads)


# ---------------------------------------------------------------------------
# Projections (steps (1)-(3), (5), (7))
# ---------------------------------------------------------------------------
def query_path(h, w_dq, g_q, w_uq, w_qr, pos, n_heads: int, eps: float, base: float, yarn=None):
    """Steps (1)-(3): c^Q = RMSNorm(W^DQ h); q^C = W^UQ c^Q; q^R = RoPE(W^QR c^Q).

    h: [T, d]; pos: [T].  Returns q^C [T, H, d_h] and q^R [T, H, d_rope].
    """
    h = _f64(h)
    c_q = rms_norm(h @ _f64(w_dq).T, g_q, eps)
    q_c = split_heads(c_q @ _f64(w_uq).T, n_heads)
    q_r_raw = split_heads(c_q @ _f64(w_qr).T, n_heads)
    q_r = rope(q_r_raw, _f64(pos)[:, None], base, yarn)
    return q_c, q_r


def latent_rows(h, w_dkv, g_kv, w_kr, pos, eps: float, base: float, yarn=None):
    """Steps (5) and (7): c^KV = RMSNorm(W^DKV h) and k^R = RoPE(W^KR h).

    These two vectors are all that is cached per token (section 一(一)3, end of
    the decoupled-RoPE equations).  Returns (c [T, d_c], k_r [T, d_rope]).
    """
    h = _f64(h)
    c = rms_norm(h @ _f64(w_dkv).T, g_kv, eps)
    k_r = rope(h @ _f64(w_kr).T, pos, base, yarn)
    return c, k_r


def cache_row(c_raw, k_raw, g_kv, pos, eps: float, base: float, yarn=None) -> np.ndarray:
    """One cached row from the raw projections: [RMSNorm(c_raw) ; RoPE(k_raw, pos)]."""
    return np.concatenate([rms_norm(c_raw, g_kv, eps), rope(k_raw, pos, base, yarn)], axis=-1)


# ---------------------------------------------------------------------------
# Attention (steps (6), (8), (9), (10)), explicit form
# ---------------------------------------------------------------------------
def explicit_attention(q_c, q_r, c, k_r, w_uk, w_uv, q_pos, scale: float,
                       heads=None, return_weights: bool = False):
    """Explicit MLA attention of some queries over one sequence's cached rows.

    q_c [T, H, d_h], q_r [T, H, d_rope] (already rotated), c [N, d_c],
    k_r [N, d_rope] (already rotated), w_uk / w_uv [H*d_h, d_c], q_pos [T]:
    query t attends to rows j <= q_pos[t].  For every head i it materialises
    k^C_{j,i} = W_i^UK c_j, k_{j,i} = [k^C_{j,i}; k^R_j], v_{j,i} = W_i^UV c_j
    and computes o_{t,i} = sum_j Softmax_j(q_{t,i} . k_{j,i} * scale) v_{j,i}.
    Returns o [T, len(heads), d_h] (and the weights [T, len(heads), N]).
    """
    q_c, q_r, c, k_r = _f64(q_c), _f64(q_r), _f64(c), _f64(k_r)
    T, H, dh = q_c.shape
    N = c.shape[0]
    heads = list(range(H)) if heads is None else list(heads)
    w_uk, w_uv = _f64(w_uk), _f64(w_uv)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    visible = np.arange(N)[None, :] <= q_pos[:, None]          # [T, N]
    out = np.zeros((T, len(heads), dh), F64)
    wts = np.zeros((T, len(heads), N), F64) if return_weights else None
    for n, i in enumerate(heads):
        wk = w_uk[i * dh:(i + 1) * dh]                         # W_i^UK [d_h, d_c]
        wv = w_uv[i * dh:(i + 1) * dh]                         # W_i^UV [d_h, d_c]
        k_c = c @ wk.T                                          # [N, d_h]
        v = c @ wv.T                                            # [N, d_h]
        k = np.concatenate([k_c, k_r], axis=1)                  # [N, d_h + d_rope]
        q = np.concatenate([q_c[:, i], q_r[:, i]], axis=1)      # [T, d_h + d_rope]
        s = (q @ k.T) * scale
        s = np.where(visible, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        e = np.exp(s)
        a = e / e.sum(axis=1, keepdims=True)
        out[:, n] = a @ v
        if return_weights:
            wts[:, n] = a
    return (out, wts) if return_weights else out


def absorbed_attention(q_c, q_r, c, k_r, w_uk, w_uv, q_pos, scale: float, heads=None):
    """The same attention with W^UK folded into the query and W^UV after the sum.

    q_lat_{t,i} = W_i^UK^T q^C_{t,i}; score = q_lat . c_j + q^R_{t,i} . k^R_j;
    o_{t,i} = W_i^UV sum_j a_j c_j  (【思考】 on absorption, and the score split
    into a latent term and a RoPE term in section 一(一)3).
    """
    q_c, q_r, c, k_r = _f64(q_c), _f64(q_r), _f64(c), _f64(k_r)
    T, H, dh = q_c.shape
    N, dc = c.shape
    heads = list(range(H)) if heads is None else list(heads)
    nh = len(heads)
    sel = slice(None) if heads == list(range(H)) else heads
    w_uk = _f64(w_uk).reshape(H, dh, dc)[sel]                # W_i^UK, [n, d_h, d_c]
    w_uv = _f64(w_uv).reshape(H, dh, dc)[sel]                # W_i^UV
    visible = np.arange(N)[None, None, :] <= np.asarray(q_pos, np.int64)[:, None, None]
    # q_lat_{t,i} = W_i^UK^T q^C_{t,i}, all selected heads at once ([n, T, d_c])
    q_lat = np.matmul(q_c[:, sel].transpose(1, 0, 2), w_uk)
    s = (q_lat.transpose(1, 0, 2).reshape(T * nh, dc) @ c.T + q_r[:, sel].reshape(T * nh, -1) @ k_r.T) * scale
    s = np.where(visible, s.reshape(T, nh, N), -np.inf)
    s = s - s.max(axis=2, keepdims=True)
    e = np.exp(s)
    a = e / e.sum(axis=2, keepdims=True)
    o_lat = (a.reshape(T * nh, N) @ c).reshape(T, nh, dc)     # sum_j a_j c_j
    # o_{t,i} = W_i^UV o_lat_{t,i}
    return np.matmul(o_lat.transpose(1, 0, 2), w_uv.transpose(0, 2, 1)).transpose(1, 0, 2)


# ---------------------------------------------------------------------------
# Output projection (【思考】 on absorption: u_t = W^O [o_{t,1}; ...; o_{t,n_h}])
# ---------------------------------------------------------------------------
def output_projection(o, w_o) -> np.ndarray:
    """u = W^O [o_1; ...; o_{n_h}] for every token: o [T, H, d_h], W^O [d, H*d_h] -> u [T, d]."""
    o = _f64(o)
    return o.reshape(o.shape[0], -1) @ _f64(w_o).T


def fold_output(w_o, w_uv, n_heads: int) -> np.ndarray:
    """W^O' = [W_1^O W_1^UV, ..., W_{n_h}^O W_{n_h}^UV]  ([d, H*d_c]).

    W_i^O is the d_h-column block i of W^O; W_i^UV the d_h-row block i of W^UV.
    """
    w_o, w_uv = _f64(w_o), _f64(w_uv)
    dh = w_o.shape[1] // n_heads
    return np.concatenate([w_o[:, i * dh:(i + 1) * dh] @ w_uv[i * dh:(i + 1) * dh] for i in range(n_heads)], axis=1)


def folded_output(o_lat, w_o_fold) -> np.ndarray:
    """u = W^O' [o^lat_1; ...; o^lat_{n_h}] with o^lat_i = sum_j a_j c_j: o_lat [T, H, d_c] -> u [T, d]."""
    o_lat = _f64(o_lat)
    return o_lat.reshape(o_lat.shape[0], -1) @ _f64(w_o_fold).T


# ---------------------------------------------------------------------------
# Split-context partials and their merge
# ---------------------------------------------------------------------------
def latent_partial(q_lat, q_r, c, k_r, scale: float, lo: int, hi: int):
    """Softmax partial of one query head over rows [lo, hi) of its visible range.

    Returns (m, l, acc): m = max score, l = sum_j e^{s_j - m},
    acc = sum_j e^{s_j - m} c_j.  An empty range gives (-inf, 0, 0).
    """
    q_lat, q_r, c, k_r = _f64(q_lat), _f64(q_r), _f64(c), _f64(k_r)
    if hi <= lo:
        return -np.inf, 0.0, np.zeros(c.shape[1], F64)
    s = (c[lo:hi] @ q_lat + k_r[lo:hi] @ q_r) * scale
    m = s.max()
    e = np.exp(s - m)
    return m, e.sum(), e @ c[lo:hi]


def merge_partials(ms, ls, accs) -> np.ndarray:
    """Combine split partials: m* = max m_k; result = sum e^{m_k-m*} acc_k / sum e^{m_k-m*} l_k.

    This is the identity softmax(x) over a union of disjoint ranges satisfies;
    the pages are silent on splitting, so the merge is written from it.
    """
    ms = _f64(ms)
    ls = _f64(ls)
    accs = _f64(accs)
    m_star = ms.max()
    w = np.exp(ms - m_star)
    return (w[:, None] * accs).sum(axis=0) / (w * ls).sum()


# ---------------------------------------------------------------------------
# Whole operations, as the library exposes them
# ---------------------------------------------------------------------------
def decode(rows_per_seq, kv_lens, s_q: int, q_nope, q_pe, w_uk, w_uv, d_c: int, scale: float,
           seqs=None, heads=None) -> np.ndarray:
    """One decode step over cached rows ([c ; k^R] per token, position order).

    rows_per_seq[b] is [kv_len_b, d_c + d_rope]; q_nope [B, s_q, H, d_h];
    q_pe [B, s_q, H, d_rope] (rotated).  Returns o [len(seqs), s_q, len(heads), d_h].
    """
    seqs = range(len(kv_lens)) if seqs is None else seqs
    outs = []
    for b in seqs:
        rows = _f64(rows_per_seq[b])
        kv = int(kv_lens[b])
        q_pos = kv - s_q + np.arange(s_q)
        outs.append(explicit_attention(q_nope[b], q_pe[b], rows[:kv, :d_c], rows[:kv, d_c:],
                                       w_uk, w_uv, q_pos, scale, heads=heads))
    return np.stack(outs)


def prefill(h, w, n_heads: int, eps: float, base: float, scale: float, start_pos: int = 0,
            past_rows=None, tokens=None, heads=None, yarn=None, kv_fp8: bool = False):
    """Steps (1)-(10) for one sequence: h [L, d] holds tokens start_pos .. start_pos+L-1.

    ``past_rows`` [start_pos, d_c + d_rope] are the rows already cached for
    earlier positions.  Returns (o [len(tokens), len(heads), d_h], new_rows
    [L, d_c + d_rope]).  ``tokens`` selects which new tokens' outputs to compute.
    With ``yarn`` the RoPE frequencies are YaRN's and the logits are scaled by
    yarn_logit_factor(s) on top of ``scale``.  With ``kv_fp8`` the cache holds
    c^KV in the FP8 format (quantize_latent_fp8) and attention reads those
    values; new_rows are then the dequantised rows.
    """
    h = _f64(h)
    L = h.shape[0]
    pos = start_pos + np.arange(L)
    d_c = np.asarray(w["w_dkv"]).shape[0]
    c, k_r = latent_rows(h, w["w_dkv"], w["g_kv"], w["w_kr"], pos, eps, base, yarn)
    if kv_fp8:
        c = quantize_latent_fp8(c)[2]
    new_rows = np.concatenate([c, k_r], axis=1)
    rows = new_rows if past_rows is None or start_pos == 0 else np.concatenate([_f64(past_rows), new_rows])
    tokens = np.arange(L) if tokens is None else np.asarray(tokens)
    q_c, q_r = query_path(h[tokens], w["w_dq"], w["g_q"], w["w_uq"], w["w_qr"], pos[tokens],
                          n_heads, eps, base, yarn)
    eff_scale = scale if yarn is None else scale * yarn_logit_factor(yarn["s"])
    o = explicit_attention(q_c, q_r, rows[:, :d_c], rows[:, d_c:], w["w_uk"], w["w_uv"],
                           pos[tokens], eff_scale, heads=heads)
    return o, new_rows


# ---------------------------------------------------------------------------
# FP8 latent cache: E4M3 codes with one power-of-two scale per 1 x 128 tile
# ---------------------------------------------------------------------------
E4M3_MAX = 448.0
FP8_TILE = 128


def e4m3_value(codes) -> np.ndarray:
    """Value of E4M3 codes (uint8): sign bit 7, exponent bits 6..3 (bias 7),
    mantissa bits 2..0; exponent field 0 is subnormal (m/8 * 2^-6); exponent
    15 with mantissa 7 is NaN; there is no infinity."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(F64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    return np.where((e == 15) & (m == 7), np.nan, sign * mag)


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code to each x (|x| <= 448), ties to the even code.

    Within a binade [2^k, 2^(k+1)), k >= -6, neighbouring values are 2^(k-3)
    apart; below 2^-6 (subnormals) they are 2^-9 apart.  The magnitude is
    rounded to a multiple of that spacing (numpy's rint rounds halves to even,
    and an even multiple is an even mantissa), and a value that rounds up to
    the next power of two is that power's code.  The sign bit is kept, so
    small negative values give -0 (0x80)."""
    x = _f64(x)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("E4M3 encoding takes finite |x| <= 448")
    a = np.abs(x)
    k = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    k = np.where(a >= 2.0 ** -6, k, -6.0)
    # log2 near a power of two may land one off: fix k so 2^k <= a < 2^(k+1)
    k = np.where((a >= 2.0 ** -6) & (2.0 ** k > a), k - 1, k)
    k = np.where((a >= 2.0 ** -6) & (2.0 ** (k + 1) <= a), k + 1, k)
    step = 2.0 ** (k - 3)
    q = np.rint(a / step) * step  # the rounded magnitude
    code = np.zeros(a.shape, dtype=np.int64)
    sub = q < 2.0 ** -6
    code = np.where(sub, np.rint(q / 2.0 ** -9), code)
    kq = np.floor(np.log2(np.where(sub, 1.0, q)))
    kq = np.where(~sub & (2.0 ** kq > q), kq - 1, kq)
    mant = np.rint((q / 2.0 ** kq - 1.0) * 8.0)
    code = np.where(sub, code, ((kq + 7) * 8 + mant)).astype(np.int64)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def fp8_tile_exponent(amax) -> np.ndarray:
    """Smallest integer e with amax <= 448 * 2^e (e = 0 for an all-zero tile)."""
    amax = _f64(amax)
    e = np.ceil(np.log2(np.where(amax > 0, amax, E4M3_MAX) / E4M3_MAX))
    e = np.where(amax > E4M3_MAX * 2.0 ** e, e + 1, e)
    e = np.where((amax > 0) & (amax <= E4M3_MAX * 2.0 ** (e - 1)), e - 1, e)
    return e.astype(np.int64)


def quantize_latent_fp8(c):
    """c [..., d_c] -> (codes uint8 [..., d_c], tile exponents int [..., d_c/128],
    dequantised float64 [..., d_c]).  Codes are decided on float32(c)."""
    x = np.asarray(c, dtype=np.float32).astype(F64)
    tiles = x.reshape(x.shape[:-1] + (x.shape[-1] // FP8_TILE, FP8_TILE))
    e = fp8_tile_exponent(np.max(np.abs(tiles), axis=-1))
    scale = 2.0 ** e[..., None]
    codes = e4m3_encode(tiles / scale)
    deq = e4m3_value(codes) * scale
    return codes.reshape(x.shape), e, deq.reshape(x.shape)


def cache_row_fp8(c_raw, k_raw, g_kv, pos, eps: float, base: float, yarn=None):
    """A cached row in the FP8 format: (codes, tile exponents, k^R, and the row
    the attention reads, [dequantised RMSNorm(c_raw) ; RoPE(k_raw, pos)])."""
    codes, e, c_deq = quantize_latent_fp8(rms_norm(c_raw, g_kv, eps))
    k_r = rope(k_raw, pos, base, yarn)
    return codes, e, k_r, np.concatenate([c_deq, k_r], axis=-1)


# ---------------------------------------------------------------------------
# Paged layout
# ---------------------------------------------------------------------------
def paged_slot(block_table, b: int, pos: int, page_size: int):
    """Where token ``pos`` of sequence ``b`` lives: (page id, slot in page)."""
    return int(block_table[b][pos // page_size]), pos % page_size


def paged_gather(pool, block_table, b: int, n: int, page_size: int) -> np.ndarray:
    """Rows 0..n-1 of sequence b, read through the block table."""
    return np.stack([pool[paged_slot(block_table, b, p, page_size)] for p in range(n)]) if n else \
        np.zeros((0,) + pool.shape[2:], pool.dtype)
