"""Seeded synthetic inputs for the MLA library and its oracle.

This module is shared by both sides of every parity check, so it holds none of
the attention arithmetic: only random draws (``numpy.random.default_rng`` seeded
with ``[config_id, tensor_id]``), the rounding of those draws to the storage
dtype, and the *structure* of each workload (sequence lengths, page counts and
the shuffled block table).  Whatever the method computes from these inputs is
written separately in ``oracle/`` and in the HIP kernels.

Shapes follow the DeepSeek-V3 model hyper-parameters listed on the notes page
"【论文解读】DeepSeek-V3" (section 二(二)1 "模型超参数"): n_h = 128 heads,
d_h = 128, d_c = 512, d_c' = 1536, d_h^R = 64, hidden size d = 7168.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Shape:
    """Dimensions of one MLA layer (names follow the notes page's symbols)."""

    n_heads: int
    d_head: int
    d_rope: int
    d_c: int
    d_cq: int
    d_model: int
    page_size: int = 64
    rope_base: float = 10000.0
    rms_eps: float = 1e-6

    @property
    def row(self) -> int:
        """Elements cached per token: the latent c^KV followed by k^R."""
        return self.d_c + self.d_rope

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d_head + self.d_rope))


V3 = Shape(n_heads=128, d_head=128, d_rope=64, d_c=512, d_cq=1536, d_model=7168)
TINY = Shape(n_heads=4, d_head=16, d_rope=8, d_c=32, d_cq=48, d_model=64)


# --------------------------------------------------------------------------
# Tensor ids.  Every tensor of a workload has its own stream so that changing
# the size of one never changes the values of another.
# --------------------------------------------------------------------------
T_H, T_WDQ, T_GQ, T_WUQ, T_WQR, T_WDKV, T_GKV, T_WKR, T_WUK, T_WUV = range(1, 11)
T_CACHE, T_QNOPE, T_QPE, T_LENS, T_PERM, T_CKV_RAW, T_KR_RAW, T_POS = range(20, 28)


def rng(config_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([int(config_id), int(tensor_id)])


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), kept as float32.

    Inputs handed to a bf16 kernel must be exactly representable so that the
    oracle and the kernel start from identical values.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def normal(config_id: int, tensor_id: int, shape, std: float = 1.0, bf16: bool = True) -> np.ndarray:
    a = rng(config_id, tensor_id).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return round_to_bf16(a) if bf16 else a


def weights(config_id: int, s: Shape, bf16: bool = True, gain_spread: float = 0.0) -> dict:
    """All projection weights of one layer, stored [out, in] row-major.

    Each weight is drawn from N(0, 1/fan_in) with fan_in its input width.  The
    RMSNorm gains are 1, or U(1 - spread, 1 + spread) when ``gain_spread`` > 0.
    """
    H, dh, dr, dc, dcq, d = s.n_heads, s.d_head, s.d_rope, s.d_c, s.d_cq, s.d_model

    def w(tid, out, inp):
        return normal(config_id, tid, (out, inp), std=1.0 / np.sqrt(inp), bf16=bf16)

    def gain(tid, n):
        if gain_spread <= 0.0:
            return np.ones(n, np.float32)
        g = rng(config_id, tid).uniform(1.0 - gain_spread, 1.0 + gain_spread, size=n).astype(np.float32)
        return round_to_bf16(g) if bf16 else g

    return {
        "w_dq": w(T_WDQ, dcq, d),
        "g_q": gain(T_GQ, dcq),
        "w_uq": w(T_WUQ, H * dh, dcq),
        "w_qr": w(T_WQR, H * dr, dcq),
        "w_dkv": w(T_WDKV, dc, d),
        "g_kv": gain(T_GKV, dc),
        "w_kr": w(T_WKR, dr, d),
        "w_uk": w(T_WUK, H * dh, dc),
        "w_uv": w(T_WUV, H * dh, dc),
    }


def hidden(config_id: int, s: Shape, B: int, L: int, bf16: bool = True) -> np.ndarray:
    """Layer input h ~ N(0, 1), shape [B, L, d]."""
    return normal(config_id, T_H, (B, L, s.d_model), bf16=bf16)


@dataclass
class DecodeInputs:
    """One decode step: cached rows per sequence plus the step's queries.

    ``rows`` is [sum(kv_lens), d_c + d_rope]; sequence b owns rows
    ``row_offsets[b] : row_offsets[b] + kv_lens[b]`` in position order.
    """

    shape: Shape
    kv_lens: np.ndarray
    s_q: int
    rows: np.ndarray
    row_offsets: np.ndarray
    q_nope: np.ndarray
    q_pe: np.ndarray
    w_uk: np.ndarray
    w_uv: np.ndarray
    extra: dict = field(default_factory=dict)

    def seq_rows(self, b: int) -> np.ndarray:
        o = int(self.row_offsets[b])
        return self.rows[o:o + int(self.kv_lens[b])]


def decode_inputs(config_id: int, s: Shape, context_lens, s_q: int, bf16: bool = True) -> DecodeInputs:
    """Synthetic decode step.

    ``context_lens`` counts the tokens cached before this step; the step's
    ``s_q`` new tokens are already in the cache, so kv_len = context + s_q.
    Cached c^KV and k^R, q^C and the (already rotated) q^R are N(0, 1);
    W^UK and W^UV are N(0, 1/d_c).
    """
    ctx = np.asarray(context_lens, dtype=np.int64)
    B = ctx.shape[0]
    kv = ctx + s_q
    offs = np.zeros(B, np.int64)
    offs[1:] = np.cumsum(kv)[:-1]
    H, dh, dr, dc = s.n_heads, s.d_head, s.d_rope, s.d_c
    rows = normal(config_id, T_CACHE, (int(kv.sum()), dc + dr), bf16=bf16)
    q_nope = normal(config_id, T_QNOPE, (B, s_q, H, dh), bf16=bf16)
    q_pe = normal(config_id, T_QPE, (B, s_q, H, dr), bf16=bf16)
    w_uk = normal(config_id, T_WUK, (H * dh, dc), std=1.0 / np.sqrt(dc), bf16=bf16)
    w_uv = normal(config_id, T_WUV, (H * dh, dc), std=1.0 / np.sqrt(dc), bf16=bf16)
    return DecodeInputs(s, kv.astype(np.int32), s_q, rows, offs, q_nope, q_pe, w_uk, w_uv)


def uniform_lengths(config_id: int, B: int, lo: int, hi: int) -> np.ndarray:
    """Context lengths drawn uniformly from the integers lo..hi inclusive."""
    return rng(config_id, T_LENS).integers(lo, hi + 1, size=B).astype(np.int64)


def block_table(config_id: int, kv_lens, page_size: int, shuffle: bool = True, spare_pages: int = 0):
    """Page assignment for a paged cache.

    Sequence b needs ceil(kv_len_b / page_size) pages.  The pool holds exactly
    the pages needed (plus ``spare_pages``); pages are handed out in the order of
    a seeded random permutation when ``shuffle``.  Unused table entries are -1.
    Returns (block_table [B, max_pages] int32, num_pages).
    """
    kv = np.asarray(kv_lens, dtype=np.int64)
    need = (kv + page_size - 1) // page_size
    total = int(need.sum())
    num_pages = total + int(spare_pages)
    order = rng(config_id, T_PERM).permutation(num_pages) if shuffle else np.arange(num_pages)
    maxp = max(1, int(need.max()) if need.size else 1)
    bt = np.full((kv.shape[0], maxp), -1, np.int32)
    k = 0
    for b in range(kv.shape[0]):
        n = int(need[b])
        bt[b, :n] = order[k:k + n]
        k += n
    return bt, num_pages


def append_inputs(config_id: int, s: Shape, n: int, bf16: bool = True):
    """Raw (pre-norm, pre-rotation) c^KV and k^R rows for a cache append."""
    ckv = normal(config_id, T_CKV_RAW, (n, s.d_c), bf16=bf16)
    kr = normal(config_id, T_KR_RAW, (n, s.d_rope), bf16=bf16)
    return ckv, kr


# The five workloads the library is measured on.  The decode ones give the
# context length per sequence; the prefill ones the sequence length.
WORKLOADS = {
    1: dict(kind="prefill", shape=TINY, B=1, L=64, dtype="f32"),
    2: dict(kind="decode", shape=V3, B=64, context=4096, s_q=1, dtype="bf16"),
    3: dict(kind="prefill", shape=V3, B=1, L=8192, dtype="bf16"),
    4: dict(kind="decode", shape=V3, B=4, context=131072, s_q=1, dtype="bf16"),
    5: dict(kind="decode", shape=V3, B=128, context=(1, 32768), s_q=2, dtype="bf16"),
}


def config_context_lens(config_id: int) -> np.ndarray:
    c = WORKLOADS[config_id]
    if isinstance(c["context"], tuple):
        lo, hi = c["context"]
        return uniform_lengths(config_id, c["B"], lo, hi)
    return np.full(c["B"], c["context"], np.int64)
