"""Python binding of libmla (Multi-head Latent Attention for MI355X / gfx950).

Argument marshalling only: every function takes torch tensors (device memory,
or host memory where noted), passes their data pointers and the current HIP
stream to the C ABI declared in ``include/mla.h``, and raises ``MLAError`` on a
non-OK status.  Every step of the computation runs in the library's kernels;
there is no fallback path.  Building the library: ``build.build()``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_OUT_OF_RANGE, MLA_ERR_WORKSPACE, MLA_ERR_HIP = range(6)
MLA_F32, MLA_BF16 = 0, 1
PREFILL_AUTO, PREFILL_ABSORBED, PREFILL_EXPLICIT = 0, 1, 2
ABI_VERSION = 4  # MLA_ABI_VERSION of the include/mla.h this binding mirrors
MLA_FLAG_BAD_PAGE, MLA_FLAG_BAD_POS, MLA_FLAG_BAD_LEN, MLA_FLAG_BAD_SEQ = 1, 2, 4, 8


class MLAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


class _Config(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("d_head", ctypes.c_int32), ("d_rope", ctypes.c_int32),
                ("d_c", ctypes.c_int32), ("d_cq", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("softmax_scale", ctypes.c_float), ("rope_base", ctypes.c_float),
                ("rms_eps", ctypes.c_float), ("dtype", ctypes.c_int32), ("prefill_form", ctypes.c_int32),
                ("yarn_s", ctypes.c_float), ("yarn_alpha", ctypes.c_float), ("yarn_beta", ctypes.c_float),
                ("yarn_orig_ctx", ctypes.c_int32), ("kv_fp8", ctypes.c_int32)]


class _Cache(ctypes.Structure):
    _fields_ = [("pool", ctypes.c_void_p), ("num_pages", ctypes.c_int64), ("block_table", ctypes.c_void_p),
                ("max_pages_per_seq", ctypes.c_int32), ("err_flags", ctypes.c_void_p)]


class _Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_dq", "g_q", "w_uq", "w_qr", "w_dkv", "g_kv", "w_kr", "w_uk", "w_uv")]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with head_latent_attention_06_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        CP, KP, WP = ctypes.POINTER(_Config), ctypes.POINTER(_Cache), ctypes.POINTER(_Weights)
        sig = {
            "mla_abi_version": (I32, []),
            "mla_cache_row_bytes": (ctypes.c_int64, [CP]),
            "mla_status_string": (ctypes.c_char_p, [I32]),
            "mla_cache_append": (I32, [CP, KP, P, P, P, P, P, I32, I32, P]),
            "mla_project_kv_workspace_size": (I32, [CP, I32, I32, ctypes.POINTER(SZ)]),
            "mla_project_kv": (I32, [CP, KP, WP, P, I32, I32, I32, P, SZ, P]),
            "mla_prefill_workspace_size": (I32, [CP, I32, I32, I32, ctypes.POINTER(SZ)]),
            "mla_prefill": (I32, [CP, KP, WP, P, I32, I32, I32, P, P, SZ, P]),
            "mla_decode_workspace_size": (I32, [CP, I32, I32, I32, ctypes.POINTER(SZ)]),
            "mla_decode": (I32, [CP, KP, P, I32, I32, I32, P, P, P, P, P, P, SZ, P]),
            "mla_decode_num_splits": (I32, [CP, I32, I32, I32]),
            "mla_decode_profiled": (I32, [CP, KP, P, I32, I32, I32, P, P, P, P, P, P, SZ, P, P, P]),
            "mla_prefill_profiled": (I32, [CP, KP, WP, P, I32, I32, I32, P, P, SZ, P, P, P]),
            "mla_output_projection_workspace_size": (I32, [CP, I32, I32, ctypes.POINTER(SZ)]),
            "mla_output_projection": (I32, [CP, P, I32, P, P, I32, P, SZ, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().mla_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != MLA_OK:
        raise MLAError(status, where)


@dataclass
class Config:
    """Layer dimensions; defaults are the DeepSeek-V3 MLA shapes."""

    n_heads: int = 128
    d_head: int = 128
    d_rope: int = 64
    d_c: int = 512
    d_cq: int = 1536
    d_model: int = 7168
    page_size: int = 64
    softmax_scale: float | None = None
    rope_base: float = 10000.0
    rms_eps: float = 1e-6
    dtype: torch.dtype = torch.bfloat16
    prefill_form: int = PREFILL_AUTO  # PREFILL_AUTO / PREFILL_ABSORBED / PREFILL_EXPLICIT
    # YaRN long-context extension; off while yarn_s <= 1 (the V3 values are s = 40,
    # alpha = 1, beta = 32 over an original 4096-token window)
    yarn_s: float = 0.0
    yarn_alpha: float = 1.0
    yarn_beta: float = 32.0
    yarn_orig_ctx: int = 4096
    # FP8 latent cache: E4M3 codes of c^KV with a power-of-two scale per 128
    # values, k^R in bf16; 656-byte rows (bf16 compute only)
    kv_fp8: bool = False

    @property
    def row(self) -> int:
        return self.d_c + self.d_rope

    @property
    def row_bytes(self) -> int:
        """Bytes per cached row (a uint8 pool of [pages, page_size, row_bytes] fits any config)."""
        n = lib().mla_cache_row_bytes(ctypes.byref(self._c()))
        if n < 0:
            raise MLAError(MLA_ERR_INVALID_ARG, "mla_cache_row_bytes")
        return n

    def _c(self) -> _Config:
        scale = self.softmax_scale if self.softmax_scale is not None else (self.d_head + self.d_rope) ** -0.5
        dt = {torch.bfloat16: MLA_BF16, torch.float32: MLA_F32}[self.dtype]
        return _Config(self.n_heads, self.d_head, self.d_rope, self.d_c, self.d_cq, self.d_model, self.page_size,
                       scale, self.rope_base, self.rms_eps, dt, self.prefill_form, self.yarn_s, self.yarn_alpha,
                       self.yarn_beta, self.yarn_orig_ctx, int(self.kv_fp8))


@dataclass
class PagedCache:
    """Caller-owned paged latent cache: pool [num_pages, page_size, d_c + d_rope]."""

    pool: torch.Tensor
    block_table: torch.Tensor          # [n_seqs, max_pages] int32
    err_flags: torch.Tensor | None = None  # [1] int32 or None

    def _c(self) -> _Cache:
        return _Cache(self.pool.data_ptr(), self.pool.shape[0], self.block_table.data_ptr(),
                      self.block_table.shape[1], self.err_flags.data_ptr() if self.err_flags is not None else None)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _weights(w: dict) -> _Weights:
    return _Weights(*[_ptr(w.get(n)) for n in ("w_dq", "g_q", "w_uq", "w_qr", "w_dkv", "g_kv", "w_kr", "w_uk",
                                              "w_uv")])


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------
def mla_cache_append(cfg: Config, cache: PagedCache, ckv_raw, kr_raw, g_kv, seq_idx, pos, stream=None) -> None:
    """Append rows [RMSNorm(ckv_raw[i]) ; RoPE(kr_raw[i], pos[i])] for sequences seq_idx."""
    n = ckv_raw.shape[0]
    _check(lib().mla_cache_append(ctypes.byref(cfg._c()), ctypes.byref(cache._c()), _ptr(ckv_raw), _ptr(kr_raw),
                                  _ptr(g_kv), _ptr(seq_idx), _ptr(pos), n, cache.block_table.shape[0],
                                  _stream(stream)), "mla_cache_append")


def mla_project_kv_workspace_size(cfg: Config, B: int, L: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().mla_project_kv_workspace_size(ctypes.byref(cfg._c()), B, L, ctypes.byref(n)),
           "mla_project_kv_workspace_size")
    return n.value


def mla_project_kv(cfg: Config, cache: PagedCache, weights: dict, h, start_pos: int = 0, ws=None,
                   stream=None) -> None:
    """[W^DKV ; W^KR] h for h [B, L, d_model], then append the rows at start_pos .. start_pos+L-1."""
    B, L = h.shape[0], h.shape[1]
    if ws is None:
        ws = _workspace(mla_project_kv_workspace_size(cfg, B, L), h.device)
    _check(lib().mla_project_kv(ctypes.byref(cfg._c()), ctypes.byref(cache._c()), ctypes.byref(_weights(weights)),
                                _ptr(h), B, L, start_pos, _ptr(ws), ws.numel(), _stream(stream)), "mla_project_kv")


def mla_prefill_workspace_size(cfg: Config, B: int, L: int, start_pos: int = 0) -> int:
    n = ctypes.c_size_t()
    _check(lib().mla_prefill_workspace_size(ctypes.byref(cfg._c()), B, L, start_pos, ctypes.byref(n)),
           "mla_prefill_workspace_size")
    return n.value


def mla_prefill(cfg: Config, cache: PagedCache, weights: dict, h, out, start_pos: int = 0, ws=None,
                stream=None, attn_events=None) -> None:
    """Causal prefill of h [B, L, d_model] into out [B, L, n_heads, d_head].

    attn_events: optional (start, stop) raw hipEvent_t handles recorded around
    the attention kernel (mla_prefill_profiled)."""
    B, L = h.shape[0], h.shape[1]
    if ws is None:
        ws = _workspace(mla_prefill_workspace_size(cfg, B, L, start_pos), h.device)
    ev0, ev1 = attn_events if attn_events is not None else (None, None)
    _check(lib().mla_prefill_profiled(ctypes.byref(cfg._c()), ctypes.byref(cache._c()),
                                      ctypes.byref(_weights(weights)), _ptr(h), B, L, start_pos, _ptr(out), _ptr(ws),
                                      ws.numel(), _stream(stream), ev0, ev1), "mla_prefill")


def mla_output_projection_workspace_size(cfg: Config, T: int, width: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().mla_output_projection_workspace_size(ctypes.byref(cfg._c()), T, width, ctypes.byref(n)),
           "mla_output_projection_workspace_size")
    return n.value


def mla_output_projection(cfg: Config, x, w_o, u, ws=None, stream=None) -> None:
    """u [T, d_model] = x [T, width] W^O^T with W^O [d_model, width] (width = n_heads * d_head,
    or n_heads * d_c for the folded W^O')."""
    T, width = x.shape[0], x.numel() // max(x.shape[0], 1)
    if ws is None:
        ws = _workspace(max(mla_output_projection_workspace_size(cfg, T, width), 1), x.device)
    _check(lib().mla_output_projection(ctypes.byref(cfg._c()), _ptr(x), width, _ptr(w_o), _ptr(u), T, _ptr(ws),
                                       ws.numel(), _stream(stream)), "mla_output_projection")


def mla_decode_workspace_size(cfg: Config, B: int, s_q: int, max_kv_len: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().mla_decode_workspace_size(ctypes.byref(cfg._c()), B, s_q, max_kv_len, ctypes.byref(n)),
           "mla_decode_workspace_size")
    return n.value


def mla_decode_num_splits(cfg: Config, B: int, s_q: int, max_kv_len: int) -> int:
    return int(lib().mla_decode_num_splits(ctypes.byref(cfg._c()), B, s_q, max_kv_len))


def mla_decode(cfg: Config, cache: PagedCache, kv_lens, max_kv_len: int, q_nope, q_pe, w_uk, w_uv, out, ws=None,
               stream=None, attn_events=None) -> None:
    """One decode step: q_nope [B, s_q, H, d_head], q_pe [B, s_q, H, d_rope] -> out [B, s_q, H, d_head].

    attn_events: optional (start, stop) raw hipEvent_t handles recorded around
    the attention kernel (mla_decode_profiled)."""
    B, s_q = q_nope.shape[0], q_nope.shape[1]
    if ws is None:
        ws = _workspace(mla_decode_workspace_size(cfg, B, s_q, max_kv_len), q_nope.device)
    ev0, ev1 = attn_events if attn_events is not None else (None, None)
    _check(lib().mla_decode_profiled(ctypes.byref(cfg._c()), ctypes.byref(cache._c()), _ptr(kv_lens),
                                     int(max_kv_len), B, s_q, _ptr(q_nope), _ptr(q_pe), _ptr(w_uk), _ptr(w_uv),
                                     _ptr(out), _ptr(ws), ws.numel(), _stream(stream), ev0, ev1), "mla_decode")
