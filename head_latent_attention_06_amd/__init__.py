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
ABI_VERSION = 5  # MLA_ABI_VERSION of the include/mla.h this binding mirrors
MLA_FLAG_BAD_PAGE, MLA_FLAG_BAD_POS, MLA_FLAG_BAD_LEN, MLA_FLAG_BAD_SEQ = 1, 2, 4, 8


class MLAError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}" + (f" ({detail})" if detail else ""))


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
            "mla_decode_noalloc": (I32, [CP, KP, P, I32, I32, I32, P, P, P, P, P, P]),
            "mla_stream_read": (I32, [P, ctypes.c_int64, P, P]),
            "mla_mfma_rate": (I32, [P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, P, P, P]),
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
    """Caller-owned paged latent cache: pool [num_pages, page_size, d_c + d_rope]
    (any element type whose row is Config.row_bytes bytes, e.g. uint8 [.., 656]
    for the FP8 cache)."""

    pool: torch.Tensor
    block_table: torch.Tensor          # [n_seqs, max_pages] int32
    err_flags: torch.Tensor | None = None  # [1] int32 or None

    def _c(self) -> _Cache:
        return _Cache(self.pool.data_ptr(), self.pool.shape[0], self.block_table.data_ptr(),
                      self.block_table.shape[1], self.err_flags.data_ptr() if self.err_flags is not None else None)


# ---------------------------------------------------------------------------
# Argument checks, made before any call into the library (the library checks
# sizes and pointers too, but it cannot see a tensor's shape, dtype or layout:
# a pool of the wrong row width would make its kernels address past it).
def _bad(where: str, detail: str):
    raise MLAError(MLA_ERR_INVALID_ARG, where, detail)


def _tensor(where: str, name: str, t, dtype=None, shape=None) -> None:
    """t is a contiguous tensor of dtype with the given shape (None = any extent);
    where it lives is checked by _on_gpu once every shape has been."""
    if not isinstance(t, torch.Tensor):
        _bad(where, f"{name} is not a tensor")
    if dtype is not None and t.dtype != dtype:
        _bad(where, f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and (t.dim() != len(shape) or
                              any(want is not None and got != want for got, want in zip(t.shape, shape))):
        _bad(where, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        _bad(where, f"{name} is not contiguous")


def _on_gpu(where: str, **tensors) -> None:
    for name, t in tensors.items():
        if t is not None and t.device.type != "cuda":
            _bad(where, f"{name} is on {t.device}, expected a GPU tensor")


def _cache_ok(where: str, cfg: "Config", cache: PagedCache, n_seqs: int) -> None:
    p = cache.pool
    if not isinstance(p, torch.Tensor) or p.dim() != 3:
        _bad(where, "pool must be [num_pages, page_size, row]")
    if p.shape[1] != cfg.page_size:
        _bad(where, f"pool pages hold {p.shape[1]} tokens, the config says {cfg.page_size}")
    if p.shape[2] * p.element_size() != cfg.row_bytes:
        _bad(where, f"pool rows are {p.shape[2] * p.element_size()} bytes, the config needs {cfg.row_bytes}")
    _tensor(where, "pool", p)
    _tensor(where, "block_table", cache.block_table, torch.int32, (None, None))
    if cache.block_table.shape[0] < n_seqs:
        _bad(where, f"block_table has {cache.block_table.shape[0]} rows for {n_seqs} sequences")
    if cache.err_flags is not None:
        _tensor(where, "err_flags", cache.err_flags, torch.int32)
        if cache.err_flags.numel() < 1:
            _bad(where, "err_flags is empty")


def _ws_bytes(where: str, ws) -> int:
    _tensor(where, "workspace", ws)
    _on_gpu(where, workspace=ws)
    return ws.numel() * ws.element_size()


def _cache_on_gpu(where: str, cache: PagedCache) -> None:
    _on_gpu(where, pool=cache.pool, block_table=cache.block_table, err_flags=cache.err_flags)


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


def _weight_shapes(cfg: "Config") -> dict:
    H = cfg.n_heads
    return {"w_dq": (cfg.d_cq, cfg.d_model), "g_q": (cfg.d_cq,), "w_uq": (H * cfg.d_head, cfg.d_cq),
            "w_qr": (H * cfg.d_rope, cfg.d_cq), "w_dkv": (cfg.d_c, cfg.d_model), "g_kv": (cfg.d_c,),
            "w_kr": (cfg.d_rope, cfg.d_model), "w_uk": (H * cfg.d_head, cfg.d_c), "w_uv": (H * cfg.d_head, cfg.d_c)}


def _weights_ok(where: str, cfg: "Config", w: dict, names) -> None:
    shapes = _weight_shapes(cfg)
    for n in names:
        if w.get(n) is None:
            _bad(where, f"weight {n} is missing")
        _tensor(where, n, w[n], cfg.dtype, shapes[n])


# ---------------------------------------------------------------------------
def mla_cache_append(cfg: Config, cache: PagedCache, ckv_raw, kr_raw, g_kv, seq_idx, pos, stream=None) -> None:
    """Append rows [RMSNorm(ckv_raw[i]) ; RoPE(kr_raw[i], pos[i])] for sequences seq_idx."""
    where = "mla_cache_append"
    n = ckv_raw.shape[0]
    _cache_ok(where, cfg, cache, 0)
    _tensor(where, "ckv_raw", ckv_raw, cfg.dtype, (n, cfg.d_c))
    _tensor(where, "kr_raw", kr_raw, cfg.dtype, (n, cfg.d_rope))
    _tensor(where, "g_kv", g_kv, cfg.dtype, (cfg.d_c,))
    _tensor(where, "seq_idx", seq_idx, torch.int32, (n,))
    _tensor(where, "pos", pos, torch.int32, (n,))
    _on_gpu(where, ckv_raw=ckv_raw, kr_raw=kr_raw, g_kv=g_kv, seq_idx=seq_idx, pos=pos)
    _cache_on_gpu(where, cache)
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
    where = "mla_project_kv"
    _tensor(where, "h", h, cfg.dtype, (None, None, cfg.d_model))
    B, L = h.shape[0], h.shape[1]
    _cache_ok(where, cfg, cache, B)
    _weights_ok(where, cfg, weights, ("w_dkv", "w_kr", "g_kv"))
    _on_gpu(where, h=h, **{k: weights[k] for k in ("w_dkv", "w_kr", "g_kv")})
    _cache_on_gpu(where, cache)
    if ws is None:
        ws = _workspace(mla_project_kv_workspace_size(cfg, B, L), h.device)
    _check(lib().mla_project_kv(ctypes.byref(cfg._c()), ctypes.byref(cache._c()), ctypes.byref(_weights(weights)),
                                _ptr(h), B, L, start_pos, _ptr(ws), _ws_bytes(where, ws), _stream(stream)), where)


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
    where = "mla_prefill"
    _tensor(where, "h", h, cfg.dtype, (None, None, cfg.d_model))
    B, L = h.shape[0], h.shape[1]
    _tensor(where, "out", out, cfg.dtype, (B, L, cfg.n_heads, cfg.d_head))
    _cache_ok(where, cfg, cache, B)
    _weights_ok(where, cfg, weights, tuple(_weight_shapes(cfg)))
    _on_gpu(where, h=h, out=out, **{k: weights[k] for k in _weight_shapes(cfg)})
    _cache_on_gpu(where, cache)
    if ws is None:
        ws = _workspace(mla_prefill_workspace_size(cfg, B, L, start_pos), h.device)
    args = [ctypes.byref(cfg._c()), ctypes.byref(cache._c()), ctypes.byref(_weights(weights)), _ptr(h), B, L,
            start_pos, _ptr(out), _ptr(ws), _ws_bytes(where, ws), _stream(stream)]
    if attn_events is None:
        _check(lib().mla_prefill(*args), where)
    else:
        _check(lib().mla_prefill_profiled(*args, *attn_events), where)


def mla_output_projection_workspace_size(cfg: Config, T: int, width: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().mla_output_projection_workspace_size(ctypes.byref(cfg._c()), T, width, ctypes.byref(n)),
           "mla_output_projection_workspace_size")
    return n.value


def mla_output_projection(cfg: Config, x, w_o, u, ws=None, stream=None) -> None:
    """u [T, d_model] = x [T, width] W^O^T with W^O [d_model, width] (width = n_heads * d_head,
    or n_heads * d_c for the folded W^O')."""
    where = "mla_output_projection"
    _tensor(where, "x", x, cfg.dtype)
    if x.dim() < 2:
        _bad(where, "x must be [T, width] or [T, n_heads, d_head]")
    T, width = x.shape[0], x.numel() // max(x.shape[0], 1)
    _tensor(where, "w_o", w_o, cfg.dtype, (cfg.d_model, width))
    _tensor(where, "u", u, cfg.dtype, (T, cfg.d_model))
    _on_gpu(where, x=x, w_o=w_o, u=u)
    if ws is None:
        ws = _workspace(max(mla_output_projection_workspace_size(cfg, T, width), 1), x.device)
    _check(lib().mla_output_projection(ctypes.byref(cfg._c()), _ptr(x), width, _ptr(w_o), _ptr(u), T, _ptr(ws),
                                       _ws_bytes(where, ws), _stream(stream)), where)


def mla_decode_workspace_size(cfg: Config, B: int, s_q: int, max_kv_len: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().mla_decode_workspace_size(ctypes.byref(cfg._c()), B, s_q, max_kv_len, ctypes.byref(n)),
           "mla_decode_workspace_size")
    return n.value


def mla_decode_num_splits(cfg: Config, B: int, s_q: int, max_kv_len: int) -> int:
    return int(lib().mla_decode_num_splits(ctypes.byref(cfg._c()), B, s_q, max_kv_len))


def _decode_inputs_ok(where, cfg, cache, kv_lens, q_nope, q_pe, w_uk, w_uv, out):
    _tensor(where, "q_nope", q_nope, cfg.dtype, (None, None, cfg.n_heads, cfg.d_head))
    B, s_q = q_nope.shape[0], q_nope.shape[1]
    _tensor(where, "q_pe", q_pe, cfg.dtype, (B, s_q, cfg.n_heads, cfg.d_rope))
    _tensor(where, "w_uk", w_uk, cfg.dtype, (cfg.n_heads * cfg.d_head, cfg.d_c))
    _tensor(where, "w_uv", w_uv, cfg.dtype, (cfg.n_heads * cfg.d_head, cfg.d_c))
    _tensor(where, "out", out, cfg.dtype, (B, s_q, cfg.n_heads, cfg.d_head))
    _tensor(where, "kv_lens", kv_lens, torch.int32, (B,))
    _cache_ok(where, cfg, cache, B)
    _on_gpu(where, q_nope=q_nope, q_pe=q_pe, w_uk=w_uk, w_uv=w_uv, out=out, kv_lens=kv_lens)
    _cache_on_gpu(where, cache)
    return B, s_q


def mla_decode_noalloc(cfg: Config, cache: PagedCache, kv_lens, max_kv_len: int, q_nope, q_pe, w_uk, w_uv, out,
                       stream=None) -> None:
    """mla_decode with the library's per-GPU scratch array as its workspace
    (allocates nothing; calls on one GPU must not overlap)."""
    where = "mla_decode_noalloc"
    B, s_q = _decode_inputs_ok(where, cfg, cache, kv_lens, q_nope, q_pe, w_uk, w_uv, out)
    _check(lib().mla_decode_noalloc(ctypes.byref(cfg._c()), ctypes.byref(cache._c()), _ptr(kv_lens),
                                    int(max_kv_len), B, s_q, _ptr(q_nope), _ptr(q_pe), _ptr(w_uk), _ptr(w_uv),
                                    _ptr(out), _stream(stream)), where)


def mla_decode(cfg: Config, cache: PagedCache, kv_lens, max_kv_len: int, q_nope, q_pe, w_uk, w_uv, out, ws=None,
               stream=None, attn_events=None) -> None:
    """One decode step: q_nope [B, s_q, H, d_head], q_pe [B, s_q, H, d_rope] -> out [B, s_q, H, d_head].

    attn_events: optional (start, stop) raw hipEvent_t handles recorded around
    the attention kernel (mla_decode_profiled)."""
    where = "mla_decode"
    B, s_q = _decode_inputs_ok(where, cfg, cache, kv_lens, q_nope, q_pe, w_uk, w_uv, out)
    if ws is None:
        ws = _workspace(mla_decode_workspace_size(cfg, B, s_q, max_kv_len), q_nope.device)
    args = [ctypes.byref(cfg._c()), ctypes.byref(cache._c()), _ptr(kv_lens), int(max_kv_len), B, s_q, _ptr(q_nope),
            _ptr(q_pe), _ptr(w_uk), _ptr(w_uv), _ptr(out), _ptr(ws), _ws_bytes(where, ws), _stream(stream)]
    if attn_events is None:
        _check(lib().mla_decode(*args), where)
    else:
        _check(lib().mla_decode_profiled(*args, *attn_events), where)


def mla_mfma_rate(operands, iters: int, shape: int = 16, sink=None, clocks=None, stream=None) -> None:
    """A stream of independent MFMAs on all CUs (2^20 FLOP per wave per
    round, `iters` rounds, one workgroup of four waves per CU) with operand
    fragments taken from `operands` (a contiguous GPU bf16 tensor of at least
    256 KiB): the sustained matrix-core rate.  shape 16 or 32 picks the
    16x16x32 or the 32x32x16 instruction.  clocks (optional, a zeroed GPU
    int64 tensor of 2 elements) receives the core-clock cycles and 100 MHz
    ticks the workgroups spent in their MFMA rounds."""
    where = "mla_mfma_rate"
    _tensor(where, "operands", operands, torch.bfloat16)
    if sink is not None:
        _tensor(where, "sink", sink, torch.float32)
    if clocks is not None:
        _tensor(where, "clocks", clocks, torch.int64)
        if clocks.numel() < 2:
            _bad(where, "clocks needs 2 elements")
    _on_gpu(where, operands=operands, sink=sink, clocks=clocks)
    _check(lib().mla_mfma_rate(_ptr(operands), operands.numel() * 2, int(iters), int(shape),
                               None if sink is None else _ptr(sink), None if clocks is None else _ptr(clocks),
                               _stream(stream)), where)


def mla_stream_read(src, sink=None, stream=None) -> None:
    """Read all of src (a contiguous GPU tensor) once: the HBM read ceiling.
    sink (optional, a GPU int32 tensor) receives 0x9E3779B9 only when that is
    the XOR of all 32-bit words read, which lets a test check that every word
    is read exactly once."""
    where = "mla_stream_read"
    _tensor(where, "src", src)
    if sink is not None:
        _tensor(where, "sink", sink, torch.int32)
    _on_gpu(where, src=src, sink=sink)
    _check(lib().mla_stream_read(_ptr(src), src.numel() * src.element_size(),
                                 None if sink is None else _ptr(sink), _stream(stream)), where)
