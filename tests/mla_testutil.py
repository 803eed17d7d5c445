"""Helpers shared by the GPU tests: upload seeded inputs, lay out paged caches,
compare against the float64 oracle."""
from __future__ import annotations

import numpy as np
import torch

import head_latent_attention_06_amd as mla
import mla_inputs as mi

BF16_TOL = 1e-2   # rel-L2 bound for bf16 storage with fp32 accumulation
F32_TOL = 1e-5    # rel-L2 bound for the fp32 path
SENTINEL = 0xFFFF  # bf16 bit pattern of untouched cache slots (a NaN)


def rel_l2(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def dev(a: np.ndarray, dtype=torch.bfloat16) -> torch.Tensor:
    """Upload float32 values (already representable in dtype) to the GPU."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(dtype)


def host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def config(shape: mi.Shape, dtype=torch.bfloat16) -> mla.Config:
    return mla.Config(n_heads=shape.n_heads, d_head=shape.d_head, d_rope=shape.d_rope, d_c=shape.d_c,
                      d_cq=shape.d_cq, d_model=shape.d_model, page_size=shape.page_size, rope_base=shape.rope_base,
                      rms_eps=shape.rms_eps, dtype=dtype)


def paged_cache(cfg: mla.Config, num_pages: int, block_table: np.ndarray, fill_bits: int = SENTINEL) -> mla.PagedCache:
    """An empty pool whose every element holds fill_bits (bf16) or NaN (fp32)."""
    if cfg.dtype == torch.bfloat16:
        signed = fill_bits - 65536 if fill_bits >= 32768 else fill_bits
        pool = torch.full((num_pages, cfg.page_size, cfg.row), signed, dtype=torch.int16, device="cuda")
        pool = pool.view(torch.bfloat16)
    else:
        pool = torch.full((num_pages, cfg.page_size, cfg.row), float("nan"), dtype=torch.float32, device="cuda")
    bt = torch.from_numpy(np.ascontiguousarray(block_table, np.int32)).to("cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    return mla.PagedCache(pool, bt, err)


def fill_cache(cache: mla.PagedCache, rows_per_seq, block_table: np.ndarray, page_size: int, dtype) -> None:
    """Scatter each sequence's rows into its pages (layout only, no arithmetic)."""
    for b, rows in enumerate(rows_per_seq):
        n = rows.shape[0]
        if n == 0:
            continue
        pos = np.arange(n)
        pages = block_table[b, pos // page_size].astype(np.int64)
        flat = torch.from_numpy(pages * page_size + pos % page_size).to("cuda")
        cache.pool.view(-1, cache.pool.shape[-1])[flat] = dev(rows, dtype)


def decode_setup(inp: mi.DecodeInputs, dtype=torch.bfloat16, shuffle=True, config_id=0, spare_pages=0):
    s = inp.shape
    cfg = config(s, dtype)
    bt, npages = mi.block_table(config_id, inp.kv_lens, s.page_size, shuffle=shuffle, spare_pages=spare_pages)
    cache = paged_cache(cfg, npages, bt)
    fill_cache(cache, [inp.seq_rows(b) for b in range(len(inp.kv_lens))], bt, s.page_size, dtype)
    t = dict(q_nope=dev(inp.q_nope, dtype), q_pe=dev(inp.q_pe, dtype), w_uk=dev(inp.w_uk, dtype),
             w_uv=dev(inp.w_uv, dtype), kv_lens=torch.from_numpy(inp.kv_lens.astype(np.int32)).to("cuda"))
    return cfg, cache, bt, t


def run_decode(cfg, cache, t, max_kv: int) -> torch.Tensor:
    B, s_q, H = t["q_nope"].shape[0], t["q_nope"].shape[1], cfg.n_heads
    out = torch.empty((B, s_q, H, cfg.d_head), dtype=cfg.dtype, device="cuda")
    mla.mla_decode(cfg, cache, t["kv_lens"], max_kv, t["q_nope"], t["q_pe"], t["w_uk"], t["w_uv"], out)
    return out


def oracle_decode(inp: mi.DecodeInputs, seqs=None, heads=None):
    from oracle import mla_oracle as om
    s = inp.shape
    rows = [inp.seq_rows(b) for b in range(len(inp.kv_lens))]
    return om.decode(rows, inp.kv_lens, inp.s_q, inp.q_nope, inp.q_pe, inp.w_uk, inp.w_uv, s.d_c, s.scale,
                     seqs=seqs, heads=heads)
