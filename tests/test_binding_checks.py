"""The Python binding rejects tensors of the wrong shape, dtype, layout or
device before it calls into the library (so no kernel ever sees them).  These
tests need no GPU: each case fails in the checks, before any launch."""
import pytest
import torch

import head_latent_attention_06_amd as mla


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import os
    if not os.path.exists(mla.LIB_PATH):
        from head_latent_attention_06_amd import build
        build.build()
    mla.lib()


def _decode_args(cfg, B=2, s_q=1, pool=None, bt=None, dtype=torch.bfloat16):
    H, dh, dr, dc = cfg.n_heads, cfg.d_head, cfg.d_rope, cfg.d_c
    pool = torch.zeros((4, cfg.page_size, cfg.row), dtype=dtype) if pool is None else pool
    bt = torch.zeros((B, 2), dtype=torch.int32) if bt is None else bt
    return dict(cfg=cfg, cache=mla.PagedCache(pool, bt), kv_lens=torch.full((B,), 5, dtype=torch.int32),
                max_kv_len=5, q_nope=torch.zeros((B, s_q, H, dh), dtype=dtype),
                q_pe=torch.zeros((B, s_q, H, dr), dtype=dtype), w_uk=torch.zeros((H * dh, dc), dtype=dtype),
                w_uv=torch.zeros((H * dh, dc), dtype=dtype), out=torch.zeros((B, s_q, H, dh), dtype=dtype),
                ws=torch.zeros(256, dtype=torch.uint8))


def _raises(fn, text, **kw):
    with pytest.raises(mla.MLAError) as e:
        fn(**kw)
    assert e.value.status == mla.MLA_ERR_INVALID_ARG
    assert text in str(e.value), str(e.value)


def test_fp8_sized_pool_with_bf16_config_is_rejected():
    """A uint8 pool of 656-byte FP8 rows used with kv_fp8=False would make the
    kernels address 1152-byte rows, past the allocation."""
    cfg = mla.Config()
    pool = torch.zeros((4, 64, 656), dtype=torch.uint8)
    _raises(mla.mla_decode, "pool rows are 656 bytes, the config needs 1152", **_decode_args(cfg, pool=pool))
    # and the other way round
    cfg8 = mla.Config(kv_fp8=True)
    pool = torch.zeros((4, 64, 576), dtype=torch.bfloat16)
    _raises(mla.mla_decode, "pool rows are 1152 bytes, the config needs 656", **_decode_args(cfg8, pool=pool))


def test_pool_page_size_and_rank_checked():
    cfg = mla.Config()
    _raises(mla.mla_decode, "pool pages hold 32 tokens",
            **_decode_args(cfg, pool=torch.zeros((4, 32, 576), dtype=torch.bfloat16)))
    _raises(mla.mla_decode, "pool must be", **_decode_args(cfg, pool=torch.zeros((4 * 64, 576), dtype=torch.bfloat16)))
    nc = torch.zeros((4, 576, 64), dtype=torch.bfloat16).transpose(1, 2)
    _raises(mla.mla_decode, "pool is not contiguous", **_decode_args(cfg, pool=nc))


def test_block_table_checked():
    cfg = mla.Config()
    _raises(mla.mla_decode, "block_table has dtype torch.int64",
            **_decode_args(cfg, bt=torch.zeros((2, 2), dtype=torch.int64)))
    _raises(mla.mla_decode, "block_table has 1 rows for 2 sequences",
            **_decode_args(cfg, bt=torch.zeros((1, 2), dtype=torch.int32)))


def test_decode_tensor_checks():
    cfg = mla.Config()
    a = _decode_args(cfg)
    _raises(mla.mla_decode, "q_nope has dtype torch.float32", **{**a, "q_nope": a["q_nope"].float()})
    _raises(mla.mla_decode, "q_pe has shape", **{**a, "q_pe": torch.zeros((2, 1, 128, 32), dtype=torch.bfloat16)})
    _raises(mla.mla_decode, "w_uk has shape", **{**a, "w_uk": torch.zeros((512, 16384), dtype=torch.bfloat16)})
    _raises(mla.mla_decode, "out has shape", **{**a, "out": torch.zeros((2, 2, 128, 128), dtype=torch.bfloat16)})
    _raises(mla.mla_decode, "kv_lens has dtype torch.int64", **{**a, "kv_lens": a["kv_lens"].long()})
    qt = torch.zeros((2, 1, 128, 128), dtype=torch.bfloat16).transpose(2, 3)
    _raises(mla.mla_decode, "q_nope is not contiguous", **{**a, "q_nope": qt})
    # shapes, dtypes and layouts right, but host memory: refused as well
    _raises(mla.mla_decode, "expected a GPU tensor", **a)


def test_prefill_and_append_tensor_checks():
    cfg = mla.Config()
    pool = torch.zeros((4, 64, 576), dtype=torch.bfloat16)
    cache = mla.PagedCache(pool, torch.zeros((1, 4), dtype=torch.int32))
    h = torch.zeros((1, 8, 7168), dtype=torch.bfloat16)
    out = torch.zeros((1, 8, 128, 128), dtype=torch.bfloat16)
    shapes = mla._weight_shapes(cfg)
    w = {k: torch.zeros(v, dtype=torch.bfloat16) for k, v in shapes.items()}
    _raises(mla.mla_prefill, "h has shape", cfg=cfg, cache=cache, weights=w,
            h=torch.zeros((1, 8, 4096), dtype=torch.bfloat16), out=out)
    _raises(mla.mla_prefill, "out has shape", cfg=cfg, cache=cache, weights=w, h=h,
            out=torch.zeros((1, 8, 128, 64), dtype=torch.bfloat16))
    _raises(mla.mla_prefill, "weight w_kr is missing", cfg=cfg, cache=cache,
            weights={k: v for k, v in w.items() if k != "w_kr"}, h=h, out=out)
    _raises(mla.mla_prefill, "w_qr has shape", cfg=cfg, cache=cache,
            weights={**w, "w_qr": torch.zeros((128 * 32, 1536), dtype=torch.bfloat16)}, h=h, out=out)
    _raises(mla.mla_prefill, "g_kv has dtype torch.float32", cfg=cfg, cache=cache,
            weights={**w, "g_kv": torch.zeros(512)}, h=h, out=out)
    n = 3
    args = dict(cfg=cfg, cache=cache, ckv_raw=torch.zeros((n, 512), dtype=torch.bfloat16),
                kr_raw=torch.zeros((n, 64), dtype=torch.bfloat16), g_kv=torch.zeros(512, dtype=torch.bfloat16),
                seq_idx=torch.zeros(n, dtype=torch.int32), pos=torch.zeros(n, dtype=torch.int32))
    _raises(mla.mla_cache_append, "kr_raw has shape", **{**args, "kr_raw": torch.zeros((n, 576), dtype=torch.bfloat16)})
    _raises(mla.mla_cache_append, "pos has shape", **{**args, "pos": torch.zeros(n + 1, dtype=torch.int32)})
    _raises(mla.mla_cache_append, "expected a GPU tensor", **args)


def test_output_projection_checks():
    cfg = mla.Config()
    x = torch.zeros((4, 16384), dtype=torch.bfloat16)
    _raises(mla.mla_output_projection, "w_o has shape", cfg=cfg, x=x,
            w_o=torch.zeros((7168, 8192), dtype=torch.bfloat16), u=torch.zeros((4, 7168), dtype=torch.bfloat16))
    _raises(mla.mla_output_projection, "u has shape", cfg=cfg, x=x,
            w_o=torch.zeros((7168, 16384), dtype=torch.bfloat16), u=torch.zeros((4, 4096), dtype=torch.bfloat16))
