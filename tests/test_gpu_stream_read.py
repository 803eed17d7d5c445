"""The measurement helpers: the streaming read that times the HBM read
ceiling reads every 16-byte word of its buffer, and the MFMA-rate stream runs
and validates its arguments.

Each thread of the kernel XORs the words it reads and writes the sink only
when the XOR of its four 32-bit lanes equals 0x9E3779B9.  With a zero buffer
the sink is never written; with that value planted in one word, the sink is
written exactly when some thread read that word (an odd number of times).
Planted words sit at the ends of tiles, the middle and the ragged tail, for
one word, a part tile, one tile, one tile per workgroup and several tiles per
workgroup plus a tail.
"""
import pytest
import torch

import head_latent_attention_06_amd as mla

pytestmark = pytest.mark.gpu

MAGIC = 0x9E3779B9 - (1 << 32)  # as a signed int32
TILE16 = 256 * 9  # 16-byte words per tile


def _cus() -> int:
    return torch.cuda.get_device_properties(0).multi_processor_count


def _sizes():
    g = _cus()
    return [1, 255, TILE16, TILE16 * g, TILE16 * g * 5 + 1000]


@pytest.mark.parametrize("si", range(5))
def test_every_word_read(si):
    n16 = _sizes()[si]
    buf = torch.zeros(n16 * 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    mla.mla_stream_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    ntiles = n16 // TILE16
    words = {0, n16 - 1, n16 // 2, TILE16 - 1, TILE16, ntiles * TILE16, ntiles * TILE16 - 1, n16 - 2}
    for w in sorted(x for x in words if 0 <= x < n16):
        for lane in (0, 3):
            buf[4 * w + lane] = MAGIC
            sink.zero_()
            mla.mla_stream_read(buf, sink)
            torch.cuda.synchronize()
            assert int(sink.item()) == MAGIC, (n16, w, lane)
            buf[4 * w + lane] = 0


def test_rejects_ragged_and_misaligned():
    b = torch.zeros(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(mla.MLAError):
        mla.mla_stream_read(b[:17])
    with pytest.raises(mla.MLAError):
        mla.mla_stream_read(b[1:33])


def test_mfma_rate_runs_and_rejects_bad_arguments():
    ops = torch.randn(1 << 17, device="cuda").bfloat16()  # 256 KiB
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    for shape in (16, 32):
        mla.mla_mfma_rate(ops, 4, shape, sink)
    torch.cuda.synchronize()
    assert float(sink.item()) == 0.0  # the accumulators' sum is not the magic value
    # clock counters: 200 rounds are thousands of core cycles per workgroup,
    # and the core clock lies between 0.5 GHz and the 2.4 GHz peak
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for shape in (16, 32):
        clk = torch.zeros(2, dtype=torch.int64, device="cuda")
        mla.mla_mfma_rate(ops, 200, shape, clocks=clk)
        torch.cuda.synchronize()
        cyc, ticks = (int(v) for v in clk.tolist())
        assert cyc > cus * 1000 and ticks > 0
        assert 0.5 <= 0.1 * cyc / ticks <= 2.5
    with pytest.raises(mla.MLAError):
        mla.mla_mfma_rate(ops, 4, 16, clocks=torch.zeros(1, dtype=torch.int64, device="cuda"))
    with pytest.raises(mla.MLAError):
        mla.mla_mfma_rate(ops[: (1 << 17) - 8], 4, 16)  # below 256 KiB
    with pytest.raises(mla.MLAError):
        mla.mla_mfma_rate(ops, 4, 8)  # no such shape
    with pytest.raises(mla.MLAError):
        mla.mla_mfma_rate(ops, 0, 16)
