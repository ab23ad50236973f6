"""GPU checks of the measurement aids.  The streaming read reads every 16-byte
word it is given (its combined value reaches the sink only when the words
read combine to the fixed value), including a ragged tail, and writes
nothing otherwise."""
import pytest
import torch

import int4_routed_expert_router_amd as coli

pytestmark = pytest.mark.gpu

MAGIC = 0x12345678


@pytest.mark.parametrize("n16", [1, 1000, 4096, 4097, 300_001])
def test_reads_every_word(n16):
    print("read probe: %d words" % n16, flush=True)
    buf = torch.zeros(n16 * 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    coli.coli_moe_read_probe(buf, n16 * 16, sink)
    torch.cuda.synchronize()
    assert sink.tolist() == [0, 0, 0, 0]
    # the fixed value in the last word: only a lane that loaded it writes
    buf[-4] = MAGIC
    coli.coli_moe_read_probe(buf, n16 * 16, sink)
    torch.cuda.synchronize()
    assert sink.tolist() == [MAGIC, 0, 0, 0]
    # and the first word, with the last cleared
    buf[-4] = 0
    buf[1] = MAGIC
    sink.zero_()
    coli.coli_moe_read_probe(buf, n16 * 16, sink)
    torch.cuda.synchronize()
    assert sink.tolist() == [MAGIC, 0, 0, 0]


def test_bytes_beyond_count_not_read():
    """A word past `bytes` is never loaded."""
    buf = torch.zeros(8 * 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    buf[7 * 4] = MAGIC
    coli.coli_moe_read_probe(buf, 7 * 16, sink)
    torch.cuda.synchronize()
    assert sink.tolist() == [0, 0, 0, 0]


def test_timed_by_kernel_timer():
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    timer = coli.KernelTimer(capacity=16)
    with timer:
        coli.coli_moe_read_probe(buf, buf.numel(), sink)
    torch.cuda.synchronize()
    res = timer.results()
    timer.close()
    assert [n for n, _ in res] == ["read_probe"] and res[0][1] > 0


@pytest.mark.parametrize("kind", [coli.COLI_MFMA_I8_K32, coli.COLI_MFMA_I8_K64,
                                  coli.COLI_MFMA_BF16_K32])
def test_mfma_probe_rate_below_spec(kind):
    """The matrix-core loop runs, writes nothing, and its counted operations
    over its time stay below the dense spec peak of the data type (a count
    that overstates the work, or a loop the compiler dropped, would not)."""
    print("mfma probe kind %d" % kind, flush=True)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    coli.coli_moe_mfma_probe(kind, 64, 256, sink)  # warm-up
    torch.cuda.synchronize()
    timer = coli.KernelTimer(capacity=16)
    with timer:
        ops = coli.coli_moe_mfma_probe(kind, 1024, 2048, sink)
    torch.cuda.synchronize()
    (name, ms), = timer.results()
    timer.close()
    assert name == "mfma_probe" and sink.tolist() == [0, 0, 0, 0]
    peak = 2.5e15 if kind == coli.COLI_MFMA_BF16_K32 else 5.0e15
    rate = ops / (ms * 1e-3)
    assert 0 < rate < 1.05 * peak, (rate, peak)
