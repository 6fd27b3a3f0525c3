"""The measurement kernels of include/moe_peak.h on the GPU: the streaming
read and the stream beside the MFMAs read every chunk they are meant to read
exactly once (a key planted in one chunk of an otherwise zero buffer shows up
in the XOR they keep; a chunk read twice or never would cancel or miss it),
and the MFMA loops write a finite, repeatable sum for every wave."""
import pytest
import torch

pytestmark = pytest.mark.gpu

KEY = 0x9E3779B9  # the value the kernels compare the XOR of what they read with


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from group_limited_routing_router_amd import moe as m
    m.load_library()
    return m


def _keyed(chunks, at):
    buf = torch.zeros(chunks * 4, dtype=torch.int32, device="cuda")
    buf[at * 4] = KEY - (1 << 32)  # as int32
    return buf


@pytest.mark.parametrize("nontemporal", [False, True])
def test_stream_read_covers_every_chunk_once(moe, nontemporal):
    wg = 4
    chunks = wg * 256 * 8 * 3 + 37  # three whole steps of the grid and a ragged tail
    for at in (0, 1, wg * 256 * 8 + 5, chunks - 38, chunks - 1):
        print(f"[case] stream read key at chunk {at} of {chunks}", flush=True)
        buf = _keyed(chunks, at)
        sink = torch.zeros(4, dtype=torch.int32, device="cuda")
        moe.moe_peak_stream_read(buf, sink, wg, nontemporal=nontemporal)
        torch.cuda.synchronize()
        assert int(sink[0]) & 0xFFFFFFFF == KEY
    # no key: the sink is left alone
    sink = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    moe.moe_peak_stream_read(torch.zeros(chunks * 4, dtype=torch.int32, device="cuda"), sink, wg)
    torch.cuda.synchronize()
    assert int(sink[0]) == 7


@pytest.mark.parametrize("random_operands", [False, True])
def test_mfma_loop_writes_every_wave(moe, random_operands):
    wg = 64
    outs = []
    for _ in range(2):
        sink = torch.full((4 * wg,), float("nan"), dtype=torch.float32, device="cuda")
        flops = moe.moe_peak_mfma_bf16(40, sink, wg, random_operands=random_operands)
        torch.cuda.synchronize()
        assert flops == wg * 4 * 40 * 8 * 32768
        assert bool(torch.isfinite(sink).all())
        outs.append(sink.cpu())
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("loads", [0, 1, 2, 4])
def test_mfma_stream_reads_its_span_once(moe, loads):
    wg, steps = 8, 16
    nthreads = wg * 256
    span = (steps + 8) * loads * nthreads  # chunks one launch reads
    chunks = max(span, 1)
    zero = torch.zeros(chunks * 4, dtype=torch.int32, device="cuda")
    base = torch.full((4 * wg,), float("nan"), dtype=torch.float32, device="cuda")
    flops, nbytes = moe.moe_peak_mfma_stream(zero if loads else None, loads, steps, base, wg)
    torch.cuda.synchronize()
    assert flops == wg * 4 * steps * 16 * 32768 and nbytes == nthreads * steps * loads * 16
    assert bool(torch.isfinite(base).all())
    if not loads:
        return
    # thread 0 (lane 0 of wave 0, whose sum is stored) reads chunks n * nthreads
    for n in (0, 3, (steps + 8) * loads - 1):
        print(f"[case] stream beside MFMAs, {loads} loads, key at chunk {n * nthreads}", flush=True)
        sink = torch.full((4 * wg,), float("nan"), dtype=torch.float32, device="cuda")
        moe.moe_peak_mfma_stream(_keyed(chunks, n * nthreads), loads, steps, sink, wg)
        torch.cuda.synchronize()
        d = (sink - base).cpu()
        assert abs(float(d[0]) - 1.0) < 1e-3, float(d[0])
        assert torch.equal(d[1:], torch.zeros_like(d[1:]))
