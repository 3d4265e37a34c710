"""The benchmark's reference kernels (libarnfp8_ref.so) do what their figures
claim: the traffic twin writes, per 16-byte chunk, the XOR of the chunk's
loads (16 bytes) and its halves folded to 8 bytes; the write-only kernel
writes its pattern over every byte; the read-only kernel writes nothing; the
exchange kernel advances every workgroup's count by one per launch with no
wait running out.  Checked against plain PyTorch integer ops on the device."""
import ctypes

import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def ref():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bench

    return bench.ref_library()


def _arr(ts):
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _xor_chunks(streams):
    """XOR of the streams, viewed as int32 words."""
    acc = streams[0].view(torch.int32).clone()
    for s in streams[1:]:
        acc ^= s.view(torch.int32)
    return acc


@pytest.mark.parametrize("S,rows,cols,threads,vpt", [(9, 37, 7168, 448, 2), (5, 8, 7168, 512, 2),
                                                      (9, 5, 8192, 1024, 1), (5, 64, 1024, 128, 1)])
def test_twin_writes_the_xor_of_its_loads(ref, S, rows, cols, threads, vpt):
    g = torch.Generator(device=DEV).manual_seed(S * 1000 + rows)
    xs = [torch.randint(-2**31, 2**31 - 1, (rows, cols // 2), generator=g, device=DEV,
                        dtype=torch.int32).view(torch.bfloat16) for _ in range(S)]
    out16 = torch.zeros((rows, cols), dtype=torch.bfloat16, device=DEV)
    out8 = torch.zeros((rows, cols), dtype=torch.uint8, device=DEV)
    st = ref.arnref_twin(_arr(xs), S, out16.data_ptr(), out8.data_ptr(), rows, 2 * cols, threads,
                         vpt, _stream())
    assert st == 0
    torch.cuda.synchronize()
    want = _xor_chunks(xs).view(rows, cols // 8, 4)  # 4 words per 16-byte chunk
    assert torch.equal(out16.view(torch.int32).view(rows, cols // 8, 4), want)
    folded = torch.stack([want[..., 0] ^ want[..., 2], want[..., 1] ^ want[..., 3]], dim=-1)
    assert torch.equal(out8.view(torch.int32).view(rows, cols // 8, 2), folded)


def test_write_kernel_covers_every_byte_and_read_kernel_writes_nothing(ref):
    rows, cols = 33, 7168
    outs = [torch.zeros((rows, cols), dtype=torch.bfloat16, device=DEV) for _ in range(2)]
    assert ref.arnref_write(_arr(outs), 2, rows, 2 * cols, 0, 0, _stream()) == 0
    torch.cuda.synchronize()
    for o in outs:
        w = o.view(torch.int32).view(rows, cols // 8, 4)
        assert torch.all(w[..., 2] == 0x3F803F80) and torch.all(w[..., 3] == 0x3F803F80)
        assert torch.equal(w[..., 0], torch.arange(rows, device=DEV, dtype=torch.int32)
                           .view(rows, 1).expand(rows, cols // 8))
    xs = [torch.randn((rows, cols), device=DEV).to(torch.bfloat16) for _ in range(9)]
    sink = torch.full((rows, 16), 0x5A, dtype=torch.uint8, device=DEV)
    assert ref.arnref_read(_arr(xs), 9, sink.data_ptr(), rows, 2 * cols, 0, 0, _stream()) == 0
    torch.cuda.synchronize()
    assert torch.all(sink == 0x5A)


def test_bad_reference_arguments_are_rejected_before_launch(ref):
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device=DEV)
    a = _arr([x] * 9)
    assert ref.arnref_read(a, 7, x.data_ptr(), 4, 128, 0, 0, _stream()) == 4  # unsupported count
    assert ref.arnref_read(a, 9, x.data_ptr(), 4, 120, 0, 0, _stream()) == 3  # not 16-byte rows
    assert ref.arnref_twin(a, 9, x.data_ptr(), x.data_ptr(), 4, 128, 96, 1, _stream()) == 3
    assert ref.arnref_empty(4, 96, _stream()) == 3
    assert ref.arnref_exchange(x.data_ptr(), 250, 8, 8, x.data_ptr(), _stream()) == 3


@pytest.mark.parametrize("S,stride", [(2, 1), (8, 1), (2, 8), (8, 8)])
def test_exchange_counts_advance_in_step(ref, S, stride):
    nwg = 256
    words = torch.zeros((nwg,), dtype=torch.int64, device=DEV)
    timeouts = torch.zeros((1,), dtype=torch.int32, device=DEV)
    for _ in range(5):
        assert ref.arnref_exchange(words.data_ptr(), nwg, S, stride, timeouts.data_ptr(),
                                   _stream()) == 0
    torch.cuda.synchronize()
    assert int(timeouts.item()) == 0
    counts = (words >> 32).cpu()
    payload = (words & 0xFFFFFFFF).cpu()
    assert torch.all(counts == 5)
    assert torch.equal(payload, torch.arange(nwg, dtype=torch.int64))
