"""The benchmark's streaming probes (bench_probe.hip, built beside bench.py
into bench_probe.so): host validation without a GPU, and on the GPU the copy
and XOR results over whole buffers."""

import pytest
import torch

import bench


def test_probe_validation_without_a_gpu():
    if torch.cuda.device_count() > 0:
        pytest.skip("host-validation test runs only without a GPU")
    f = bench.probe_lib().bench_stream_probe
    p = 0x1000  # 16-byte aligned, never dereferenced
    assert f(2, p, p, p, 10240, None) == -1       # unknown kind
    assert f(0, p, None, p, 10000, None) == -1    # not whole 10 KiB rows
    assert f(1, p, None, p, 10240, None) == -1    # kind 1 needs b
    assert f(0, p + 4, None, p, 10240, None) == -1
    assert f(0, None, None, None, 0, None) == 0   # nothing to do


def test_window_probe_validation_without_a_gpu():
    if torch.cuda.device_count() > 0:
        pytest.skip("host-validation test runs only without a GPU")
    f = bench.probe_lib().bench_window_probe
    p = 0x1000
    assert f(2, p, p, p, 2, 8, 3, 1, 4, 0, None) == -1    # unknown kind
    assert f(0, p, None, p, 0, 8, 3, 1, 4, 0, None) == -1  # no samples
    assert f(0, p, None, p, 2, 0, 3, 1, 4, 0, None) == -1  # no rows
    assert f(0, p, None, p, 2, 8, 11, 1, 4, 0, None) == -1  # row past 10 KiB
    assert f(0, p, None, p, 2, 8, 0, 1, 4, 0, None) == -1   # empty row
    assert f(0, p, None, p, 2, 8, 3, 5, 4, 0, None) == -1   # bps > grid
    assert f(0, p, None, p, 2, 8, 3, 0, 4, 0, None) == -1   # bps < 1
    assert f(0, p, None, p, 2, 8, 3, 1, 4, -1, None) == -1  # negative skew
    assert f(1, p, None, p, 2, 8, 3, 1, 4, 0, None) == -1   # kind 1 needs b
    assert f(0, p + 4, None, p, 2, 8, 3, 1, 4, 0, None) == -1  # misaligned
    with pytest.raises(ValueError):  # sizes checked before the library
        bench.run_window_probe(0, torch.zeros(10), torch.zeros(10), 1, 1, 1,
                               1, 1)


@pytest.mark.gpu
def test_probe_results():
    print("[probe] copy and xor over 37 rows", flush=True)
    n = 10240 * 37
    a = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda")
    b = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda")
    d = torch.zeros_like(a)
    bench.run_probe(0, a, d)
    torch.cuda.synchronize()
    assert torch.equal(d, a)
    bench.run_probe(1, a, d, b=b)
    torch.cuda.synchronize()
    assert torch.equal(d, a ^ b)
    with pytest.raises(ValueError):
        bench.run_probe(0, a[:10000], d[:10000])
    with pytest.raises(ValueError):
        bench.run_probe(5, a, d)


@pytest.mark.gpu
@pytest.mark.parametrize("B,N,row_kib,bps,grid,skew", [
    (3, 37, 3, 2, 7, 5),     # ragged: the last group idles, skew wraps
    (1, 100, 6, 4, 4, 0),    # one flat window
    (5, 9, 1, 1, 3, 97),     # skew longer than a sample
])
def test_window_probe_results(B, N, row_kib, bps, grid, skew):
    print(f"[probe] window walk B={B} N={N} row={row_kib} KiB", flush=True)
    n = B * N * row_kib * 1024
    a = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda")
    b = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda")
    d = torch.zeros_like(a)
    bench.run_window_probe(0, a, d, B, N, row_kib, bps, grid, skew)
    torch.cuda.synchronize()
    assert torch.equal(d, a)
    bench.run_window_probe(1, a, d, B, N, row_kib, bps, grid, skew, b=b)
    torch.cuda.synchronize()
    assert torch.equal(d, a ^ b)
