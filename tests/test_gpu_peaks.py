"""GPU: the measured-ceiling kernels (ix_peaks.h) do the work they are timed on: the copy is
exact, the gather reads exactly the listed rows (XOR checksum against numpy), and the
MFMA loop runs for every VALU setting."""
import numpy as np
import pytest
import torch

from indexed_sparse_attention_ix_amd import binding as bd
from parity_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_peak_copy_exact():
    say("[ix_peak_copy] 3 MiB + 48 bytes")
    n = 3 * (1 << 20) + 48
    src = torch.randint(0, 256, (n,), dtype=torch.int32).to(torch.uint8).to(DEV)
    dst = torch.zeros_like(src)
    bd.ix_peak_copy(src.data_ptr(), dst.data_ptr(), n, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_peak_gather_checksum():
    say("[ix_peak_gather] 4096 rows of 256 B, 100003 gathers with out-of-range rows")
    g = torch.Generator().manual_seed(5)
    table = torch.randint(-2**31, 2**31 - 1, (4096 * 64,), generator=g, dtype=torch.int32)
    rows = torch.randint(-5, 4096 + 5, (100003,), generator=g, dtype=torch.int32)
    out = torch.zeros(1, dtype=torch.int32, device=DEV)
    table_d, rows_d = table.to(DEV), rows.to(DEV)   # kept alive until the kernel has run
    bd.ix_peak_gather(table_d.data_ptr(), 4096 * 256, rows_d.data_ptr(), rows.numel(),
                      out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    t = table.numpy().view(np.uint32).reshape(4096, 64)
    row_x = np.bitwise_xor.reduce(t, axis=1)
    r = rows.numpy()
    valid = r[(r >= 0) & (r < 4096)]
    counts = np.bincount(valid, minlength=4096)
    want = np.bitwise_xor.reduce(np.where(counts % 2 == 1, row_x, 0))
    assert int(out.cpu().numpy().view(np.uint32)[0]) == int(want)


def test_peak_mfma_runs():
    ops = torch.full((34 * 64 * 32,), 0x38, dtype=torch.uint8, device=DEV)
    for nv in (0, 4, 8, 12):
        say(f"[ix_peak_mfma_fp8] valu_per_mfma={nv}")
        out = torch.zeros(1, dtype=torch.float32, device=DEV)
        bd.ix_peak_mfma_fp8(ops.data_ptr(), nv, 8, 4, out.data_ptr(),
                            torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all() and out.item() != 0.0


def test_peak_atomic_add_counts():
    say("[ix_peak_atomic_add] 1000 rows, 50007 listed rows with out-of-range entries")
    g = torch.Generator().manual_seed(9)
    rows = torch.randint(-3, 1003, (50007,), generator=g, dtype=torch.int32)
    table = torch.zeros(1000 * 128, dtype=torch.float32, device=DEV)
    rows_d = rows.to(DEV)
    bd.ix_peak_atomic_add(table.data_ptr(), 1000, rows_d.data_ptr(), rows.numel(),
                          torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    r = rows.numpy()
    want = np.bincount(r[(r >= 0) & (r < 1000)], minlength=1000).astype(np.float32)
    got = table.view(1000, 128).cpu().numpy()
    assert np.array_equal(got, np.repeat(want[:, None], 128, axis=1))
