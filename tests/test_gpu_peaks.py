"""GPU: the measured-ceiling kernels (ix_peaks.h) do the work they are timed on: the copy is
exact, the read-only stream, the row gather and the selection gather read exactly the bytes
they should (XOR checksums against numpy), and the MFMA loop runs for every VALU setting."""
import numpy as np
import pytest
import torch

from indexed_sparse_attention_ix_amd import peaks as pk
from parity_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_peak_copy_exact():
    say("[ix_peak_copy] 3 MiB + 48 bytes")
    n = 3 * (1 << 20) + 48
    src = torch.randint(0, 256, (n,), dtype=torch.int32).to(torch.uint8).to(DEV)
    dst = torch.zeros_like(src)
    pk.ix_peak_copy(src.data_ptr(), dst.data_ptr(), n, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


@pytest.mark.parametrize("blocks", [1000, 4096])
def test_peak_gather_checksum(blocks):
    say(f"[ix_peak_gather] 4096 rows of 256 B, 100003 gathers with out-of-range rows, {blocks} blocks")
    g = torch.Generator().manual_seed(5)
    table = torch.randint(-2**31, 2**31 - 1, (4096 * 64,), generator=g, dtype=torch.int32)
    rows = torch.randint(-5, 4096 + 5, (100003,), generator=g, dtype=torch.int32)
    out = torch.zeros(blocks, dtype=torch.int32, device=DEV)
    table_d, rows_d = table.to(DEV), rows.to(DEV)   # kept alive until the kernel has run
    pk.ix_peak_gather(table_d.data_ptr(), 4096 * 256, rows_d.data_ptr(), rows.numel(), blocks,
                      out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    t = table.numpy().view(np.uint32).reshape(4096, 64)
    row_x = np.bitwise_xor.reduce(t, axis=1)
    r = rows.numpy()
    valid = r[(r >= 0) & (r < 4096)]
    counts = np.bincount(valid, minlength=4096)
    want = np.bitwise_xor.reduce(np.where(counts % 2 == 1, row_x, 0))
    assert int(np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))) == int(want)


@pytest.mark.parametrize("blocks,nt", [(7, 0), (1000, 0), (1000, 1)])
def test_peak_gather_wide_checksum(blocks, nt):
    """Load step i of wave w reads its rows in segment (w + i) mod n_seg: the XOR of all words
    read, computed on the host from that mapping, with rows outside a segment reading zero."""
    n_seg, seg_rows, n = 3, 1024, 70001
    say(f"[ix_peak_gather_wide] {n_seg} segments of {seg_rows} rows, {n} gathers, {blocks} blocks")
    g = torch.Generator().manual_seed(6)
    table = torch.randint(-2**31, 2**31 - 1, (n_seg * seg_rows * 64,), generator=g, dtype=torch.int32)
    rows = torch.randint(-3, seg_rows + 3, (n,), generator=g, dtype=torch.int32)
    out = torch.zeros(blocks, dtype=torch.int32, device=DEV)
    table_d, rows_d = table.to(DEV), rows.to(DEV)
    pk.ix_peak_gather_wide(table_d.data_ptr(), seg_rows * 256, n_seg, rows_d.data_ptr(), n, blocks,
                           nt, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    row_x = np.bitwise_xor.reduce(table.numpy().view(np.uint32).reshape(n_seg, seg_rows, 64), axis=2)
    groups = blocks * 256 // 16           # 16 lanes per row read
    r = np.arange(n)
    step, rem = r // (groups * 8), r % (groups * 8)
    wave = (rem % groups) // 4            # 4 lane groups per wave
    seg = (wave + step) % n_seg
    rv = rows.numpy()
    ok = (rv >= 0) & (rv < seg_rows)
    counts = np.zeros((n_seg, seg_rows), dtype=np.int64)
    np.add.at(counts, (seg[ok], rv[ok]), 1)
    want = np.bitwise_xor.reduce(np.where(counts % 2 == 1, row_x, 0).ravel())
    assert int(np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))) == int(want)


def test_peak_mfma_runs():
    ops = torch.full((34 * 64 * 32,), 0x38, dtype=torch.uint8, device=DEV)
    for nv in (0, 4, 8, 12):
        say(f"[ix_peak_mfma_fp8] valu_per_mfma={nv}")
        out = torch.zeros(1, dtype=torch.float32, device=DEV)
        pk.ix_peak_mfma_fp8(ops.data_ptr(), nv, 8, 4, out.data_ptr(),
                            torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all() and out.item() != 0.0


def test_peak_atomic_add_counts():
    say("[ix_peak_atomic_add] 1000 rows, 50007 listed rows with out-of-range entries")
    g = torch.Generator().manual_seed(9)
    rows = torch.randint(-3, 1003, (50007,), generator=g, dtype=torch.int32)
    table = torch.zeros(1000 * 128, dtype=torch.float32, device=DEV)
    rows_d = rows.to(DEV)
    pk.ix_peak_atomic_add(table.data_ptr(), 1000, rows_d.data_ptr(), rows.numel(),
                          torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    r = rows.numpy()
    want = np.bincount(r[(r >= 0) & (r < 1000)], minlength=1000).astype(np.float32)
    got = table.view(1000, 128).cpu().numpy()
    assert np.array_equal(got, np.repeat(want[:, None], 128, axis=1))


@pytest.mark.parametrize("n,blocks,nt", [(5 * (1 << 20) + 32, 777, 1), (5 * (1 << 20) + 32, 4096, 0),
                                         ((1 << 30) + 48, 1024, 1)])
def test_peak_read_checksum(n, blocks, nt):
    """The last case crosses the 1 GiB segment boundary of the kernel's buffer resources."""
    say(f"[ix_peak_read] {n} bytes, {blocks} blocks, nontemporal {nt}")
    g = torch.Generator().manual_seed(6)
    src = torch.randint(-2**31, 2**31 - 1, (n // 4,), generator=g, dtype=torch.int32)
    out = torch.zeros(blocks, dtype=torch.int32, device=DEV)
    src_d = src.to(DEV)
    pk.ix_peak_read(src_d.data_ptr(), n, blocks, nt, out.data_ptr(),
                    torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(src.numpy().view(np.uint32))
    assert int(np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))) == int(want)


@pytest.mark.parametrize("d,splits,occ", [(128, 1, 0), (128, 3, 2), (64, 2, 3)])
def test_peak_gather_selection_checksum(d, splits, occ):
    say(f"[ix_peak_gather_selection] d={d} splits={splits} blocks_per_cu={occ}, ragged kv_len")
    g = torch.Generator().manual_seed(7 + d + splits)
    B, T, S, H_kv, k = 2, 37, 700, 2, 100
    kc = torch.randint(-2**15, 2**15 - 1, (B, S, H_kv, d), generator=g, dtype=torch.int16)
    vc = torch.randint(-2**15, 2**15 - 1, (B, S, H_kv, d), generator=g, dtype=torch.int16)
    idx = torch.randint(-3, S, (B, T, k), generator=g, dtype=torch.int32)
    kvl = torch.tensor([S, 450], dtype=torch.int32)
    out = torch.zeros(B * T * H_kv * splits, dtype=torch.int32, device=DEV)
    dev = [x.to(DEV) for x in (kc, vc, idx, kvl)]
    pk.ix_peak_gather_selection(dev[0].data_ptr(), dev[1].data_ptr(), dev[2].data_ptr(),
                                dev[3].data_ptr(), B, T, S, H_kv, d, k, splits, occ, out.data_ptr(),
                                torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    # XOR of each valid entry's K and V rows (per KV head), counted once per entry
    want = np.uint32(0)
    K = kc.numpy().view(np.uint16).astype(np.uint32)
    V = vc.numpy().view(np.uint16).astype(np.uint32)
    for b in range(B):
        rows = idx[b].numpy().reshape(-1)
        rows = rows[(rows >= 0) & (rows < int(kvl[b]))]
        cnt = np.bincount(rows, minlength=S) % 2
        for h in range(H_kv):
            kw = (K[b, :, h, 0::2] | (K[b, :, h, 1::2] << 16)).astype(np.uint32)
            vw = (V[b, :, h, 0::2] | (V[b, :, h, 1::2] << 16)).astype(np.uint32)
            rx = np.bitwise_xor.reduce(kw, axis=1) ^ np.bitwise_xor.reduce(vw, axis=1)
            want ^= np.bitwise_xor.reduce(np.where(cnt == 1, rx, 0).astype(np.uint32))
    assert int(np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))) == int(want)
