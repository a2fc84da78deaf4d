"""The HBM probes move the data they claim to (needs a gfx950 GPU): the copy reproduces its
input bit for bit, the two-input probes write the XOR of their inputs (and the second input),
the write probe its pattern, and the read probe leaves its sink alone; sizes that end inside a
tile and every access shape and grid are covered."""
import pytest
import torch

from deep_learning_normalization_amd import probes

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 16 * 1000 + 16 * 3, (8 << 20) + 16 * 37])
@pytest.mark.parametrize("unroll,nt,grid", [(1, 0, 0), (2, 1, 0), (4, 0, 64), (8, 1, 3)])
def test_probe_moves_its_streams(nbytes, unroll, nt, grid):
    print("[gpu] probe %d bytes unroll %d nt %d grid %d" % (nbytes, unroll, nt, grid), flush=True)
    n = nbytes // 4
    g = torch.Generator(device="cuda").manual_seed(nbytes + unroll)
    a = torch.randint(-2 ** 31, 2 ** 31 - 1, (n,), dtype=torch.int32, device="cuda", generator=g)
    b = torch.randint(-2 ** 31, 2 ** 31 - 1, (n,), dtype=torch.int32, device="cuda", generator=g)
    guard = 64
    c = torch.full((n + guard,), 7, dtype=torch.int32, device="cuda")
    d = torch.full((n + guard,), 9, dtype=torch.int32, device="cuda")
    probes.probe(1, 1, [a], [c], nbytes, unroll, nt, grid)
    torch.cuda.synchronize()
    assert torch.equal(c[:n], a) and (c[n:] == 7).all()
    probes.probe(2, 1, [a, b], [c], nbytes, unroll, nt, grid)
    torch.cuda.synchronize()
    assert torch.equal(c[:n], a ^ b)
    probes.probe(2, 2, [a, b], [c, d], nbytes, unroll, nt, grid)
    torch.cuda.synchronize()
    assert torch.equal(c[:n], a ^ b) and torch.equal(d[:n], b) and (d[n:] == 9).all()
    key = 0x12345
    probes.probe(0, 1, [], [c], nbytes, unroll, nt, grid, key=key)
    torch.cuda.synchronize()
    v = c[:n].view(-1, 4)
    assert (v[:, 0] == key).all() and (v[:, 2] == key).all()
    assert torch.equal(v[:, 1], torch.arange(n // 4, device="cuda", dtype=torch.int32))
    # the read probe writes its sink only where a thread's XOR of what it read equals the key:
    # over zeros every thread's XOR is 0
    z = torch.zeros(n, dtype=torch.int32, device="cuda")
    sink = torch.full((4,), 5, dtype=torch.int32, device="cuda")
    probes.probe(1, 0, [z], [sink], nbytes, unroll, nt, grid, key=1)
    torch.cuda.synchronize()
    assert (sink == 5).all()
    probes.probe(1, 0, [z], [sink], nbytes, unroll, nt, grid, key=0)
    torch.cuda.synchronize()
    assert (sink == 0).all()


def test_ceilings_report_every_mix():
    print("[gpu] ceilings", flush=True)
    c = probes.ceilings(stream_bytes=64 << 20, pool=8, iters=3,
                        variants=[(4, 0, 0), (8, 1, 0)])
    assert set(c) == set(probes.MIXES)
    for name, e in c.items():
        nin, nout = probes.MIXES[name]
        assert e["streams"] == "%dR%dW" % (nin, nout)
        assert 100.0 < e["GBps"] < 8000.0 * 1.05, (name, e)


def _mfma_expected(shape, nt, iters):
    """What every thread of the matrix-core probe stores, from the operand layouts: lane l of a
    wavefront supplies row l % R of A and column l % R of B with the 8 values of k at
    8 * (l // R) (R = 32 or 16), and holds the outputs of column l % R; for 32 x 32 blocks the
    rows 8 * (j // 4) + 4 * (l // 32) + j % 4 of registers j, for 16 x 16 blocks the rows
    4 * (l // 16) + j. Small integers keep every sum exact in fp32."""
    import numpy as np
    R, KB = (32, 16) if shape == 32 else (16, 32)
    out = np.zeros(nt)
    for w in range(nt // 64):
        t = np.arange(64) + 64 * w
        i = np.arange(8)
        a = ((t[:, None] + i[None, :]) & 15).astype(np.float64)
        b = ((t[:, None] ^ i[None, :]) & 15).astype(np.float64)
        A = np.zeros((R, KB))
        B = np.zeros((KB, R))
        for l in range(64):
            A[l % R, 8 * (l // R):8 * (l // R) + 8] = a[l]
            B[8 * (l // R):8 * (l // R) + 8, l % R] = b[l]
        D = A @ B
        for l in range(64):
            if shape == 32:
                rows = [8 * (j // 4) + 4 * (l // 32) + j % 4 for j in range(16)]
            else:
                rows = [4 * (l // 16) + j for j in range(4)]
            out[64 * w + l] = 8 * iters * D[rows, l % R].sum()
    return out


@pytest.mark.parametrize("shape,waves", [(32, 1), (32, 2), (16, 1), (16, 2)])
def test_mfma_probe_computes_what_it_claims(shape, waves):
    print("[gpu] mfma probe %d waves %d" % (shape, waves), flush=True)
    import numpy as np
    nt = 256 * waves
    grid, iters = 3, 5
    out = torch.full((grid * nt + 64,), -1.0, device="cuda")
    assert probes.lib().mfma_probe(shape, waves, grid, iters, out.data_ptr(), None, None,
                                   None) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = _mfma_expected(shape, nt, iters)
    for g in range(grid):
        assert np.array_equal(got[g * nt:(g + 1) * nt], want), (shape, waves, g)
    assert (got[grid * nt:] == -1.0).all()


def test_mfma_ceiling_is_plausible():
    print("[gpu] mfma ceiling", flush=True)
    c = probes.mfma_ceiling(iters=512, launches=4)
    for k in ("32x32x16", "16x16x32"):
        assert 100.0 < c[k]["TFLOPs"] <= 2500.0, c


@pytest.mark.parametrize("waves", [1, 2, 4])
def test_lds_probe_reads_what_it_claims(waves):
    """Every thread's XOR of its reads, recomputed on the host from the fill pattern and the
    read schedule."""
    print("[gpu] lds probe %d waves" % waves, flush=True)
    import numpy as np
    nt, grid, iters = 256 * waves, 2, 3
    out = torch.zeros(grid * nt, dtype=torch.int32, device="cuda")
    assert probes.lib().lds_probe(waves, grid, iters, out.data_ptr(), None, None, None) == 0
    torch.cuda.synchronize()
    words = (np.arange(16384, dtype=np.uint64) * 2654435761) & 0xFFFFFFFF
    want = np.zeros(nt, dtype=np.uint64)
    for t in range(nt):
        lane, wave = t & 63, t >> 6
        acc, base = 0, (wave * 1024) & 65535
        for _ in range(iters):
            for u in range(8):
                off = (base + u * 1024 + lane * 16) & 65520
                for k in range(4):
                    acc ^= int(words[off // 4 + k])
            base = (base + 8192) & 65535
        want[t] = acc
    got = out.cpu().numpy().view(np.uint32).astype(np.uint64)
    for g in range(grid):
        assert np.array_equal(got[g * nt:(g + 1) * nt], want), (waves, g)


def test_lds_read_rate_is_plausible():
    print("[gpu] lds read rate", flush=True)
    r = probes.lds_read_rate(iters=512, launches=4)
    for v in r.values():
        assert 10.0 < v["bytes_per_clk_per_cu"] < 1024.0, r
