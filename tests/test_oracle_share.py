"""Pins for the oracle's two-stage row share and staging layout (CPU only).

Source: Modular Mojo API docs, "allreduce_rmsnorm_fp8" (2-stage path: each
GPU owns ceildiv(rows, ngpus) rows and stages their fp8 data and scales, the
scales padded to the SIMD width).
"""
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "p1_stage_bytes.txt")


def golden_rows():
    out = []
    for line in open(GOLDEN):
        if line.strip() and not line.startswith("#"):
            out.append([int(v) for v in line.split()])
    return out


def test_stage_bytes_golden(orc):
    for rows, cols, ngpus, simd, share, want in golden_rows():
        assert orc.stage_bytes(rows, cols, ngpus, simd) == want, (rows, cols, ngpus, simd)
        assert max(orc.share_rows(rows, ngpus, k)[1] for k in range(ngpus)) == share


@pytest.mark.parametrize("rows", [0, 1, 5, 7, 8, 33, 64, 100, 8192])
@pytest.mark.parametrize("ngpus", [1, 2, 3, 4, 7, 8])
def test_shares_partition_the_rows(orc, rows, ngpus):
    """Brute force: row i belongs to rank i // ceil(rows / ngpus); the shares
    are contiguous, disjoint and cover every row once."""
    S = -(-rows // ngpus) if rows else 0
    owner = [i // S for i in range(rows)] if S else []
    covered = []
    for k in range(ngpus):
        first, count = orc.share_rows(rows, ngpus, k)
        assert 0 <= count <= S
        mine = [i for i in range(rows) if owner[i] == k]
        assert list(range(first, first + count)) == mine
        covered += mine
    assert covered == list(range(rows))


def test_stage_share_layout(orc):
    rng = np.random.default_rng(40)
    rows, cols, ngpus = 11, 24, 4
    q = rng.integers(0, 256, size=(rows, cols), dtype=np.uint8)
    s = rng.standard_normal(rows).astype(np.float32)
    S = 3
    for k in range(ngpus):
        slot = orc.stage_share(q, s, ngpus, k, fill=0xA5)
        assert slot.size == S * cols + 16
        first, count = orc.share_rows(rows, ngpus, k)
        data = slot[: S * cols].reshape(S, cols)
        assert np.array_equal(data[:count], q[first:first + count])
        assert np.all(data[count:] == 0xA5)
        sc = slot[S * cols: S * cols + 4 * S].view(np.float32)
        assert np.array_equal(sc[:count], s[first:first + count])
        assert np.all(slot[S * cols + 4 * count:] == 0xA5)


def test_single_rank_slot_is_the_full_output(orc):
    rng = np.random.default_rng(41)
    q = rng.integers(0, 256, size=(4, 16), dtype=np.uint8)
    s = rng.standard_normal(4).astype(np.float32)
    slot = orc.stage_share(q, s, 1, 0)
    assert np.array_equal(slot[:64], q.reshape(-1))
    assert np.array_equal(slot[64:80].view(np.float32), s)
