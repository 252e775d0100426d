"""Helpers for the GPU parity tests: build a pool on the device from seeded
inputs, mirror it into an oracle CacheState, and compare the library's result
with the oracle's (page tables and lengths bit-exact, c_kv and stub rows
bit-exact, rotated k_pe within 1 bf16 ulp)."""

from __future__ import annotations

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import leyline_oracle as O  # noqa: E402
from synth import random_rows_np, random_rows_torch  # noqa: E402

KV = O.KV_LORA_RANK


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mla_paged_cache_amd import leyline  # noqa: F401  (fails loudly if the library is missing)
    return leyline


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


class DevicePool:
    """A pool on cuda:0 plus its host mirror for the oracle."""

    def __init__(self, L, num_pages, P, max_seqs, max_pages, seed=0, host_rows=True, pairing=0, oracle_layers=None):
        leyline = need_gpu()
        self.L, self.num_pages, self.P = L, num_pages, P
        shape = (L, num_pages, P, O.ROW)
        if host_rows:
            rows = random_rows_np(seed, shape)
            self.data = torch.from_numpy(rows.view(np.int16)).view(torch.bfloat16).to("cuda")
        else:
            self.data = random_rows_torch(seed, shape, "cuda")
        self.table = torch.full((max_seqs, max_pages), -1, dtype=torch.int32, device="cuda")
        self.pool = leyline.Pool(self.data, self.table, pairing=pairing)
        self.oracle_layers = list(range(L)) if oracle_layers is None else list(oracle_layers)
        self.state = O.CacheState.empty(len(self.oracle_layers), num_pages, P, max_pages, with_rows=False)

    def snapshot_rows(self):
        """Copy the checked layers to the host into the oracle state."""
        self.state.layers = [self.data[L].view(torch.int16).cpu().numpy().view(np.uint16).copy()
                             for L in self.oracle_layers]

    def set_pages(self, seq, pages, n):
        self.pool.seq_set_pages(seq, pages, n)
        self.state.set_pages(seq, pages, n)

    def stub(self, seed, r_len):
        """Stub rows [L][r_len][576] on the device and on the host."""
        if r_len == 0:
            return None, None
        rows = random_rows_np(seed, (self.L, r_len, O.ROW))
        dev = torch.from_numpy(rows.view(np.int16)).view(torch.bfloat16).to("cuda")
        return dev, rows[self.oracle_layers]

    def close(self):
        self.pool.close()
        del self.data, self.table
        torch.cuda.empty_cache()


def ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in bf16 steps between bit patterns (sign-magnitude ordered;
    +0 and -0 are equal)."""
    def key(x):
        x = x.astype(np.int32)
        mag = x & 0x7FFF
        return np.where(x & 0x8000, -mag, mag)
    return np.abs(key(a) - key(b))


def compare_seq(dp: DevicePool, expected: O.CacheState, seq: int, max_ulp: int = 1):
    """Library state of `seq` against the oracle's: length, next position,
    page table (host copy and device row), and every live row of the checked
    layers.  Returns the largest k_pe ulp distance seen."""
    n, pos, pages = dp.pool.seq_get(seq)
    assert n == expected.lengths[seq], (n, expected.lengths[seq])
    assert pos == expected.next_pos[seq]
    assert list(pages) == list(expected.tables[seq])
    dev_row = dp.table[seq, :len(pages)].cpu().numpy()
    assert np.array_equal(dev_row, pages)
    worst = 0
    if n == 0:
        return worst
    P = dp.P
    j = np.arange(n)
    phys = torch.from_numpy((pages.astype(np.int64)[j // P] * P + j % P)).to("cuda")
    for li, L in enumerate(dp.oracle_layers):
        got = dp.data[L].view(-1, O.ROW)[phys].view(torch.int16).cpu().numpy().view(np.uint16)
        exp = expected.logical_rows(seq, li)
        assert np.array_equal(got[:, :KV], exp[:, :KV]), f"c_kv differs (layer {L})"
        d = ulp_distance(got[:, KV:], exp[:, KV:])
        worst = max(worst, int(d.max()))
        assert worst <= max_ulp, f"k_pe differs by {worst} ulp (layer {L})"
    return worst


def assert_same_free(dp: DevicePool, expected: O.CacheState):
    assert dp.pool.free_pages() == len(expected.free)
