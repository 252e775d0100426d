"""The binding rejects caller tensors of the wrong shape, dtype, layout or
device with ValueError before any pointer reaches the library (no GPU
needed: the checks run on host metadata; a pool or context object is made
without a device, so a call that got past its checks would fail in the
library with LL_EINVAL on the NULL handle instead)."""

import types

import numpy as np
import pytest
import torch

from mla_paged_cache_amd import leyline as L

CPU = torch.device("cpu")
NULL_STREAM = types.SimpleNamespace(cuda_stream=0)   # so no torch stream is looked up


def fake_pool(layers=2, gqa=False):
    p = object.__new__(L.GqaPool if gqa else L.Pool)
    p._h = None
    p.device = CPU
    p._dev = 0
    p.num_layers = layers
    if gqa:
        p.heads, p.head_dim = 2, 64
        p.row = 128
    return p


def fake_ctx():
    c = object.__new__(L.KvsMask)
    c._h = None
    c.device = 0
    c._tdev = CPU
    return c


def test_rope_rows_checks_angles_and_out():
    p = fake_pool()
    ang = torch.zeros(8, dtype=torch.int64)
    with pytest.raises(ValueError):
        p.rope_rows(0, 0, ang.to(torch.int32))
    with pytest.raises(ValueError):
        p.rope_rows(0, 0, torch.zeros(16, dtype=torch.int64)[::2])
    for bad in (torch.zeros((2, 7, L.ROW), dtype=torch.bfloat16),          # too few rows
                torch.zeros((1, 8, L.ROW), dtype=torch.bfloat16),          # too few layers
                torch.zeros((2, 8, L.ROW), dtype=torch.float16),           # wrong dtype
                torch.zeros((2, 8, 2 * L.ROW), dtype=torch.bfloat16)[:, :, :L.ROW]):  # rows not contiguous
        with pytest.raises(ValueError):
            p.rope_rows(0, 0, ang, out=bad)
    with pytest.raises(L.LeylineError):   # shapes fine: reaches the library, which refuses the NULL pool
        p.rope_rows(0, 0, ang, out=torch.zeros((2, 8, L.ROW), dtype=torch.bfloat16), stream=NULL_STREAM)
    g = fake_pool(gqa=True)
    with pytest.raises(ValueError):
        g.rope_rows(0, 0, ang, out=torch.zeros((2, 8, L.ROW), dtype=torch.bfloat16))


def test_evict_checks_keep_and_offsets():
    p = fake_pool()
    keep = np.ones(10, np.uint8)
    with pytest.raises(ValueError):
        p.evict([0], keep, [0])                                   # not a tensor
    with pytest.raises(ValueError):
        p.evict([0], torch.ones(10, dtype=torch.int32), [0])      # wrong dtype
    with pytest.raises(ValueError):
        p.evict([0, 1], torch.ones(10, dtype=torch.uint8), [0])   # one offset for two sequences
    with pytest.raises(L.LeylineError):   # the length query needs the pool: the NULL handle is refused
        p.evict([0], torch.ones(10, dtype=torch.uint8), [0])


def test_kvs_calls_check_their_tensors():
    c = fake_ctx()
    death = torch.zeros((2, 256), dtype=torch.int32)
    for bad in (torch.zeros((2, 256, 7), dtype=torch.int32),      # too few words per row
                torch.zeros((2, 256, 8), dtype=torch.int64),      # wrong dtype
                torch.zeros((1, 256, 8), dtype=torch.int32)):     # too few rollouts
        with pytest.raises(ValueError):
            c.dense_mask(death, out=bad)
    with pytest.raises(ValueError):
        c.dense_mask(death.to(torch.int64))
    with pytest.raises(ValueError):
        c.block_mask(death.t(), 128, 128)                          # not contiguous
    with pytest.raises(L.LeylineError):
        c.dense_mask(death, out=torch.zeros((2, 256, 8), dtype=torch.int32), stream=NULL_STREAM)
    logs = L._Logs(2, (L._KvsRolloutLog * 2)(), [], torch.zeros(1, dtype=torch.uint8))
    with pytest.raises(ValueError):
        c.death_times(logs, 256, out=(torch.zeros((2, 255), dtype=torch.int32), torch.zeros(2, dtype=torch.int32)))
    with pytest.raises(ValueError):
        c.death_times(logs, 256, out=(death, torch.zeros(3, dtype=torch.int32)))
