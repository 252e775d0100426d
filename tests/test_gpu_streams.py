"""Calls on one pool from different streams.  Each call's device work follows
the previous call's on the same pool, whichever stream either ran on (the
ordering rule of the C ABI), so successive splices ("Leyline", sections
2.1-2.3) and evictions ("KV-streams", "how it works"), each issued on another
stream, must give exactly the oracle's sequential result; so must a per-row
gather read on a third stream afterwards."""

import numpy as np
import pytest

from oracle import leyline_oracle as O
from synth import permuted_pages

from gpu_common import DevicePool, assert_same_free, compare_seq, need_gpu, say, torch, ulp_distance

pytestmark = pytest.mark.gpu


def test_splices_and_evictions_on_alternating_streams():
    L = need_gpu()
    say("calls on alternating streams")
    dp = DevicePool(2, 800, 16, 3, 200, seed=61)
    perm = permuted_pages(61, 800)
    dp.set_pages(0, perm[:150], 2390)
    dp.set_pages(1, perm[150:260], 1751)
    dp.set_pages(2, perm[260:300], 633)
    dp.snapshot_rows()
    state = dp.state
    cur = torch.cuda.current_stream()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    order = [s1, s2, cur, s1, s2, s2, cur, s1, s2]
    rng = np.random.default_rng(61)
    keep_alive = []   # inputs stay allocated until the device is done with them
    for k, st in enumerate(order):
        if k % 3 == 2:
            seqs = [1, 2]
            masks = [(rng.random(state.lengths[s]) < 0.7).astype(np.uint8) for s in seqs]
            state, _ = O.evict(state, seqs, masks)
            keep = torch.from_numpy(np.concatenate(masks)).to("cuda")
            offsets = np.array([0, len(masks[0])], np.int64)
            keep_alive.append(keep)
            st.wait_stream(cur)      # the mask upload ran on the current stream
            dp.pool.evict(seqs, keep, offsets, stream=st)
        else:
            lib_dirs, ora_dirs = [], []
            for s in (0, 2):
                n = state.lengths[s]
                s0 = int(rng.integers(0, n + 1))
                s1_ = int(rng.integers(s0, n + 1))
                r = int(rng.integers(0, 20))
                dev, host = dp.stub(1000 * k + s, r)
                keep_alive.append(dev)
                lib_dirs.append(L.Directive(s, s0, s1_, dev))
                ora_dirs.append(O.Directive(s, s0, s1_, r, host))
            state, _ = O.splice(state, ora_dirs)
            st.wait_stream(cur)
            dp.pool.splice(lib_dirs, stream=st)
    n0 = state.lengths[0]
    angles = np.random.default_rng(62).integers(-5000, 5000, size=n0).astype(np.int64)
    ang = torch.from_numpy(angles).to("cuda")
    s2.wait_stream(cur)
    out = dp.pool.rope_rows(0, 0, ang, out=True, stream=s2)
    torch.cuda.synchronize()
    for s in range(3):
        compare_seq(dp, state, s)
    assert_same_free(dp, state)
    exp = O.rope_rows(state, 0, 0, angles)
    for li in range(2):
        got = out[li].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got[:, :512], exp[li][:, :512])
        assert ulp_distance(got[:, 512:], exp[li][:, 512:]).max() <= 1
    del keep_alive
    dp.close()
