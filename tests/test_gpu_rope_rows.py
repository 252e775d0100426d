"""GPU parity of ll_rope_rows, the per-row-angle RoPE rotation (each row turned
by its own angle steps, e.g. back by its position before VECTOR's K -> V
reconstruction; "VECTOR", gist.science summary, method), against the CPU
oracle through the C ABI.

Non-band values bit-exact, bands within 1 bf16 ulp (the float64 cos/sin come
from the device's math library on one side and the host's libm on the other;
they agree after float32 rounding except at rounding ties one float64 ulp
wide, so 0 is expected and the count of differing values is reported)."""

import numpy as np
import pytest

from oracle import leyline_oracle as O
from synth import np_rng, permuted_pages, random_normal_np, random_rows_np

from gpu_common import DevicePool, need_gpu, say, torch, ulp_distance
from test_gpu_gqa import GqaDevicePool

pytestmark = pytest.mark.gpu


def _angles(seed, n, big=False):
    rng = np_rng(seed, 0)
    a = rng.integers(-200000, 200000, size=n)
    if big:
        big_values = [2 ** 31 - 1, -(2 ** 31), 10 ** 9 + 7, -987654321]
        a[:min(4, n)] = big_values[:min(4, n)]
    return a.astype(np.int64)


def _cmp_rows(got, exp, bands, width):
    """got/exp uint16 [n, width]; bands: list of (off, dim).  Returns the
    number of band values 1 ulp apart; asserts everything else."""
    mask = np.zeros(width, bool)
    for off, dim in bands:
        mask[off:off + dim] = True
    assert np.array_equal(got[:, ~mask], exp[:, ~mask])
    d = ulp_distance(got[:, mask], exp[:, mask])
    assert d.max(initial=0) <= 1
    return int(np.count_nonzero(d))


@pytest.mark.parametrize("P,pairing", [(1, 0), (8, 1), (16, 0), (16, 1), (32, 0)])
def test_mla_gather_and_in_place(P, pairing):
    L = need_gpu()
    say(f"rope rows MLA P={P} pairing={pairing}")
    n_tok = 900
    pages = -(-n_tok // P)
    dp = DevicePool(2, 2 * pages, P, 1, 2 * pages, seed=3, pairing=pairing)
    dp.set_pages(0, permuted_pages(3, 2 * pages)[:pages], n_tok)
    dp.snapshot_rows()
    pname = "half" if pairing else "interleaved"
    flips = 0
    for (r0, n, big) in ((0, 1, True), (17, 500, True), (n_tok - 333, 333, False)):
        a = _angles(r0 + n, n, big)
        ad = torch.from_numpy(a).cuda()
        out = dp.pool.rope_rows(0, r0, ad, out=True)
        torch.cuda.synchronize()
        exp = O.rope_rows(dp.state, 0, r0, a, pairing=pname)
        for li in range(2):
            got = out[li].view(torch.int16).cpu().numpy().view(np.uint16)
            flips += _cmp_rows(got, exp[li], [(512, 64)], O.ROW)
        st = dp.pool.last_stats()
        assert st.alg_bytes == 2 * n * 2 * 1152
    # in place: the pool's rows change, nothing else
    a = _angles(7, 600)
    dp.pool.rope_rows(0, 100, torch.from_numpy(a).cuda())
    torch.cuda.synchronize()
    new = O.rope_rows(dp.state, 0, 100, a, pairing=pname, in_place=True)
    for li in range(2):
        flat = dp.data[li].view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1, O.ROW)
        exp_flat = new.layers[li].reshape(-1, O.ROW)
        flips += _cmp_rows(flat, exp_flat, [(512, 64)], O.ROW)
    say(f"  band values 1 ulp apart: {flips}")
    dp.close()


@pytest.mark.parametrize("H,D,rot,pairing", [(2, 64, 64, 0), (4, 128, 64, 1), (8, 128, 128, 1), (3, 64, 32, 0)])
def test_gqa_gather_and_in_place(H, D, rot, pairing):
    need_gpu()
    say(f"rope rows GQA H={H} D={D} rot={rot} pairing={pairing}")
    P, n_tok = 16, 700
    pages = -(-n_tok // P)
    dp = GqaDevicePool(2, 2 * pages, P, 1, 2 * pages, H, D, rot, seed=5, pairing=pairing)
    dp.set_pages(0, permuted_pages(5, 2 * pages)[:pages], n_tok)
    dp.snapshot_rows()
    bands = [(h * D, rot) for h in range(H)]
    a = _angles(11, 400, big=True)
    out = dp.pool.rope_rows(0, 123, torch.from_numpy(a).cuda(), out=True)
    torch.cuda.synchronize()
    exp = O.rope_rows(dp.state, 0, 123, a, pairing=dp.pairing)
    flips = 0
    for li in range(2):
        got = out[li].reshape(400, H * D).view(torch.int16).cpu().numpy().view(np.uint16)
        flips += _cmp_rows(got, exp[li], bands, H * D)
    v_before = dp.v.clone()
    dp.pool.rope_rows(0, 0, torch.from_numpy(a).cuda())
    torch.cuda.synchronize()
    assert torch.equal(dp.v, v_before)
    new = O.rope_rows(dp.state, 0, 0, a, pairing=dp.pairing, in_place=True)
    for li in range(2):
        flat = dp.k[li].reshape(-1, H * D).view(torch.int16).cpu().numpy().view(np.uint16)
        flips += _cmp_rows(flat, new.layers[2 * li].reshape(-1, H * D), bands, H * D)
    say(f"  band values 1 ulp apart: {flips}")
    dp.close()


@pytest.mark.slow
def test_mla_32k_27_layers_back_to_position_free_keys():
    """Every row of a 32768-token, 27-layer MLA cache holds
    k_pe = bf16(RoPE(p) k) at its position p; gathering all of them with
    angles -p gives the position-free keys within two bf16 roundings, and
    layers 0 and 26 match the oracle."""
    L = need_gpu()
    say("rope rows 32k x 27 back-rotation")
    P, n_tok, layers = 16, 32768, 27
    pages = n_tok // P
    dp = DevicePool(layers, pages + 64, P, 1, pages, seed=1, host_rows=False, oracle_layers=[0, 26])
    T = permuted_pages(1, pages + 64)[:pages]
    dp.set_pages(0, T, n_tok)
    pos = np.arange(n_tok)
    phys = torch.from_numpy(T.astype(np.int64)[pos // P] * P + pos % P).cuda()
    k_raw = {}
    for l in (0, 26):
        k = random_normal_np(40 + l, (n_tok, 64))
        k_raw[l] = k
        kpe = O.f32_to_bf16(O.rotate_f64(k, pos).astype(np.float32))
        flat = dp.data[l].view(torch.int16).view(-1, O.ROW)
        flat[phys, 512:] = torch.from_numpy(kpe.view(np.int16)).cuda()
    torch.cuda.synchronize()
    dp.snapshot_rows()
    a = -pos.astype(np.int64)
    out = dp.pool.rope_rows(0, 0, torch.from_numpy(a).cuda(), out=True)
    torch.cuda.synchronize()
    exp = O.rope_rows(dp.state, 0, 0, a)
    flips = 0
    for li, l in enumerate((0, 26)):
        got = out[l].view(torch.int16).cpu().numpy().view(np.uint16)
        flips += _cmp_rows(got, exp[li], [(512, 64)], O.ROW)
        back = O.bf16_to_f32(got[:, 512:]).astype(np.float64)
        rel = np.linalg.norm(back - k_raw[l]) / np.linalg.norm(k_raw[l])
        say(f"  layer {l}: relative L2 to the position-free keys {rel:.3e}")
        assert rel < 4e-3
    st = dp.pool.last_stats()
    assert st.alg_bytes == layers * n_tok * 2 * 1152
    # the same turn in place: every layer's bands change (the one-kernel
    # in-place path, three batches of nine layers), layers 0 and 26 compared
    dp.pool.rope_rows(0, 0, torch.from_numpy(a).cuda())
    torch.cuda.synchronize()
    assert dp.pool.last_stats().alg_bytes == layers * n_tok * 2 * 128
    new = O.rope_rows(dp.state, 0, 0, a, in_place=True)
    for li, l in enumerate((0, 26)):
        got = dp.data[l].view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1, O.ROW)
        flips += _cmp_rows(got, new.layers[li].reshape(-1, O.ROW), [(512, 64)], O.ROW)
    say(f"  band values 1 ulp apart: {flips}")
    dp.close()


@pytest.mark.parametrize("pairing", [0, 1])
def test_mla_in_place_layers_in_separate_allocations(pairing):
    """Layers that are not one allocation (no common stride): the in-place
    kernel reads each layer's base from the pool's pointer array."""
    L = need_gpu()
    say(f"rope rows MLA in place, separate layer tensors, pairing={pairing}")
    P, n_tok, layers = 16, 777, 10
    pages = -(-n_tok // P)
    host = random_rows_np(21, (layers, 2 * pages, P, O.ROW))
    tensors = []
    for l in (3, 0, 7, 1, 9, 2, 8, 4, 6, 5):   # allocated out of order: no single stride
        tensors.append((l, torch.from_numpy(host[l].view(np.int16)).view(torch.bfloat16).cuda()))
    data = [t for _, t in sorted(tensors, key=lambda x: x[0])]
    table = torch.full((1, 2 * pages), -1, dtype=torch.int32, device="cuda")
    pool = L.Pool(data, table, pairing=pairing)
    T = permuted_pages(21, 2 * pages)[:pages]
    pool.seq_set_pages(0, T, n_tok)
    st = O.CacheState.empty(layers, 2 * pages, P, 2 * pages, with_rows=False)
    st.layers = [host[l].copy() for l in range(layers)]
    st.set_pages(0, T, n_tok)
    a = _angles(17, 500, big=True)
    pool.rope_rows(0, 111, torch.from_numpy(a).cuda())
    torch.cuda.synchronize()
    new = O.rope_rows(st, 0, 111, a, pairing="half" if pairing else "interleaved", in_place=True)
    flips = 0
    for l in range(layers):
        flat = data[l].view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1, O.ROW)
        flips += _cmp_rows(flat, new.layers[l].reshape(-1, O.ROW), [(512, 64)], O.ROW)
    say(f"  band values 1 ulp apart: {flips}")
    pool.close()


@pytest.mark.parametrize("P,pairing", [(4, 0), (4, 1), (16, 1)])
def test_mla_in_place_eleven_layers(P, pairing):
    """In place over 11 layers (one batch of nine layers and a partial one),
    rows starting off an 8-row boundary and ending in a partial group."""
    need_gpu()
    say(f"rope rows MLA in place, 11 layers, P={P} pairing={pairing}")
    n_tok = 1000
    pages = -(-n_tok // P)
    dp = DevicePool(11, 2 * pages, P, 1, 2 * pages, seed=9, pairing=pairing)
    dp.set_pages(0, permuted_pages(9, 2 * pages)[:pages], n_tok)
    dp.snapshot_rows()
    a = _angles(13, 741, big=True)
    dp.pool.rope_rows(0, 203, torch.from_numpy(a).cuda())
    torch.cuda.synchronize()
    new = O.rope_rows(dp.state, 0, 203, a, pairing="half" if pairing else "interleaved", in_place=True)
    flips = 0
    for li in range(11):
        flat = dp.data[li].view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1, O.ROW)
        flips += _cmp_rows(flat, new.layers[li].reshape(-1, O.ROW), [(512, 64)], O.ROW)
    say(f"  band values 1 ulp apart: {flips}")
    dp.close()


def test_errors():
    L = need_gpu()
    dp = DevicePool(1, 16, 16, 1, 16, seed=2)
    dp.set_pages(0, list(range(4)), 60)
    a = torch.zeros(10, dtype=torch.int64, device="cuda")
    with pytest.raises(L.LeylineError):
        dp.pool.rope_rows(0, 55, a)            # rows 55..64 pass the end
    with pytest.raises(L.LeylineError):
        dp.pool.rope_rows(3, 0, a)             # unknown sequence
    assert L._lib.ll_rope_rows(dp.pool._h, 0, 0, 5, None, None, 0, None) == L.LL_EINVAL
    out = torch.empty((1, 10, O.ROW), dtype=torch.bfloat16, device="cuda")
    assert L._lib.ll_rope_rows(dp.pool._h, 0, 0, 10, a.data_ptr(), out.data_ptr() + 8, 0, None) == L.LL_EINVAL
    dp.close()
