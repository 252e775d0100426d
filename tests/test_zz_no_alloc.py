"""leyline_splice_noalloc, the splice that allocates no device memory (its
plan space is the library's static device array), against leyline_splice
through the C ABI: two pools built from the same seeded rows and tables, the
same batches applied to each, every byte of every layer, the page tables and
the books compared -- two calls in a row, the second smaller than the first
(the array keeps the first call's plan, which the second overwrites in
part).  Batches outside its limits are refused with nothing changed."""

import ctypes

import numpy as np
import pytest

from synth import permuted_pages, random_rows_np

from gpu_common import need_gpu, say, torch

pytestmark = pytest.mark.gpu


def _pools(L, layers, pages, P, seqs, gqa=False):
    """Two pools with identical contents: (pool, data, table) each."""
    out = []
    for _ in range(2):
        if gqa:
            H, D = 4, 64
            k = torch.from_numpy(random_rows_np(3, (layers, pages, P, H * D)).view(np.int16)).view(torch.bfloat16)
            v = torch.from_numpy(random_rows_np(4, (layers, pages, P, H * D)).view(np.int16)).view(torch.bfloat16)
            k, v = k.reshape(layers, pages, P, H, D).cuda(), v.reshape(layers, pages, P, H, D).cuda()
            table = torch.full((seqs, pages), -1, dtype=torch.int32, device="cuda")
            pool = L.GqaPool(k, v, table, rotary_dim=32, pairing=L.ROPE_HALF)
            out.append((pool, (k, v), table))
        else:
            data = torch.from_numpy(random_rows_np(3, (layers, pages, P, 576)).view(np.int16)).view(torch.bfloat16).cuda()
            table = torch.full((seqs, pages), -1, dtype=torch.int32, device="cuda")
            out.append((L.Pool(data, table), (data,), table))
    return out


def _same(a, b, seqs):
    (pa, da, ta), (pb, db, tb) = a, b
    torch.cuda.synchronize()
    for x, y in zip(da, db):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16)), "rows differ"
    assert torch.equal(ta, tb), "device page tables differ"
    for s in seqs:
        ga, gb = pa.seq_get(s), pb.seq_get(s)
        assert ga[0] == gb[0] and ga[1] == gb[1] and np.array_equal(ga[2], gb[2])
    assert pa.free_pages() == pb.free_pages()
    sa, sb = pa.last_stats(), pb.last_stats()
    assert (sa.alg_bytes, sa.rows_moved, sa.rows_rotated_inplace, sa.fresh_pages) == \
           (sb.alg_bytes, sb.rows_moved, sb.rows_rotated_inplace, sb.fresh_pages)
    assert sb.planned_on_device == 1


@pytest.mark.parametrize("gqa", [False, True])
def test_noalloc_splice_matches_splice_twice_in_a_row(gqa):
    L = need_gpu()
    say(f"no-alloc splice vs splice, gqa={gqa}")
    layers, pages, P = 3, 2000, 16
    a, b = _pools(L, layers, pages, P, 3, gqa)
    perm = permuted_pages(8, pages)
    lens = (9000, 5000, 3000)
    off = 0
    for s, n in enumerate(lens):
        k = -(-n // P)
        for pool, _, _ in (a, b):
            pool.seq_set_pages(s, perm[off:off + k], n)
        off += k
    torch.cuda.synchronize()

    def stub(r, seed):
        if gqa:
            k = torch.from_numpy(random_rows_np(seed, (layers, r, 4, 64)).view(np.int16)).view(torch.bfloat16).cuda()
            v = torch.from_numpy(random_rows_np(seed + 1, (layers, r, 4, 64)).view(np.int16)).view(torch.bfloat16).cuda()
            return k, v
        return torch.from_numpy(random_rows_np(seed, (layers, r, 576)).view(np.int16)).view(torch.bfloat16).cuda(), None

    # call 1: three directives -- fresh pages with a stub, a whole-page shift
    # turned in place, and a FORGET
    k1, v1 = stub(21, 50)
    first = [L.Directive(0, 1000, 4003, k1, stub_v=v1), L.Directive(1, 512, 1536, None),
             L.Directive(2, 700, 900, None, mode=L.FORGET)]
    a[0].splice(first)
    b[0].splice(first, noalloc=True)
    _same(a, b, range(3))
    st = b[0].last_stats()
    assert st.fresh_pages > 0 and st.rows_rotated_inplace > 0
    # call 2: one smaller directive
    k2, v2 = stub(3, 60)
    second = [L.Directive(1, 100, 120, k2, stub_v=v2)]
    a[0].splice(second)
    b[0].splice(second, noalloc=True)
    _same(a, b, range(3))
    assert b[0].last_stats().fresh_pages < st.fresh_pages
    for pool, _, _ in (a, b):
        pool.close()


def test_noalloc_splice_refuses_what_it_cannot_plan_and_changes_nothing():
    L = need_gpu()
    say("no-alloc splice limits")
    layers, P, pages = 1, 1, 80000
    (pool, (data,), table), _ = _pools(L, layers, 2 * pages, P, 20)
    # 20 sequences: a batch of 17 directives is beyond the device planner
    for s in range(20):
        pool.seq_set_pages(s, np.arange(s * 64, s * 64 + 64), 64)
    dirs = [L.Directive(s, 10, 20, None) for s in range(17)]
    before = table.clone()
    with pytest.raises(L.LeylineError) as ei:
        pool.splice(dirs, noalloc=True)
    assert ei.value.status == L.LL_EUNSUPPORTED and "device" in str(ei.value)
    # a plan beyond the 4 MiB array: at page size 1, two stub rows in front of
    # 66001 rows make 66001 in-place tasks plus 2 fresh pages, 64 bytes each
    pool.seq_free(19)
    pool.seq_set_pages(19, np.arange(3000, 3000 + 66001), 66001)
    big = torch.from_numpy(random_rows_np(5, (layers, 2, 576)).view(np.int16)).view(torch.bfloat16).cuda()
    with pytest.raises(L.LeylineError) as ei:
        pool.splice([L.Directive(19, 0, 0, big)], noalloc=True)
    assert ei.value.status == L.LL_EUNSUPPORTED and "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.equal(table[:19], before[:19])
    assert pool.seq_get(19)[0] == 66001 and pool.seq_get(0)[0] == 64
    # the same batch through leyline_splice still works
    pool.splice([L.Directive(19, 0, 0, big)])
    torch.cuda.synchronize()
    assert pool.seq_get(19)[0] == 66003
    pool.close()
