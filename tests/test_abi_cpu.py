"""Host-side checks of the C ABI that need no GPU: the built library loads and
exports every function include/leyline.h declares, the binding declares the
same set, descriptor validation fails before any device call, and the host's
float32 cos/sin table of the delta-rotation (Leyline summary, section 2.2) is
the oracle's."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "leyline.h")
LIB = os.path.join(ROOT, "mla_paged_cache_amd", "libleyline.so")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libleyline.so is not built: run __graft_entry__.build()")
    return ctypes.CDLL(LIB)


def test_header_declares_the_path_entry_points():
    names = _declared()
    for n in ("leyline_splice", "kv_evict_compact", "ll_ptable_reindex", "ll_pool_create", "ll_last_plan_bytes",
              "ll_rope_delta_table", "ll_last_error"):
        assert n in names
    assert len(names) == 29


# a page passage, or "no passage" for bookkeeping; the no-allocation splice
# names the callers it is for instead
CITATION = re.compile(r"\[Leyline\] section|\[KV-streams\] \"|VECTOR|no passage of the pages|"
                      r"callers that cannot allocate")


def test_every_declaration_cites_its_passage_or_says_it_has_none():
    """Each function declaration is preceded (after the previous declaration
    ends) by a comment that names the page section defining the operation,
    says that it is library bookkeeping with no passage behind it, or (the
    splice that allocates nothing) names the callers it is for.  Two
    declarations with nothing between them share the comment before the
    first."""
    text = open(HEADER).read()
    decl = re.compile(r"^(?:ll_status|void|const char\*)\s+\*?\s*([a-z_][a-z0-9_]*)\s*\(", re.M)
    prev_end, last_comment = 0, None
    checked = 0
    for m in decl.finditer(text):
        between = text[prev_end:m.start()]
        comments = re.findall(r"/\*.*?\*/", between, flags=re.S)
        if comments:
            last_comment = " ".join(comments)
        assert last_comment and CITATION.search(last_comment), m.group(1)
        prev_end = text.index(";", m.end()) + 1
        checked += 1
    assert checked == len(_declared())


def test_splice_planner_setter_checks_its_arguments():
    from mla_paged_cache_amd import leyline as L
    assert L._lib.ll_pool_set_splice_planner(None, L.SPLICE_PLAN_HOST) == L.LL_EINVAL
    assert "NULL" in L._lib.ll_last_error().decode()


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_binding_covers_the_header():
    from mla_paged_cache_amd import leyline
    assert sorted(leyline.EXPORTS) == _declared()


def test_pool_create_rejects_bad_descriptors_before_touching_a_device():
    from mla_paged_cache_amd import leyline as L
    ptrs = (ctypes.c_void_p * 2)(16, 32)
    base = dict(num_layers=2, page_size=16, num_pages=8, max_seqs=1, max_pages_per_seq=8,
                kv_lora_rank=512, rope_dim=64, rope_pairing=0, rope_base=10000.0,
                layer_base=ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p)), page_table=64, device=0)
    cases = [
        (dict(page_size=12), L.LL_EINVAL),
        (dict(page_size=512), L.LL_EINVAL),
        (dict(num_layers=0), L.LL_EINVAL),
        (dict(kv_lora_rank=128), L.LL_EUNSUPPORTED),
        (dict(rope_dim=32), L.LL_EUNSUPPORTED),
        (dict(rope_pairing=7), L.LL_EINVAL),
        (dict(rope_base=-1.0), L.LL_EINVAL),
        (dict(page_table=None), L.LL_EINVAL),
        (dict(device=-1), L.LL_EINVAL),
    ]
    for change, code in cases:
        d = L._PoolDesc(**{**base, **change})
        h = ctypes.c_void_p()
        assert L._lib.ll_pool_create(ctypes.byref(d), ctypes.byref(h)) == code, change
        assert not h.value
        assert L._lib.ll_last_error().decode()
    misaligned = (ctypes.c_void_p * 2)(16, 40)
    d = L._PoolDesc(**{**base, "layer_base": ctypes.cast(misaligned, ctypes.POINTER(ctypes.c_void_p))})
    assert L._lib.ll_pool_create(ctypes.byref(d), ctypes.byref(ctypes.c_void_p())) == L.LL_EINVAL


def test_gqa_pool_create_rejects_bad_descriptors_before_touching_a_device():
    from mla_paged_cache_amd import leyline as L
    kp = (ctypes.c_void_p * 2)(16, 32)
    vp = (ctypes.c_void_p * 2)(48, 64)
    base = dict(num_layers=2, page_size=16, num_pages=8, max_seqs=1, max_pages_per_seq=8,
                num_kv_heads=8, head_dim=128, rotary_dim=128, rope_pairing=1, rope_base=500000.0,
                k_layer_base=ctypes.cast(kp, ctypes.POINTER(ctypes.c_void_p)),
                v_layer_base=ctypes.cast(vp, ctypes.POINTER(ctypes.c_void_p)), page_table=64, device=0)
    cases = [
        (dict(page_size=3), L.LL_EINVAL),
        (dict(num_kv_heads=0), L.LL_EUNSUPPORTED),
        (dict(head_dim=100), L.LL_EUNSUPPORTED),
        (dict(rotary_dim=96), L.LL_EUNSUPPORTED),        # not a power of two
        (dict(rotary_dim=8), L.LL_EUNSUPPORTED),         # below 16
        (dict(rotary_dim=256), L.LL_EUNSUPPORTED),       # does not divide head_dim 128
        (dict(head_dim=512, rotary_dim=512), L.LL_EUNSUPPORTED),
        (dict(num_kv_heads=512, head_dim=128), L.LL_EUNSUPPORTED),  # row wider than 32768
        (dict(rope_pairing=3), L.LL_EINVAL),
        (dict(v_layer_base=None), L.LL_EINVAL),
        (dict(page_table=None), L.LL_EINVAL),
    ]
    for change, code in cases:
        d = L._GqaPoolDesc(**{**base, **change})
        h = ctypes.c_void_p()
        assert L._lib.ll_pool_create_gqa(ctypes.byref(d), ctypes.byref(h)) == code, change
        assert not h.value
    misaligned = (ctypes.c_void_p * 2)(48, 72)
    d = L._GqaPoolDesc(**{**base, "v_layer_base": ctypes.cast(misaligned, ctypes.POINTER(ctypes.c_void_p))})
    assert L._lib.ll_pool_create_gqa(ctypes.byref(d), ctypes.byref(ctypes.c_void_p())) == L.LL_EINVAL


def test_trainer_mask_calls_reject_bad_arguments_before_touching_a_device():
    """Argument checks run before the context is used (a dummy context is
    enough) and before any device call."""
    from mla_paged_cache_amd import leyline as L
    fake = ctypes.create_string_buffer(512)
    ctx = ctypes.cast(fake, ctypes.c_void_p)
    vp = ctypes.c_void_p
    times = (ctypes.c_int64 * 2)(10, 10)
    lens = (ctypes.c_int64 * 2)(10, 10)
    log = L._KvsRolloutLog(20, 2, times, lens, 0)
    assert L._lib.kvs_death_times(None, ctypes.byref(log), 1, 32, vp(64), vp(64), vp(64), None) == L.LL_EINVAL
    # event times must strictly increase
    assert L._lib.kvs_death_times(ctx, ctypes.byref(log), 1, 32, vp(64), vp(64), vp(64), None) == L.LL_EINVAL
    times[1] = 15
    lens[1] = 16     # more rows than tokens generated
    assert L._lib.kvs_death_times(ctx, ctypes.byref(log), 1, 32, vp(64), vp(64), vp(64), None) == L.LL_EINVAL
    lens[1] = 12
    assert L._lib.kvs_death_times(ctx, ctypes.byref(log), 1, 16, vp(64), vp(64), vp(64), None) == L.LL_EINVAL
    times[1] = 21    # beyond n_tokens
    assert L._lib.kvs_death_times(ctx, ctypes.byref(log), 1, 32, vp(64), vp(64), vp(64), None) == L.LL_EINVAL
    for bq, bk in ((12, 16), (16, 2048), (8, 16)):
        assert L._lib.kvs_block_mask(ctx, vp(64), 1, 256, bq, bk, vp(64), vp(64), vp(64), vp(64), None) == L.LL_EINVAL
    assert L._lib.kvs_dense_mask(ctx, vp(64), 1, 200, vp(64), None) == L.LL_EINVAL   # not a multiple of 128
    assert L._lib.kvs_dense_mask(ctx, vp(64), 1, 256, vp(72), None) == L.LL_EINVAL   # misaligned


def test_null_pool_calls_fail_cleanly():
    from mla_paged_cache_amd import leyline as L
    assert L._lib.leyline_splice(None, None, 0, None) == L.LL_EINVAL
    assert L._lib.kv_evict_compact(None, None, 0, None, None, None) == L.LL_EINVAL
    assert L._lib.ll_ptable_reindex(None, 0, None, 0, None) == L.LL_EINVAL
    assert L._lib.ll_status_str(L.LL_ENOMEM).decode() == "LL_ENOMEM"


def test_host_rope_table_equals_oracle():
    from mla_paged_cache_amd import leyline as L
    from oracle import leyline_oracle as O
    for delta in (-6120, -1984, 0, 1, 7, 8191, -131071, 10 ** 6):
        c, s = L.rope_delta_table(delta)
        co, so = O.delta_cos_sin(delta)
        assert np.array_equal(c, co) and np.array_equal(s, so), delta
