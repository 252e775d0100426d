"""Python binding of libleyline.so (include/leyline.h): argument marshalling only.

Every step of the splice / evict path runs in the library's HIP kernels and
C++ host planner; this module turns torch tensors into device pointers and
the current torch stream into a hipStream_t, and turns status codes into
exceptions.  If the library is missing, importing this module fails loudly.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libleyline.so")

LL_OK, LL_EINVAL, LL_ERANGE, LL_ENOMEM, LL_EUNSUPPORTED, LL_EDEVICE, LL_EPOISONED = 0, -1, -2, -3, -4, -5, -6
AMORTIZE, FORGET, PIN, DECAY, SCRATCH = 0, 1, 2, 3, 4
ROPE_INTERLEAVED, ROPE_HALF = 0, 1
SPLICE_PLAN_AUTO, SPLICE_PLAN_HOST = 0, 1
KV_LORA_RANK, ROPE_DIM = 512, 64
ROW = KV_LORA_RANK + ROPE_DIM

# Every symbol include/leyline.h declares.
EXPORTS = (
    "ll_pool_create", "ll_pool_destroy", "ll_seq_alloc", "ll_seq_set_pages", "ll_seq_free",
    "ll_seq_get", "ll_pool_free_pages", "leyline_splice", "kv_evict_compact", "ll_ptable_reindex",
    "ll_rope_delta_table", "ll_last_plan_stats", "ll_pool_set_profiling", "ll_profile_read",
    "ll_last_error", "ll_status_str", "ll_pool_create_gqa",
    "kvs_ctx_create", "kvs_ctx_destroy", "kvs_death_times", "kvs_block_mask", "kvs_dense_mask",
    "ll_rope_rows", "ll_pool_set_splice_planner", "ll_pool_set_page_reuse", "ll_last_plan_bytes", "ll_seq_lengths",
    "leyline_splice_noalloc", "ll_pool_set_dispatch_limit",
)


class LeylineError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


class _PoolDesc(ctypes.Structure):
    _fields_ = [
        ("num_layers", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_seqs", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("kv_lora_rank", ctypes.c_int32),
        ("rope_dim", ctypes.c_int32),
        ("rope_pairing", ctypes.c_int32),
        ("rope_base", ctypes.c_double),
        ("layer_base", ctypes.POINTER(ctypes.c_void_p)),
        ("page_table", ctypes.c_void_p),
        ("device", ctypes.c_int32),
    ]


class _GqaPoolDesc(ctypes.Structure):
    _fields_ = [
        ("num_layers", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_seqs", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("rotary_dim", ctypes.c_int32),
        ("rope_pairing", ctypes.c_int32),
        ("rope_base", ctypes.c_double),
        ("k_layer_base", ctypes.POINTER(ctypes.c_void_p)),
        ("v_layer_base", ctypes.POINTER(ctypes.c_void_p)),
        ("page_table", ctypes.c_void_p),
        ("device", ctypes.c_int32),
    ]


class _Directive(ctypes.Structure):
    _fields_ = [
        ("seq_id", ctypes.c_int32),
        ("mode", ctypes.c_int32),
        ("s_start", ctypes.c_int64),
        ("s_end", ctypes.c_int64),
        ("r_len", ctypes.c_int64),
        ("r_rows", ctypes.c_void_p),
        ("r_layer_stride_bytes", ctypes.c_int64),
        ("r_rows_v", ctypes.c_void_p),
        ("r_layer_stride_bytes_v", ctypes.c_int64),
    ]


class _KvsRolloutLog(ctypes.Structure):
    _fields_ = [
        ("n_tokens", ctypes.c_int64),
        ("n_events", ctypes.c_int32),
        ("event_time", ctypes.POINTER(ctypes.c_int64)),
        ("mask_len", ctypes.POINTER(ctypes.c_int64)),
        ("mask_offset", ctypes.c_int64),
    ]


class _PlanStats(ctypes.Structure):
    _fields_ = [
        ("alg_bytes", ctypes.c_int64),
        ("rows_moved", ctypes.c_int64),
        ("rows_rotated_inplace", ctypes.c_int64),
        ("fresh_pages", ctypes.c_int64),
        ("freed_pages", ctypes.c_int64),
        ("table_entries", ctypes.c_int64),
        ("planned_on_device", ctypes.c_int64),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with mla_paged_cache_amd._build.build() "
                          "(the splice path has no fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64, vp = ctypes.POINTER, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    sig = {
        "ll_pool_create": (i32, [P(_PoolDesc), P(vp)]),
        "ll_pool_create_gqa": (i32, [P(_GqaPoolDesc), P(vp)]),
        "ll_pool_destroy": (None, [vp]),
        "ll_seq_alloc": (i32, [vp, i64, P(i32), vp]),
        "ll_seq_set_pages": (i32, [vp, i32, vp, i64, vp]),
        "ll_seq_free": (i32, [vp, i32]),
        "ll_seq_get": (i32, [vp, i32, P(i64), P(i64), P(i32), i32, P(i32)]),
        "ll_pool_free_pages": (i32, [vp, P(i64)]),
        "leyline_splice": (i32, [vp, P(_Directive), i32, vp]),
        "leyline_splice_noalloc": (i32, [vp, P(_Directive), i32, vp]),
        "kv_evict_compact": (i32, [vp, vp, i32, vp, vp, vp]),
        "ll_ptable_reindex": (i32, [vp, i32, vp, i32, vp]),
        "ll_rope_delta_table": (i32, [ctypes.c_double, i32, i64, P(ctypes.c_float), P(ctypes.c_float)]),
        "ll_last_plan_stats": (i32, [vp, P(_PlanStats)]),
        "ll_last_plan_bytes": (i32, [vp, P(i64), P(i64), P(i64)]),
        "ll_seq_lengths": (i32, [vp, vp, i32, vp]),
        "ll_pool_set_profiling": (i32, [vp, i32]),
        "ll_pool_set_splice_planner": (i32, [vp, i32]),
        "ll_pool_set_page_reuse": (i32, [vp, i32]),
        "ll_pool_set_dispatch_limit": (i32, [vp, i64]),
        "ll_profile_read": (i32, [vp, i32, P(i64), P(ctypes.c_double), P(i64), P(ctypes.c_float), i64]),
        "ll_rope_rows": (i32, [vp, i32, i64, i64, vp, vp, i64, vp]),
        "kvs_ctx_create": (i32, [i32, P(vp)]),
        "kvs_ctx_destroy": (None, [vp]),
        "kvs_death_times": (i32, [vp, P(_KvsRolloutLog), i32, i64, vp, vp, vp, vp]),
        "kvs_block_mask": (i32, [vp, vp, i32, i64, i32, i32, vp, vp, vp, vp, vp]),
        "kvs_dense_mask": (i32, [vp, vp, i32, i64, vp, vp]),
        "ll_last_error": (ctypes.c_char_p, []),
        "ll_status_str": (ctypes.c_char_p, [i32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def _status_name(s: int) -> str:
    return _lib.ll_status_str(s).decode()


def _check(status: int) -> None:
    if status != LL_OK:
        raise LeylineError(status, _lib.ll_last_error().decode())


def _i32_array(values):
    """(contiguous int32 array, its address); an int32 ndarray that is
    already contiguous is used as it is."""
    if isinstance(values, np.ndarray) and values.dtype == np.int32 and values.flags.c_contiguous:
        a = values.reshape(-1)
    else:
        a = np.ascontiguousarray(np.asarray(values, dtype=np.int32)).reshape(-1)
    return a, (a.ctypes.data if a.size else None)


def _require(t, name: str, dtype, shape, device) -> None:
    """Raise ValueError unless `t` is a contiguous tensor of `dtype` and
    exactly `shape` on `device` (checked before any kernel sees its pointer)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dtype != dtype or t.device != device or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: need a contiguous {dtype} tensor of shape {tuple(shape)} on {device}, got "
                         f"{t.dtype} {tuple(t.shape)} on {t.device}{'' if t.is_contiguous() else ' (not contiguous)'}")


def _stream_handle(stream, device: int) -> int:
    """The hipStream_t of `stream`, or of the current torch stream of
    `device` (the device the pool or context lives on) when stream is None."""
    if stream is not None:
        return stream.cuda_stream
    import torch
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(device)
    return torch.cuda.current_stream(device).cuda_stream


def rope_delta_table(delta: int, rope_dim: int = ROPE_DIM, base: float = 10000.0):
    """float32 (cos, sin) of delta * theta_j, as the library computes them."""
    c = np.zeros(rope_dim // 2, np.float32)
    s = np.zeros(rope_dim // 2, np.float32)
    _check(_lib.ll_rope_delta_table(base, rope_dim, int(delta),
                                    c.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                                    s.ctypes.data_as(ctypes.POINTER(ctypes.c_float))))
    return c, s


@dataclass
class Directive:
    """D = (s_start, s_end, R, m).  MLA pools: `stub` is a device bf16 tensor
    [L][r_len][576] (or [r_len][576] for a one-layer pool), or None for
    r_len = 0.  GQA / MHA pools: `stub` holds the K rows and `stub_v` the V
    rows, each [L][r_len][H][D]."""
    seq: int
    s_start: int
    s_end: int
    stub: object = None
    mode: int = AMORTIZE
    stub_v: object = None


@dataclass
class PlanStats:
    alg_bytes: int
    rows_moved: int
    rows_rotated_inplace: int
    fresh_pages: int
    freed_pages: int
    table_entries: int
    planned_on_device: int


class Pool:
    """A paged MLA cache over caller-owned torch memory.

    layers: a bf16 CUDA tensor [L][num_pages][page_size][576] or a list of L
    tensors [num_pages][page_size][576]; page_table: int32 CUDA tensor
    [max_seqs][max_pages_per_seq].  Both are kept referenced by the pool."""

    gqa = False

    def __init__(self, layers, page_table, rope_base: float = 10000.0, pairing: int = ROPE_INTERLEAVED):
        import torch
        if isinstance(layers, torch.Tensor):
            layer_list = [layers[i] for i in range(layers.shape[0])]
        else:
            layer_list = list(layers)
        if not layer_list:
            raise ValueError("no layers")
        shape = tuple(layer_list[0].shape)
        for t in layer_list:
            if t.dtype != torch.bfloat16 or not t.is_cuda or tuple(t.shape) != shape or not t.is_contiguous():
                raise ValueError("layers must be contiguous bf16 CUDA tensors of one shape [pages][P][576]")
        if len(shape) != 3 or shape[2] != ROW:
            raise ValueError("layer shape must be [num_pages][page_size][576]")
        if page_table.dtype != torch.int32 or not page_table.is_cuda or page_table.dim() != 2 \
                or not page_table.is_contiguous():
            raise ValueError("page_table must be a contiguous int32 CUDA tensor [max_seqs][max_pages_per_seq]")
        self._layers = layer_list
        self._keep = layers
        self.page_table = page_table
        self.num_layers = len(layer_list)
        self.num_pages, self.page_size = shape[0], shape[1]
        self.max_seqs, self.max_pages_per_seq = page_table.shape
        self.device = layer_list[0].device
        self._dev = self.device.index or 0
        self._ptrs = (ctypes.c_void_p * self.num_layers)(*[t.data_ptr() for t in layer_list])
        d = _PoolDesc(self.num_layers, self.page_size, self.num_pages, self.max_seqs, self.max_pages_per_seq,
                      KV_LORA_RANK, ROPE_DIM, pairing, rope_base,
                      ctypes.cast(self._ptrs, ctypes.POINTER(ctypes.c_void_p)),
                      page_table.data_ptr(), self.device.index or 0)
        h = ctypes.c_void_p()
        _check(_lib.ll_pool_create(ctypes.byref(d), ctypes.byref(h)))
        self._h = h

    # -- lifetime
    def close(self):
        if getattr(self, "_h", None):
            _lib.ll_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- sequences
    def seq_alloc(self, n_tokens: int, stream=None) -> int:
        sid = ctypes.c_int32()
        _check(_lib.ll_seq_alloc(self._h, int(n_tokens), ctypes.byref(sid), _stream_handle(stream, self._dev)))
        return sid.value

    def seq_set_pages(self, seq: int, pages, n_tokens: int, stream=None) -> None:
        arr, ptr = _i32_array(pages)
        _check(_lib.ll_seq_set_pages(self._h, int(seq), ptr, int(n_tokens), _stream_handle(stream, self._dev)))

    def seq_free(self, seq: int) -> None:
        _check(_lib.ll_seq_free(self._h, int(seq)))

    def seq_get(self, seq: int):
        """(length, next_position, page table as np.int32)."""
        n, pos, cnt = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
        _check(_lib.ll_seq_get(self._h, int(seq), ctypes.byref(n), ctypes.byref(pos), None, 0, ctypes.byref(cnt)))
        pages = np.zeros(cnt.value, np.int32)
        _check(_lib.ll_seq_get(self._h, int(seq), None, None,
                               pages.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), cnt.value, None))
        return n.value, pos.value, pages

    def free_pages(self) -> int:
        n = ctypes.c_int64()
        _check(_lib.ll_pool_free_pages(self._h, ctypes.byref(n)))
        return n.value

    # -- the path
    def _stub(self, st):
        """(r_len, pointer, layer stride in bytes) of one stub tensor."""
        import torch
        if st.dtype != torch.bfloat16 or st.device != self.device or st.shape[-1] != ROW:
            raise ValueError(f"stub must be a bf16 tensor [..., r_len, 576] on {self.device}")
        if st.dim() == 2:
            st = st.unsqueeze(0)
        if st.shape[0] != self.num_layers or st.stride(2) != 1 or st.stride(1) != ROW:
            raise ValueError("stub must be [num_layers][r_len][576] with contiguous rows")
        r_len = st.shape[1]
        return r_len, (st.data_ptr() if r_len else None), st.stride(0) * 2

    def splice(self, directives, stream=None, noalloc: bool = False) -> None:
        """Apply the directives (leyline_splice; noalloc=True:
        leyline_splice_noalloc, which allocates no device memory)."""
        n = len(directives)
        arr = (_Directive * max(1, n))()
        for i, d in enumerate(directives):
            r_len, ptr, stride, ptr_v, stride_v = 0, None, 0, None, 0
            if d.stub is not None and d.mode == AMORTIZE:
                r_len, ptr, stride = self._stub(d.stub)
                if self.gqa:
                    if d.stub_v is None:
                        raise ValueError("a GQA / MHA directive needs stub_v with stub")
                    r_v, ptr_v, stride_v = self._stub(d.stub_v)
                    if r_v != r_len:
                        raise ValueError("stub and stub_v hold different row counts")
            elif d.stub_v is not None and d.mode == AMORTIZE:
                raise ValueError("stub_v without stub")
            arr[i] = _Directive(int(d.seq), int(d.mode), int(d.s_start), int(d.s_end), int(r_len), ptr, stride,
                                ptr_v, stride_v)
        fn = _lib.leyline_splice_noalloc if noalloc else _lib.leyline_splice
        _check(fn(self._h, arr, n, _stream_handle(stream, self._dev)))

    def evict(self, seqs, keep, offsets, stream=None) -> None:
        """keep: uint8 CUDA tensor holding every mask; offsets[i]: start of
        sequence seqs[i]'s mask in it (its length is the sequence length)."""
        import torch
        if not isinstance(keep, torch.Tensor) or keep.dtype != torch.uint8 or keep.device != self.device \
                or not keep.is_contiguous():
            raise ValueError(f"keep must be a contiguous uint8 tensor on {self.device}")
        s_arr, s_ptr = _i32_array(seqs)
        o_arr = offsets if isinstance(offsets, np.ndarray) and offsets.dtype == np.int64 and offsets.flags.c_contiguous \
            else np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
        o_arr = o_arr.reshape(-1)
        if len(o_arr) != len(s_arr):
            raise ValueError(f"{len(s_arr)} sequences but {len(o_arr)} mask offsets")
        if len(s_arr):
            lens = np.empty(len(s_arr), np.int64)
            _check(_lib.ll_seq_lengths(self._h, s_ptr, len(s_arr), lens.ctypes.data))
            # a negative offset is the library's to refuse (LL_EINVAL)
            past = (o_arr >= 0) & (o_arr + lens > keep.numel())
            if past.any():
                i = int(np.argmax(past))
                raise ValueError(f"mask of sequence {int(s_arr[i])}: bytes [{int(o_arr[i])}, {int(o_arr[i] + lens[i])}) "
                                 f"outside keep's {keep.numel()}")
        _check(_lib.kv_evict_compact(self._h, s_ptr, len(s_arr), keep.data_ptr(),
                                     o_arr.ctypes.data if len(o_arr) else None, _stream_handle(stream, self._dev)))

    def rope_rows(self, seq: int, row_begin: int, angles, out=None, stream=None):
        """Turn the RoPE bands of rows [row_begin, row_begin + len(angles)) of
        a sequence by their own angle steps (angles: int64 CUDA tensor).  With
        out=None the pool is rotated in place; with out=True (or a tensor) the
        rows are gathered into [L][n][row] bf16 and returned, the pool left
        as it was."""
        import torch
        if not isinstance(angles, torch.Tensor) or angles.dtype != torch.int64 or angles.device != self.device \
                or angles.dim() != 1 or not angles.is_contiguous():
            raise ValueError(f"angles must be a contiguous 1-D int64 tensor on {self.device}")
        n = angles.numel()
        ptr, stride = None, 0
        if out is not None:
            shape = (self.num_layers, n, self.heads, self.head_dim) if self.gqa else (self.num_layers, n, ROW)
            if out is True:
                out = torch.empty(shape, dtype=torch.bfloat16, device=self.device)
            if not isinstance(out, torch.Tensor) or out.dtype != torch.bfloat16 or out.device != self.device \
                    or tuple(out.shape) != shape or not out[0].is_contiguous() or out.stride(0) < out[0].numel():
                raise ValueError(f"out must be a bf16 tensor {shape} on {self.device} with contiguous layers")
            ptr, stride = out.data_ptr(), out.stride(0) * 2
        _check(_lib.ll_rope_rows(self._h, int(seq), int(row_begin), int(n), angles.data_ptr() if n else None,
                                 ptr, stride, _stream_handle(stream, self._dev)))
        return out

    def ptable_reindex(self, seq: int, keep_pages, stream=None) -> None:
        arr, ptr = _i32_array(keep_pages)
        _check(_lib.ll_ptable_reindex(self._h, int(seq), ptr, len(arr), _stream_handle(stream, self._dev)))

    # -- counters
    def last_stats(self) -> PlanStats:
        s = _PlanStats()
        _check(_lib.ll_last_plan_stats(self._h, ctypes.byref(s)))
        return PlanStats(s.alg_bytes, s.rows_moved, s.rows_rotated_inplace, s.fresh_pages, s.freed_pages,
                         s.table_entries, s.planned_on_device)

    def set_splice_planner(self, planner: int) -> None:
        """SPLICE_PLAN_AUTO (default: small batches are planned on the device
        from kernel arguments) or SPLICE_PLAN_HOST (always staged and
        uploaded)."""
        _check(_lib.ll_pool_set_splice_planner(self._h, int(planner)))

    def set_page_reuse(self, on: bool) -> None:
        """True (default): a new page keeps an old one whose rows stay at their
        offsets.  False: every page of a rewritten sequence is fresh (the
        sequence is compacted into the lowest free pages); not on page size 1."""
        _check(_lib.ll_pool_set_page_reuse(self._h, 1 if on else 0))

    def set_dispatch_limit(self, max_items: int = 0) -> None:
        """Work-items per dispatch of a row-moving kernel (0: the packet's
        2^32 - 1; at least 1024 otherwise).  Larger launches are issued as
        several dispatches; results do not change."""
        _check(_lib.ll_pool_set_dispatch_limit(self._h, int(max_items)))

    def set_profiling(self, enable: bool, every: int = 1) -> None:
        """Time every `every`-th launch of each profiled kernel while enabled."""
        _check(_lib.ll_pool_set_profiling(self._h, max(1, int(every)) if enable else 0))

    def profile_read(self, kernel: int = 0, samples: int = 0):
        """(launches, total_ms, total_bytes) of kernel 0 (row moves), 1 (keep
        scan) or 2 (per-row rotation); with samples = k > 0 a fourth item, the
        milliseconds of the first k timed launches."""
        n, ms, b = ctypes.c_int64(), ctypes.c_double(), ctypes.c_int64()
        each = np.zeros(max(0, int(samples)), np.float32)
        _check(_lib.ll_profile_read(self._h, kernel, ctypes.byref(n), ctypes.byref(ms), ctypes.byref(b),
                                    each.ctypes.data_as(ctypes.POINTER(ctypes.c_float)) if samples else None,
                                    len(each)))
        if samples:
            return n.value, ms.value, b.value, each[:min(n.value, len(each))].astype(float).tolist()
        return n.value, ms.value, b.value


class GqaPool(Pool):
    """A paged GQA / MHA cache over caller-owned torch memory.

    k_layers, v_layers: bf16 CUDA tensors [L][num_pages][page_size][H][D] (or
    lists of L tensors [num_pages][page_size][H][D]); the first rotary_dim
    values of every K head are its RoPE band.  page_table as for Pool."""

    gqa = True

    def __init__(self, k_layers, v_layers, page_table, rotary_dim: int | None = None,
                 rope_base: float = 10000.0, pairing: int = ROPE_INTERLEAVED):
        import torch

        def planes(x):
            return [x[i] for i in range(x.shape[0])] if isinstance(x, torch.Tensor) else list(x)

        k_list, v_list = planes(k_layers), planes(v_layers)
        if not k_list or len(k_list) != len(v_list):
            raise ValueError("k_layers and v_layers must hold the same number (>= 1) of layers")
        shape = tuple(k_list[0].shape)
        if len(shape) != 4:
            raise ValueError("layer shape must be [num_pages][page_size][H][D]")
        for t in k_list + v_list:
            if t.dtype != torch.bfloat16 or not t.is_cuda or tuple(t.shape) != shape or not t.is_contiguous():
                raise ValueError("K and V layers must be contiguous bf16 CUDA tensors of one shape [pages][P][H][D]")
        if page_table.dtype != torch.int32 or not page_table.is_cuda or page_table.dim() != 2 \
                or not page_table.is_contiguous():
            raise ValueError("page_table must be a contiguous int32 CUDA tensor [max_seqs][max_pages_per_seq]")
        self._layers = k_list + v_list
        self._keep = (k_layers, v_layers)
        self.page_table = page_table
        self.num_layers = len(k_list)
        self.num_pages, self.page_size, self.heads, self.head_dim = shape
        self.rotary_dim = self.head_dim if rotary_dim is None else int(rotary_dim)
        self.row = self.heads * self.head_dim
        self.max_seqs, self.max_pages_per_seq = page_table.shape
        self.device = k_list[0].device
        self._dev = self.device.index or 0
        self._kptrs = (ctypes.c_void_p * self.num_layers)(*[t.data_ptr() for t in k_list])
        self._vptrs = (ctypes.c_void_p * self.num_layers)(*[t.data_ptr() for t in v_list])
        d = _GqaPoolDesc(self.num_layers, self.page_size, self.num_pages, self.max_seqs, self.max_pages_per_seq,
                         self.heads, self.head_dim, self.rotary_dim, pairing, rope_base,
                         ctypes.cast(self._kptrs, ctypes.POINTER(ctypes.c_void_p)),
                         ctypes.cast(self._vptrs, ctypes.POINTER(ctypes.c_void_p)),
                         page_table.data_ptr(), self.device.index or 0)
        h = ctypes.c_void_p()
        _check(_lib.ll_pool_create_gqa(ctypes.byref(d), ctypes.byref(h)))
        self._h = h

    def _stub(self, st):
        import torch
        if st.dtype != torch.bfloat16 or st.device != self.device or tuple(st.shape[-2:]) != (self.heads, self.head_dim):
            raise ValueError(f"stub rows must be bf16 tensors [..., r_len, H, D] on {self.device}")
        if st.dim() == 3:
            st = st.unsqueeze(0)
        if st.shape[0] != self.num_layers or st.stride(3) != 1 or st.stride(2) != self.head_dim \
                or st.stride(1) != self.row:
            raise ValueError("stub rows must be [num_layers][r_len][H][D] with contiguous rows")
        r_len = st.shape[1]
        return r_len, (st.data_ptr() if r_len else None), st.stride(0) * 2


@dataclass
class _Logs:
    n: int
    logs: object
    host: list
    keep: object


class KvsMask:
    """KV-streams trainer-side attention mask on one device: death times from
    the engine's eviction logs, then a block mask or a dense bit mask.

    A log is a list of (time, keep) events per rollout, keep being the mask the
    engine passed to its eviction call (uint8 over the rows held then)."""

    def __init__(self, device: int = 0):
        import torch
        h = ctypes.c_void_p()
        _check(_lib.kvs_ctx_create(int(device), ctypes.byref(h)))
        self._h = h
        self.device = device
        self._tdev = torch.device("cuda", device)

    def close(self):
        if getattr(self, "_h", None):
            _lib.kvs_ctx_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check_death(self, death):
        import torch
        if not isinstance(death, torch.Tensor) or death.dim() != 2:
            raise ValueError("death must be a 2-D int32 tensor [n][n_pad]")
        _require(death, "death", torch.int32, tuple(death.shape), self._tdev)

    def upload_logs(self, rollouts):
        """Marshal eviction logs once: rollouts is a list of (n_tokens,
        events), events a list of objects with .time and .keep (host uint8
        arrays).  The keep masks go to the device as one buffer."""
        import torch
        n = len(rollouts)
        chunks, logs, host = [], (_KvsRolloutLog * max(1, n))(), []
        off = 0
        for i, (n_tokens, events) in enumerate(rollouts):
            times = np.ascontiguousarray([int(e.time) for e in events], dtype=np.int64)
            lens = np.ascontiguousarray([len(e.keep) for e in events], dtype=np.int64)
            host += [times, lens]
            logs[i] = _KvsRolloutLog(int(n_tokens), len(events),
                                     times.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                     lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), off)
            for e in events:
                chunks.append(np.asarray(e.keep, dtype=np.uint8))
                off += len(e.keep)
        keep = torch.from_numpy(np.concatenate(chunks) if chunks else np.zeros(1, np.uint8)).to(
            torch.device("cuda", self.device))
        return _Logs(n, logs, host, keep)

    def death_times(self, rollouts, n_pad: int, stream=None, out=None):
        """Death times of the rollouts (a list as for upload_logs, or its
        result).  Returns (death int32 [n][n_pad], status int32 [n]) CUDA
        tensors."""
        import torch
        logs = rollouts if isinstance(rollouts, _Logs) else self.upload_logs(rollouts)
        dev = self._tdev
        if out is None:
            out = (torch.empty((logs.n, n_pad), dtype=torch.int32, device=dev),
                   torch.empty(logs.n, dtype=torch.int32, device=dev))
        death, status = out
        _require(death, "death", torch.int32, (logs.n, n_pad), dev)
        _require(status, "status", torch.int32, (logs.n,), dev)
        _check(_lib.kvs_death_times(self._h, logs.logs, logs.n, int(n_pad), logs.keep.data_ptr(), death.data_ptr(),
                                    status.data_ptr(), _stream_handle(stream, self.device)))
        self._last_logs = logs  # the kernel reads the keep buffer after this returns
        return death, status

    def block_mask(self, death, block_q: int, block_k: int, out=None, stream=None):
        """(partial_num [n][nq], partial_idx [n][nq][nk], full_num, full_idx).
        Without `out` the index arrays are new and filled with -1 past each
        count; with `out` (four int32 tensors of those shapes) the entries past
        each count are left as they were."""
        import torch
        self._check_death(death)
        n, n_pad = death.shape
        nq, nk = -(-n_pad // block_q), -(-n_pad // block_k)
        kw = dict(dtype=torch.int32, device=death.device)
        if out is None:
            pn, fn = torch.zeros((n, nq), **kw), torch.zeros((n, nq), **kw)
            pi, fi = torch.full((n, nq, nk), -1, **kw), torch.full((n, nq, nk), -1, **kw)
        else:
            pn, pi, fn, fi = out
            for x, shape in ((pn, (n, nq)), (pi, (n, nq, nk)), (fn, (n, nq)), (fi, (n, nq, nk))):
                if tuple(x.shape) != shape or x.dtype != torch.int32 or not x.is_contiguous() or x.device != death.device:
                    raise ValueError(f"block_mask out: need contiguous int32 {shape} on {death.device}")
        _check(_lib.kvs_block_mask(self._h, death.data_ptr(), n, n_pad, int(block_q), int(block_k), pn.data_ptr(),
                                   pi.data_ptr(), fn.data_ptr(), fi.data_ptr(), _stream_handle(stream, self.device)))
        return pn, pi, fn, fi

    def dense_mask(self, death, out=None, stream=None):
        """uint32 bits [n][n_pad][n_pad / 32] (as an int32 tensor)."""
        import torch
        self._check_death(death)
        n, n_pad = death.shape
        if out is None:
            out = torch.empty((n, n_pad, n_pad // 32), dtype=torch.int32, device=death.device)
        _require(out, "out", torch.int32, (n, n_pad, n_pad // 32), self._tdev)
        _check(_lib.kvs_dense_mask(self._h, death.data_ptr(), n, n_pad, out.data_ptr(), _stream_handle(stream, self.device)))
        return out
