"""ctypes binding of libmla (include/mla.h).

Argument marshalling only: every function here forwards to the C ABI of the
same name; torch tensors are used for device memory and the current stream.
If libmla.so has not been built, importing the binding raises -- there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmla.so")

MLA_OK = 0
MLA_ERR_INVALID_ARG = -1
MLA_ERR_UNSUPPORTED = -2
MLA_ERR_WORKSPACE = -3
MLA_ERR_HIP = -4
MLA_ERR_NO_DEVICE = -5

MLA_KV_FP8_656 = 0
MLA_KV_BF16_576 = 1
MLA_KV_V4_584 = 2
MLA_KV_V41_528 = 3

EXPORTED = ("mla_sched_meta_size", "mla_workspace_size", "mla_resolve_shape",
            "mla_get_sched_meta", "mla_plan_sched_meta_host", "mla_get_sched_meta_len",
            "mla_plan_sched_meta_len_host", "mla_sparse_decode_fwd", "mla_indexer_scores", "mla_indexer_topk",
            "mla_splitkv_combine", "mla_debug_gather_dequant", "mla_sparse_decode_noalloc",
            "mla_dense_decode_fwd", "mla_sparse_decode_extra_fwd",
            "mla_last_error", "mla_version")


class mla_shape(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int32), ("s_q", ctypes.c_int32), ("h_q", ctypes.c_int32),
                ("h_kv", ctypes.c_int32), ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("page_block_size", ctypes.c_int32),
                ("num_kv_tokens", ctypes.c_int64), ("kv_format", ctypes.c_int32),
                ("num_parts", ctypes.c_int32), ("split_granularity", ctypes.c_int32),
                ("fixed_overhead", ctypes.c_int32)]


class mla_indexer_args(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("q", ctypes.c_void_p), ("weights", ctypes.c_void_p), ("kcache", ctypes.c_void_p),
                ("page_table", ctypes.c_void_p), ("seq_len", ctypes.c_void_p), ("scores", ctypes.c_void_p),
                ("indices", ctypes.c_void_p)]


class mla_extra_kv(ctypes.Structure):
    _fields_ = [("kv", ctypes.c_void_p), ("kv_stride_block", ctypes.c_int64),
                ("page_block_size", ctypes.c_int32), ("num_kv_tokens", ctypes.c_int64),
                ("indices", ctypes.c_void_p), ("idx_stride_b", ctypes.c_int64), ("idx_stride_s", ctypes.c_int64),
                ("extra_topk", ctypes.c_int32), ("topk_length", ctypes.c_void_p)]


class mla_decode_args(ctypes.Structure):
    _fields_ = [("shape", mla_shape), ("sm_scale", ctypes.c_float),
                ("q", ctypes.c_void_p), ("q_stride_b", ctypes.c_int64),
                ("q_stride_s", ctypes.c_int64), ("q_stride_h", ctypes.c_int64),
                ("kv", ctypes.c_void_p), ("kv_stride_block", ctypes.c_int64),
                ("indices", ctypes.c_void_p), ("idx_stride_b", ctypes.c_int64),
                ("idx_stride_s", ctypes.c_int64),
                ("out", ctypes.c_void_p), ("out_stride_b", ctypes.c_int64),
                ("out_stride_s", ctypes.c_int64), ("out_stride_h", ctypes.c_int64),
                ("lse", ctypes.c_void_p),
                ("attn_sink", ctypes.c_void_p), ("topk_length", ctypes.c_void_p),
                ("sched_meta", ctypes.c_void_p), ("num_splits", ctypes.c_void_p),
                ("o_accum", ctypes.c_void_p), ("lse_accum", ctypes.c_void_p),
                ("o_accum_bytes", ctypes.c_size_t), ("lse_accum_bytes", ctypes.c_size_t)]


class MlaError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed with status {code}: {msg}")
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmla.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m sparse_mla_attention_decode_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    sz = ctypes.POINTER(ctypes.c_size_t)
    sig = {
        "mla_sched_meta_size": [P(mla_shape), sz, sz],
        "mla_workspace_size": [P(mla_shape), sz, sz],
        "mla_resolve_shape": [P(mla_shape)],
        "mla_get_sched_meta": [P(mla_shape), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p],
        "mla_plan_sched_meta_host": [P(mla_shape), ctypes.c_void_p, ctypes.c_void_p],
        "mla_get_sched_meta_len": [P(mla_shape), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p],
        "mla_plan_sched_meta_len_host": [P(mla_shape), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p],
        "mla_sparse_decode_fwd": [P(mla_decode_args), ctypes.c_void_p],
        "mla_indexer_scores": [P(mla_indexer_args), ctypes.c_void_p],
        "mla_indexer_topk": [P(mla_indexer_args), ctypes.c_void_p],
        "mla_splitkv_combine": [P(mla_decode_args), ctypes.c_void_p],
        "mla_sparse_decode_noalloc": [P(mla_decode_args), ctypes.c_void_p],
        "mla_dense_decode_fwd": [P(mla_decode_args), ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                 ctypes.c_void_p],
        "mla_debug_gather_dequant": [P(mla_decode_args), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p],
    }
    for name, argtypes in sig.items():
        f = getattr(lib, name)
        f.argtypes = argtypes
        f.restype = ctypes.c_int
    for name in ("mla_last_error", "mla_version"):
        f = getattr(lib, name)
        f.argtypes = []
        f.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(fn: str, code: int) -> int:
    if code != MLA_OK:
        raise MlaError(fn, code, load_library().mla_last_error().decode())
    return code


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return int(stream)


# ----------------------------------------------------------------------------- thin wrappers
def mla_version() -> str:
    return load_library().mla_version().decode()


def mla_last_error() -> str:
    return load_library().mla_last_error().decode()


def mla_resolve_shape(shape: mla_shape) -> mla_shape:
    s = mla_shape.from_buffer_copy(shape)
    _check("mla_resolve_shape", load_library().mla_resolve_shape(ctypes.byref(s)))
    return s


def mla_sched_meta_size(shape: mla_shape) -> Tuple[int, int]:
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    _check("mla_sched_meta_size", load_library().mla_sched_meta_size(ctypes.byref(shape), ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def mla_workspace_size(shape: mla_shape) -> Tuple[int, int]:
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    _check("mla_workspace_size", load_library().mla_workspace_size(ctypes.byref(shape), ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def mla_plan_sched_meta_host(shape: mla_shape, meta_ptr: int, num_splits_ptr: int) -> None:
    _check("mla_plan_sched_meta_host", load_library().mla_plan_sched_meta_host(ctypes.byref(shape), meta_ptr, num_splits_ptr))


def mla_get_sched_meta(shape: mla_shape, meta_ptr: int, num_splits_ptr: int, stream=None) -> None:
    _check("mla_get_sched_meta", load_library().mla_get_sched_meta(ctypes.byref(shape), meta_ptr, num_splits_ptr, _stream(stream)))


def mla_plan_sched_meta_len_host(shape: mla_shape, lengths_ptr: int, meta_ptr: int, num_splits_ptr: int) -> None:
    _check("mla_plan_sched_meta_len_host",
           load_library().mla_plan_sched_meta_len_host(ctypes.byref(shape), lengths_ptr, meta_ptr, num_splits_ptr))


def mla_get_sched_meta_len(shape: mla_shape, lengths_ptr: int, meta_ptr: int, num_splits_ptr: int,
                           stream=None) -> None:
    _check("mla_get_sched_meta_len", load_library().mla_get_sched_meta_len(
        ctypes.byref(shape), lengths_ptr, meta_ptr, num_splits_ptr, _stream(stream)))


def mla_sparse_decode_fwd(args: mla_decode_args, stream=None) -> None:
    _check("mla_sparse_decode_fwd", load_library().mla_sparse_decode_fwd(ctypes.byref(args), _stream(stream)))


def mla_splitkv_combine(args: mla_decode_args, stream=None) -> None:
    _check("mla_splitkv_combine", load_library().mla_splitkv_combine(ctypes.byref(args), _stream(stream)))


def mla_sparse_decode_extra_fwd(args: mla_decode_args, extra: mla_extra_kv, stream=None) -> None:
    _check("mla_sparse_decode_extra_fwd", load_library().mla_sparse_decode_extra_fwd(
        ctypes.byref(args), ctypes.byref(extra), _stream(stream)))


def extra_kv_args(kv, page_block_size: int, indices, topk_length=None) -> mla_extra_kv:
    """Marshal an FP4 extra cache: kv uint8 [num_blocks, page stride] (contiguous
    rows), indices int32 [b, s_q, extra_topk] (last dim contiguous), topk_length
    int32 [b] or None (device tensors).  The returned struct keeps the tensors
    alive for as long as it lives."""
    import torch
    fn = "extra_kv_args"
    _require(kv.dtype == torch.uint8 and kv.dim() == 2 and kv.stride(1) == 1, fn,
             "kv must be uint8 [num_blocks, page stride] with contiguous rows")
    _require(indices.dtype == torch.int32 and indices.dim() == 3 and indices.stride(2) == 1, fn,
             "indices must be int32 [b, s_q, extra_topk] with a contiguous last dim")
    _require(topk_length is None or (topk_length.dtype == torch.int32 and topk_length.is_contiguous()), fn,
             "topk_length must be contiguous int32 [b]")
    x = mla_extra_kv()
    x.kv, x.kv_stride_block = kv.data_ptr(), kv.stride(0)
    x.page_block_size, x.num_kv_tokens = page_block_size, kv.shape[0] * page_block_size
    x.indices, x.idx_stride_b, x.idx_stride_s = indices.data_ptr(), indices.stride(0), indices.stride(1)
    x.extra_topk = indices.shape[2]
    x.topk_length = None if topk_length is None else topk_length.data_ptr()
    x.tensors = (kv, indices, topk_length)        # the struct holds raw pointers: keep their memory alive
    return x


def mla_dense_decode_fwd(args: mla_decode_args, block_table_ptr: int, block_table_stride: int, causal: bool,
                         stream=None) -> None:
    _check("mla_dense_decode_fwd", load_library().mla_dense_decode_fwd(
        ctypes.byref(args), block_table_ptr, block_table_stride, int(causal), _stream(stream)))


def mla_sparse_decode_noalloc(args: mla_decode_args, stream=None) -> None:
    _check("mla_sparse_decode_noalloc", load_library().mla_sparse_decode_noalloc(ctypes.byref(args), _stream(stream)))


def mla_debug_gather_dequant(args: mla_decode_args, k_rows_ptr: int, v_rows_ptr: int, stream=None) -> None:
    _check("mla_debug_gather_dequant",
           load_library().mla_debug_gather_dequant(ctypes.byref(args), k_rows_ptr, v_rows_ptr, _stream(stream)))


# ----------------------------------------------------------------------------- torch plumbing
def mla_indexer_scores(args: mla_indexer_args, stream=None) -> None:
    _check("mla_indexer_scores", load_library().mla_indexer_scores(ctypes.byref(args), _stream(stream)))


def mla_indexer_topk(args: mla_indexer_args, stream=None) -> None:
    _check("mla_indexer_topk", load_library().mla_indexer_topk(ctypes.byref(args), _stream(stream)))


def _require(ok: bool, fn: str, msg: str) -> None:
    if not ok:
        raise MlaError(fn, MLA_ERR_INVALID_ARG, msg)


def indexer_args(q, weights, kcache, page_table, seq_len, topk: int, scores, indices) -> mla_indexer_args:
    """Marshal contiguous device tensors: q uint8 [b, H, 128], weights fp32 [b, H],
    kcache uint8 [num_pages, 8448], page_table int32 [b, max_pages], seq_len
    int32 [b], scores bf16 [b, max_pages * 64], indices int32 [b, topk].  The
    shapes and dtypes are checked here: the C ABI takes raw pointers."""
    import torch
    fn = "indexer_args"
    _require(q.dtype == torch.uint8 and q.dim() == 3 and q.shape[2] == 128, fn, "q must be uint8 [b, H, 128]")
    b, heads = q.shape[0], q.shape[1]
    _require(weights.dtype == torch.float32 and tuple(weights.shape) == (b, heads), fn,
             "weights must be float32 [b, H]")
    _require(kcache.dtype == torch.uint8 and kcache.dim() == 2 and kcache.shape[1] == 8448, fn,
             "kcache must be uint8 [num_pages, 8448]")
    _require(page_table.dtype == torch.int32 and page_table.dim() == 2 and page_table.shape[0] == b, fn,
             "page_table must be int32 [b, max_pages]")
    _require(seq_len.dtype == torch.int32 and tuple(seq_len.shape) == (b,), fn, "seq_len must be int32 [b]")
    _require(scores.dtype == torch.bfloat16 and tuple(scores.shape) == (b, page_table.shape[1] * 64), fn,
             "scores must be bfloat16 [b, max_pages * 64]")
    _require(indices.dtype == torch.int32 and tuple(indices.shape) == (b, topk), fn,
             "indices must be int32 [b, topk]")
    for name, t in (("q", q), ("weights", weights), ("kcache", kcache), ("page_table", page_table),
                    ("seq_len", seq_len), ("scores", scores), ("indices", indices)):
        _require(t.is_contiguous(), fn, f"{name} must be contiguous")
    a = mla_indexer_args()
    a.b, a.n_heads = b, heads
    a.max_pages, a.num_pages, a.topk = page_table.shape[1], kcache.shape[0], topk
    a.q, a.weights, a.kcache = q.data_ptr(), weights.data_ptr(), kcache.data_ptr()
    a.page_table, a.seq_len = page_table.data_ptr(), seq_len.data_ptr()
    a.scores, a.indices = scores.data_ptr(), indices.data_ptr()
    a.tensors = (q, weights, kcache, page_table, seq_len, scores, indices)   # keep the memory alive
    return a


def indexer_select(q, weights, kcache, page_table, seq_len, topk: int, scores=None, indices=None, stream=None):
    """scores -> top-k on `stream`; returns (indices int32 [b, topk], scores)."""
    import torch
    b, max_pages = page_table.shape
    if scores is None:
        scores = torch.empty((b, max_pages * 64), dtype=torch.bfloat16, device=q.device)
    if indices is None:
        indices = torch.empty((b, topk), dtype=torch.int32, device=q.device)
    a = indexer_args(q, weights, kcache, page_table, seq_len, topk, scores, indices)
    mla_indexer_scores(a, stream)
    mla_indexer_topk(a, stream)
    return indices, scores


def make_shape(b, s_q, h_q, topk, num_kv_tokens, kv_format=MLA_KV_FP8_656, page_block_size=64,
               num_parts=0, split_granularity=0, fixed_overhead=-1) -> mla_shape:
    """d_qk follows the format: 512 for the V4 / V4.1 caches, else 576."""
    d_qk = 512 if kv_format in (MLA_KV_V4_584, MLA_KV_V41_528) else 576
    return mla_shape(b=b, s_q=s_q, h_q=h_q, h_kv=1, d_qk=d_qk, d_v=512, topk=topk,
                     page_block_size=page_block_size if kv_format != MLA_KV_BF16_576 else 1,
                     num_kv_tokens=num_kv_tokens, kv_format=kv_format, num_parts=num_parts,
                     split_granularity=split_granularity, fixed_overhead=fixed_overhead)


class DecodePlan:
    """Device buffers (sched meta, split prefix, workspace, outputs) for one shape,
    allocated with torch.  The plan can be reused for every call of that shape."""

    def __init__(self, shape: mla_shape, device="cuda", closed_form: bool = False, by_length: bool = False):
        """closed_form=True (fixed_overhead 0 only) passes a NULL plan: the
        kernels evaluate the plan themselves and get_sched_meta does nothing.
        by_length=True makes the plan from the topk_length given to run()
        (mla_get_sched_meta_len), so requests cost their valid slots only."""
        import torch
        self.shape = mla_resolve_shape(shape)
        self.closed_form = closed_form
        self.by_length = by_length
        if closed_form and by_length:
            raise MlaError("DecodePlan", MLA_ERR_INVALID_ARG, "a closed-form plan cannot follow lengths")
        if closed_form and self.shape.fixed_overhead != 0:
            raise MlaError("DecodePlan", MLA_ERR_INVALID_ARG, "closed_form needs fixed_overhead 0")
        meta_b, ns_b = mla_sched_meta_size(self.shape)
        o_b, l_b = mla_workspace_size(self.shape)
        s = self.shape
        self.sched_meta = None if closed_form else torch.empty(meta_b // 4, dtype=torch.int32, device=device)
        self.num_splits = None if closed_form else torch.empty(ns_b // 4, dtype=torch.int32, device=device)
        self.o_accum = torch.empty(o_b // 4, dtype=torch.float32, device=device)
        self.lse_accum = torch.empty(l_b // 4, dtype=torch.float32, device=device)
        self.out = torch.empty((s.b, s.s_q, s.h_q, 512), dtype=torch.bfloat16, device=device)
        self.lse = torch.empty((s.b, s.h_q, s.s_q), dtype=torch.float32, device=device)

    def get_sched_meta(self, stream=None, topk_length=None):
        if self.closed_form:
            return
        if self.by_length:
            if topk_length is None:
                raise MlaError("DecodePlan", MLA_ERR_INVALID_ARG, "a by_length plan needs topk_length")
            mla_get_sched_meta_len(self.shape, topk_length.data_ptr(), self.sched_meta.data_ptr(),
                                   self.num_splits.data_ptr(), stream)
        else:
            mla_get_sched_meta(self.shape, self.sched_meta.data_ptr(), self.num_splits.data_ptr(), stream)

    def args(self, q, kv, indices, sm_scale: float = 0.0, out=None, lse=None, attn_sink=None,
             topk_length=None) -> mla_decode_args:
        """attn_sink: fp32 [h_q] device tensor or None; topk_length: int32 [b] device
        tensor or None (both contiguous)."""
        if self.by_length and topk_length is None:
            raise MlaError("DecodePlan", MLA_ERR_INVALID_ARG,
                           "a by_length plan needs the topk_length it was made from")
        out = self.out if out is None else out
        lse = self.lse if lse is None else lse
        a = mla_decode_args()
        a.shape = self.shape
        a.sm_scale = sm_scale
        a.q = q.data_ptr()
        a.q_stride_b, a.q_stride_s, a.q_stride_h = q.stride(0), q.stride(1), q.stride(2)
        a.kv = kv.data_ptr()
        a.kv_stride_block = kv.stride(0) * kv.element_size()     # bytes per page / bf16 row
        if indices is not None:                            # dense decode passes none
            a.indices = indices.data_ptr()
            a.idx_stride_b, a.idx_stride_s = indices.stride(0), indices.stride(1)
        a.out = out.data_ptr()
        a.out_stride_b, a.out_stride_s, a.out_stride_h = out.stride(0), out.stride(1), out.stride(2)
        a.lse = lse.data_ptr()
        a.attn_sink = None if attn_sink is None else attn_sink.data_ptr()
        a.topk_length = None if topk_length is None else topk_length.data_ptr()
        a.sched_meta = None if self.closed_form else self.sched_meta.data_ptr()
        a.num_splits = None if self.closed_form else self.num_splits.data_ptr()
        a.o_accum = self.o_accum.data_ptr()
        a.lse_accum = self.lse_accum.data_ptr()
        a.o_accum_bytes = self.o_accum.numel() * 4
        a.lse_accum_bytes = self.lse_accum.numel() * 4
        a.tensors = (q, kv, indices, out, lse, attn_sink, topk_length)   # keep the memory alive
        return a

    def run_dense(self, q, kv, block_table, cache_seqlens, sm_scale: float = 0.0, causal: bool = False,
                  stream=None, with_sched: bool = True, attn_sink=None):
        """Dense decode: sched (optional; a by_length plan follows cache_seqlens)
        -> mla_dense_decode_fwd -> combine.  block_table int32 [b, topk / 64]
        (row stride taken from the tensor), cache_seqlens int32 [b]."""
        import torch
        _require(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.stride(1) == 1,
                 "run_dense", "block_table must be int32 [b, pages] with contiguous rows")
        _require(cache_seqlens.dtype == torch.int32 and cache_seqlens.is_contiguous(), "run_dense",
                 "cache_seqlens must be contiguous int32 [b]")
        if with_sched:
            self.get_sched_meta(stream, cache_seqlens)
        a = self.args(q, kv, None, sm_scale, attn_sink=attn_sink, topk_length=cache_seqlens)
        mla_dense_decode_fwd(a, block_table.data_ptr(), block_table.stride(0), causal, stream)
        mla_splitkv_combine(a, stream)
        return self.out, self.lse

    def run_extra(self, q, kv, indices, extra, sm_scale: float = 0.0, stream=None, with_sched: bool = True,
                  attn_sink=None, topk_length=None):
        """V4.1 main cache + FP4 extra cache (extra: mla_extra_kv, see
        extra_kv_args): the plan's shape.topk counts main and extra slots."""
        if with_sched:
            self.get_sched_meta(stream, topk_length)
        a = self.args(q, kv, indices, sm_scale, attn_sink=attn_sink, topk_length=topk_length)
        mla_sparse_decode_extra_fwd(a, extra, stream)
        mla_splitkv_combine(a, stream)
        return self.out, self.lse

    def run(self, q, kv, indices, sm_scale: float = 0.0, stream=None, with_sched: bool = True,
            attn_sink=None, topk_length=None):
        """sched (optional) -> decode -> combine, all on `stream`."""
        if with_sched:
            self.get_sched_meta(stream, topk_length)
        a = self.args(q, kv, indices, sm_scale, attn_sink=attn_sink, topk_length=topk_length)
        mla_sparse_decode_fwd(a, stream)
        mla_splitkv_combine(a, stream)
        return self.out, self.lse
