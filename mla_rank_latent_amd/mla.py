"""Python binding of the MLA decode library (``include/mla.h``).

Argument marshalling only: each function takes torch tensors, reads their
device pointers and shapes, and calls the C entry point of the same name.
Every step of the computation runs in the library's HIP kernels.  Importing
this module loads ``libmla_rank_latent.so`` and raises ImportError if it is
missing; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla_rank_latent.so")

MLA_DTYPE_F32 = 0
MLA_DTYPE_BF16 = 1
MLA_DTYPE_BF16_FP8 = 2   # bf16 tensors, latent cache in FP8 E4M3 pages
MLA_FP8_PAGE_BYTES = 41216
_DTYPES = {"f32": MLA_DTYPE_F32, "bf16": MLA_DTYPE_BF16, "bf16_fp8": MLA_DTYPE_BF16_FP8}
MLA_STATUS_BAD_BLOCK = 0x1
MLA_STATUS_BAD_LENGTH = 0x2
MLA_STATUS_BAD_POS = 0x4

EXPORTS = ("mla_status_str", "mla_cache_bytes", "mla_cache_append", "mla_cache_append_workspace_bytes",
           "mla_cache_quantize",
           "mla_q_project", "mla_decode_workspace_bytes", "mla_decode", "mla_decode_prepare", "mla_decode_attend",
           "mla_decode_finish", "mla_prefill_workspace_bytes", "mla_prefill", "mla_prefill_expand",
           "mla_prefill_attend", "mla_layer_workspace_bytes", "mla_q_compress", "mla_out_project",
           "mla_decode_noalloc", "mla_decode_step_workspace_bytes", "mla_decode_step")
MLA_PHASE_PREPARE, MLA_PHASE_ATTEND, MLA_PHASE_FINISH, MLA_PHASE_ALL = 1, 2, 4, 7
MLA_NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (or python -m mla_rank_latent_amd.build)")
# The library must run on the same HIP runtime as the tensors and streams it is
# handed.  torch's HIP library is requested by file name (libamdhip64.so) but
# carries the soname libamdhip64.so.7, which is what the library asks for: with
# torch loaded first the loader binds the library to torch's runtime; loaded the
# other way round, the process would hold two HIP (and HSA) runtimes, and the
# library's device queries and launches would go to one that does not own the
# tensors.  So torch, when installed, is imported before the library is opened.
try:
    import torch  # noqa: F401
except ImportError:
    torch = None
_lib = ctypes.CDLL(LIB_PATH)


class MlaDims(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("d_nope", ctypes.c_int32), ("d_rope", ctypes.c_int32),
                ("d_latent", ctypes.c_int32), ("d_model", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("rope_base", ctypes.c_float)]


_P = ctypes.c_void_p
_I = ctypes.c_int32


class MlaStepArgs(ctypes.Structure):
    _fields_ = [("h", _P), ("w_dkv", _P), ("w_kr", _P), ("positions", _P), ("q_nope", _P), ("q_rope", _P),
                ("w_uk", _P), ("w_uv", _P), ("cache", _P), ("num_blocks", _I), ("block_table", _P),
                ("max_blocks", _I), ("seq_lens", _P), ("batch", _I), ("sq", _I), ("softmax_scale", ctypes.c_float),
                ("num_splits", _I), ("workspace", _P), ("workspace_bytes", ctypes.c_size_t), ("out", _P),
                ("lse", _P), ("status", _P)]
_lib.mla_status_str.restype = ctypes.c_char_p
_lib.mla_status_str.argtypes = [ctypes.c_int]
_lib.mla_cache_bytes.restype = ctypes.c_size_t
_lib.mla_cache_bytes.argtypes = [ctypes.POINTER(MlaDims), ctypes.c_int64]
_lib.mla_cache_append.restype = ctypes.c_int
_lib.mla_cache_append.argtypes = [ctypes.POINTER(MlaDims), _P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _P, ctypes.c_size_t,
                                  _P, _P]
_lib.mla_cache_append_workspace_bytes.restype = ctypes.c_size_t
_lib.mla_cache_append_workspace_bytes.argtypes = [ctypes.POINTER(MlaDims), _I, _I]
_lib.mla_cache_quantize.restype = ctypes.c_int
_lib.mla_cache_quantize.argtypes = [ctypes.POINTER(MlaDims), _P, _P, _I, _P]
_lib.mla_q_project.restype = ctypes.c_int
_lib.mla_q_project.argtypes = [ctypes.POINTER(MlaDims), _P, _P, _P, _P, _P, _P, _I, _I, _P]
_lib.mla_decode_workspace_bytes.restype = ctypes.c_size_t
_lib.mla_decode_workspace_bytes.argtypes = [ctypes.POINTER(MlaDims), _I, _I, _I]
_lib.mla_prefill_workspace_bytes.restype = ctypes.c_size_t
_lib.mla_prefill_workspace_bytes.argtypes = [ctypes.POINTER(MlaDims), _I, _I]
_lib.mla_layer_workspace_bytes.restype = ctypes.c_size_t
_lib.mla_layer_workspace_bytes.argtypes = [ctypes.POINTER(MlaDims), _I, _I, _I]
_lib.mla_q_compress.restype = ctypes.c_int
_lib.mla_q_compress.argtypes = [ctypes.POINTER(MlaDims), _I, _P, _P, _P, _P, _P, _P, _P, _I, _I, _P, ctypes.c_size_t,
                                _P]
_lib.mla_out_project.restype = ctypes.c_int
_lib.mla_out_project.argtypes = [ctypes.POINTER(MlaDims), _P, _P, _P, _I, _I, _P, ctypes.c_size_t, _P]
for _name in ("mla_prefill", "mla_prefill_expand", "mla_prefill_attend"):
    getattr(_lib, _name).restype = ctypes.c_int
    getattr(_lib, _name).argtypes = [ctypes.POINTER(MlaDims), _P, _P, _P, _P, _P, _I, _P, _I, _P, _I, _I,
                                     ctypes.c_float, _P, ctypes.c_size_t, _P, _P, _P, _P]
for _name in ("mla_decode", "mla_decode_prepare", "mla_decode_attend", "mla_decode_finish"):
    getattr(_lib, _name).restype = ctypes.c_int
    getattr(_lib, _name).argtypes = [ctypes.POINTER(MlaDims), _P, _P, _P, _P, _P, _I, _P, _I, _P, _I, _I,
                                     ctypes.c_float, _I, _P, ctypes.c_size_t, _P, _P, _P, _P]
_lib.mla_decode_step_workspace_bytes.restype = ctypes.c_size_t
_lib.mla_decode_step_workspace_bytes.argtypes = [ctypes.POINTER(MlaDims), _I, _I, _I]
_lib.mla_decode_step.restype = ctypes.c_int
_lib.mla_decode_step.argtypes = [ctypes.POINTER(MlaDims), ctypes.POINTER(MlaStepArgs), _I, _P]
_lib.mla_decode_noalloc.restype = ctypes.c_int
_lib.mla_decode_noalloc.argtypes = [ctypes.POINTER(MlaDims), _P, _P, _P, _P, _P, _I, _P, _I, _P, _I, _I,
                                    ctypes.c_float, _I, _P, _P, _P, _P]


class MlaError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} returned {code}: {mla_status_str(code)}")
        self.code = code


def dims(n_heads: int, d_nope: int, d_rope: int, d_latent: int, d_model: int, block_size: int = 64,
         dtype: str = "bf16", rope_base: float = 10000.0) -> MlaDims:
    """dtype: "bf16", "f32", or "bf16_fp8" (bf16 tensors, the cache in FP8 pages)."""
    return MlaDims(n_heads, d_nope, d_rope, d_latent, d_model, block_size, _DTYPES[dtype], rope_base)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise MlaError(fn, rc)


def mla_status_str(code: int) -> str:
    return _lib.mla_status_str(code).decode()


def mla_cache_bytes(d: MlaDims, tokens: int) -> int:
    return int(_lib.mla_cache_bytes(ctypes.byref(d), tokens))


def mla_decode_workspace_bytes(d: MlaDims, batch: int, sq: int, num_splits: int = 0) -> int:
    return int(_lib.mla_decode_workspace_bytes(ctypes.byref(d), batch, sq, num_splits))


def mla_prefill_workspace_bytes(d: MlaDims, batch: int, max_blocks: int) -> int:
    return int(_lib.mla_prefill_workspace_bytes(ctypes.byref(d), batch, max_blocks))


def mla_layer_workspace_bytes(d: MlaDims, d_qlat: int, batch: int, sq: int) -> int:
    return int(_lib.mla_layer_workspace_bytes(ctypes.byref(d), d_qlat, batch, sq))


def prepared_q_compress(d: MlaDims, d_qlat: int, h, w_dq, w_uq, w_qr, positions, q_nope, q_rope, workspace,
                        stream=None):
    """h [batch, sq, d_model] -> q_nope, q_rope (as mla_decode takes them) through the compressed query;
    returns a zero-argument launcher (arguments marshalled once, return code checked on every call).  The
    launcher keeps references to the tensors, so their memory stays valid while it lives."""
    batch, sq = int(h.shape[0]), int(h.shape[1])
    keep = (d, h, w_dq, w_uq, w_qr, positions, q_nope, q_rope, workspace)
    args = (ctypes.byref(d), d_qlat, _ptr(h), _ptr(w_dq), _ptr(w_uq), _ptr(w_qr), _ptr(positions), _ptr(q_nope),
            _ptr(q_rope), batch, sq, _ptr(workspace), _nbytes(workspace), _stream(stream))

    def launch(_keep=keep) -> None:
        _check("mla_q_compress", _lib.mla_q_compress(*args))
    return launch


def mla_q_compress(d: MlaDims, d_qlat: int, h, w_dq, w_uq, w_qr, positions, q_nope, q_rope, workspace,
                   stream=None) -> None:
    prepared_q_compress(d, d_qlat, h, w_dq, w_uq, w_qr, positions, q_nope, q_rope, workspace, stream)()


def prepared_out_project(d: MlaDims, o, w_o, u, workspace, stream=None):
    """o [batch, sq, n_heads, d_nope] -> u [batch, sq, d_model]; returns a zero-argument launcher that
    keeps references to the tensors."""
    batch, sq = int(o.shape[0]), int(o.shape[1])
    keep = (d, o, w_o, u, workspace)
    args = (ctypes.byref(d), _ptr(o), _ptr(w_o), _ptr(u), batch, sq, _ptr(workspace), _nbytes(workspace),
            _stream(stream))

    def launch(_keep=keep) -> None:
        _check("mla_out_project", _lib.mla_out_project(*args))
    return launch


def mla_out_project(d: MlaDims, o, w_o, u, workspace, stream=None) -> None:
    prepared_out_project(d, o, w_o, u, workspace, stream)()


def mla_cache_append_workspace_bytes(d: MlaDims, batch: int, t: int) -> int:
    return int(_lib.mla_cache_append_workspace_bytes(ctypes.byref(d), batch, t))


def _nbytes(t) -> int:
    return 0 if t is None else int(t.numel() * t.element_size())


def mla_cache_append(d: MlaDims, h, w_dkv, w_kr, positions, block_table, cache, workspace=None, status=None,
                     stream=None) -> None:
    """h [batch, t, d_model]; positions [batch, t] int32; block_table [batch, max_blocks] int32;
    cache [num_blocks, block_size, d_latent + d_rope] (written in place); optional ``workspace``, a byte
    tensor of at least mla_cache_append_workspace_bytes(d, batch, t), selects the split path."""
    batch, t = int(h.shape[0]), int(h.shape[1])
    _check("mla_cache_append", _lib.mla_cache_append(
        ctypes.byref(d), _ptr(h), _ptr(w_dkv), _ptr(w_kr), _ptr(positions), _ptr(block_table),
        int(block_table.shape[1]), _ptr(cache), int(cache.shape[0]), batch, t, _ptr(workspace), _nbytes(workspace),
        _ptr(status), _stream(stream)))


def mla_cache_quantize(d: MlaDims, src, pages, stream=None) -> None:
    """src [num_blocks, 64, d_latent + d_rope] bf16 -> pages [num_blocks, MLA_FP8_PAGE_BYTES] uint8 (written);
    ``d`` has dtype "bf16_fp8"."""
    _check("mla_cache_quantize", _lib.mla_cache_quantize(ctypes.byref(d), _ptr(src), _ptr(pages),
                                                         int(src.shape[0]), _stream(stream)))


def mla_q_project(d: MlaDims, h, w_q, w_qr, positions, q_nope, q_rope, stream=None) -> None:
    """h [batch, sq, d_model]; q_nope [batch, sq, n_heads, d_nope] and q_rope [batch, sq, n_heads, d_rope] written."""
    batch, sq = int(h.shape[0]), int(h.shape[1])
    _check("mla_q_project", _lib.mla_q_project(
        ctypes.byref(d), _ptr(h), _ptr(w_q), _ptr(w_qr), _ptr(positions), _ptr(q_nope), _ptr(q_rope),
        batch, sq, _stream(stream)))


def _decode_call(fn: str, d: MlaDims, q_nope, q_rope, w_uk, w_uv, cache, block_table, seq_lens, softmax_scale,
                 workspace, out, lse, status, num_splits, stream) -> None:
    batch, sq = int(q_nope.shape[0]), int(q_nope.shape[1])
    _check(fn, getattr(_lib, fn)(
        ctypes.byref(d), _ptr(q_nope), _ptr(q_rope), _ptr(w_uk), _ptr(w_uv), _ptr(cache), int(cache.shape[0]),
        _ptr(block_table), int(block_table.shape[1]), _ptr(seq_lens), batch, sq, float(softmax_scale), num_splits,
        _ptr(workspace), int(workspace.numel() * workspace.element_size()), _ptr(out), _ptr(lse), _ptr(status),
        _stream(stream)))


def mla_decode(d: MlaDims, q_nope, q_rope, w_uk, w_uv, cache, block_table, seq_lens, softmax_scale: float,
               workspace, out, lse=None, status=None, num_splits: int = 0, stream=None) -> None:
    """q_nope [batch, sq, n_heads, d_nope]; q_rope [batch, sq, n_heads, d_rope] (rotated);
    out [batch, sq, n_heads, d_nope] and optional lse [batch, sq, n_heads] float32 written.
    ``workspace`` is a byte tensor of at least mla_decode_workspace_bytes(d, batch, sq, num_splits)."""
    _decode_call("mla_decode", d, q_nope, q_rope, w_uk, w_uv, cache, block_table, seq_lens, softmax_scale,
                 workspace, out, lse, status, num_splits, stream)


def mla_decode_step_workspace_bytes(d: MlaDims, batch: int, sq: int, num_splits: int = 0) -> int:
    return int(_lib.mla_decode_step_workspace_bytes(ctypes.byref(d), batch, sq, num_splits))


def prepared_decode_step(d: MlaDims, h, w_dkv, w_kr, positions, q_nope, q_rope, w_uk, w_uv, cache, block_table,
                         seq_lens, softmax_scale: float, workspace, out, lse=None, status=None, num_splits: int = 0,
                         phases: int = MLA_PHASE_ALL, stream=None):
    """A decode step that appends its own sq tokens per sequence (mla_cache_append with t = sq, then
    mla_decode): arguments marshalled once into an mla_step_args; returns a zero-argument launcher of
    the given phases that keeps references to the tensors."""
    keep = (d, h, w_dkv, w_kr, positions, q_nope, q_rope, w_uk, w_uv, cache, block_table, seq_lens, workspace, out,
            lse, status)
    a = MlaStepArgs(_ptr(h), _ptr(w_dkv), _ptr(w_kr), _ptr(positions), _ptr(q_nope), _ptr(q_rope), _ptr(w_uk),
                    _ptr(w_uv), _ptr(cache), int(cache.shape[0]), _ptr(block_table), int(block_table.shape[1]),
                    _ptr(seq_lens), int(q_nope.shape[0]), int(q_nope.shape[1]), float(softmax_scale), num_splits,
                    _ptr(workspace), _nbytes(workspace), _ptr(out), _ptr(lse), _ptr(status))
    args = (ctypes.byref(d), ctypes.byref(a), phases, _stream(stream))

    def launch(_keep=keep, _a=a) -> None:
        _check("mla_decode_step", _lib.mla_decode_step(*args))
    return launch


def mla_decode_step(d: MlaDims, h, w_dkv, w_kr, positions, q_nope, q_rope, w_uk, w_uv, cache, block_table, seq_lens,
                    softmax_scale: float, workspace, out, lse=None, status=None, num_splits: int = 0,
                    phases: int = MLA_PHASE_ALL, stream=None) -> None:
    prepared_decode_step(d, h, w_dkv, w_kr, positions, q_nope, q_rope, w_uk, w_uv, cache, block_table, seq_lens,
                         softmax_scale, workspace, out, lse, status, num_splits, phases, stream)()


def mla_decode_noalloc(d: MlaDims, q_nope, q_rope, w_uk, w_uv, cache, block_table, seq_lens, softmax_scale: float,
                       out, lse=None, status=None, num_splits: int = 0, stream=None) -> None:
    """mla_decode without a workspace argument: the library's own per-GPU scratch array is used
    (shapes up to MLA_NOALLOC_SCRATCH_BYTES of workspace; calls that overlap on one GPU race)."""
    batch, sq = int(q_nope.shape[0]), int(q_nope.shape[1])
    _check("mla_decode_noalloc", _lib.mla_decode_noalloc(
        ctypes.byref(d), _ptr(q_nope), _ptr(q_rope), _ptr(w_uk), _ptr(w_uv), _ptr(cache), int(cache.shape[0]),
        _ptr(block_table), int(block_table.shape[1]), _ptr(seq_lens), batch, sq, float(softmax_scale), num_splits,
        _ptr(out), _ptr(lse), _ptr(status), _stream(stream)))


def mla_prefill(d: MlaDims, q_nope, q_rope, w_uk, w_uv, cache, block_table, seq_lens, softmax_scale: float,
                workspace, out, lse=None, status=None, stream=None) -> None:
    """Prefill attention for the last t tokens of each sequence.  q_nope [batch, t, n_heads, d_nope];
    q_rope [batch, t, n_heads, d_rope] (rotated); out [batch, t, n_heads, d_nope] and optional lse
    [batch, t, n_heads] float32 written.  ``workspace`` is a byte tensor of at least
    mla_prefill_workspace_bytes(d, batch, max_blocks)."""
    prepared_prefill("mla_prefill", d, q_nope, q_rope, w_uk, w_uv, cache, block_table, seq_lens, softmax_scale,
                     workspace, out, lse=lse, status=status, stream=stream)()


def prepared_prefill(fn_name: str, d: MlaDims, q_nope, q_rope, w_uk, w_uv, cache, block_table, seq_lens,
                     softmax_scale: float, workspace, out, lse=None, status=None, stream=None):
    """Marshal the arguments of ``fn_name`` (mla_prefill or one of its phases, mla_prefill_expand and
    mla_prefill_attend) once and return a zero-argument launcher; every launch still checks the return code.
    The launcher keeps references to the tensors, so their memory stays valid while it lives."""
    if fn_name not in ("mla_prefill", "mla_prefill_expand", "mla_prefill_attend"):
        raise ValueError(fn_name)
    batch, t = int(q_nope.shape[0]), int(q_nope.shape[1])
    fn = getattr(_lib, fn_name)
    keep = (d, q_nope, q_rope, w_uk, w_uv, cache, block_table, seq_lens, workspace, out, lse, status)
    args = (ctypes.byref(d), _ptr(q_nope), _ptr(q_rope), _ptr(w_uk), _ptr(w_uv), _ptr(cache), int(cache.shape[0]),
            _ptr(block_table), int(block_table.shape[1]), _ptr(seq_lens), batch, t, float(softmax_scale),
            _ptr(workspace), _nbytes(workspace), _ptr(out), _ptr(lse), _ptr(status), _stream(stream))

    def launch(_keep=keep) -> None:
        _check(fn_name, fn(*args))
    return launch


def mla_decode_prepare(d: MlaDims, q_nope, q_rope, w_uk, w_uv, cache, block_table, seq_lens, softmax_scale: float,
                       workspace, out, lse=None, status=None, num_splits: int = 0, stream=None) -> None:
    """First phase of mla_decode (absorbed queries and split plan); same arguments."""
    _decode_call("mla_decode_prepare", d, q_nope, q_rope, w_uk, w_uv, cache, block_table, seq_lens, softmax_scale,
                 workspace, out, lse, status, num_splits, stream)


def mla_decode_attend(d: MlaDims, q_nope, q_rope, w_uk, w_uv, cache, block_table, seq_lens, softmax_scale: float,
                      workspace, out, lse=None, status=None, num_splits: int = 0, stream=None) -> None:
    """Second phase of mla_decode (split-KV latent attention); same arguments."""
    _decode_call("mla_decode_attend", d, q_nope, q_rope, w_uk, w_uv, cache, block_table, seq_lens, softmax_scale,
                 workspace, out, lse, status, num_splits, stream)


def mla_decode_finish(d: MlaDims, q_nope, q_rope, w_uk, w_uv, cache, block_table, seq_lens, softmax_scale: float,
                      workspace, out, lse=None, status=None, num_splits: int = 0, stream=None) -> None:
    """Third phase of mla_decode (merge and W^UV up-projection); same arguments."""
    _decode_call("mla_decode_finish", d, q_nope, q_rope, w_uk, w_uv, cache, block_table, seq_lens, softmax_scale,
                 workspace, out, lse, status, num_splits, stream)


def prepared_cache_append(d: MlaDims, h, w_dkv, w_kr, positions, block_table, cache, workspace=None, status=None,
                          stream=None):
    """Marshal mla_cache_append's arguments once and return a zero-argument callable that launches it.
    For loops that reuse the same buffers: the per-call cost is one foreign call.  The callable keeps
    references to the tensors, so their memory stays valid while it lives."""
    fn = _lib.mla_cache_append
    keep = (d, h, w_dkv, w_kr, positions, block_table, cache, workspace, status)
    args = (ctypes.byref(d), _ptr(h), _ptr(w_dkv), _ptr(w_kr), _ptr(positions), _ptr(block_table),
            int(block_table.shape[1]), _ptr(cache), int(cache.shape[0]), int(h.shape[0]), int(h.shape[1]),
            _ptr(workspace), _nbytes(workspace), _ptr(status), _stream(stream))

    def launch(_keep=keep):
        rc = fn(*args)
        if rc != 0:
            raise MlaError("mla_cache_append", rc)
    return launch


def prepared_decode(fn_name: str, d: MlaDims, q_nope, q_rope, w_uk, w_uv, cache, block_table, seq_lens,
                    softmax_scale: float, workspace, out, lse=None, status=None, num_splits: int = 0, stream=None):
    """Marshal the arguments of ``fn_name`` (mla_decode or one of its phases) once and return a
    zero-argument callable that launches it; see prepared_cache_append."""
    if fn_name not in ("mla_decode", "mla_decode_prepare", "mla_decode_attend", "mla_decode_finish"):
        raise ValueError(fn_name)
    fn = getattr(_lib, fn_name)
    keep = (d, q_nope, q_rope, w_uk, w_uv, cache, block_table, seq_lens, workspace, out, lse, status)
    args = (ctypes.byref(d), _ptr(q_nope), _ptr(q_rope), _ptr(w_uk), _ptr(w_uv), _ptr(cache), int(cache.shape[0]),
            _ptr(block_table), int(block_table.shape[1]), _ptr(seq_lens), int(q_nope.shape[0]), int(q_nope.shape[1]),
            float(softmax_scale), num_splits, _ptr(workspace), int(workspace.numel() * workspace.element_size()),
            _ptr(out), _ptr(lse), _ptr(status), _stream(stream))

    def launch(_keep=keep):
        rc = fn(*args)
        if rc != 0:
            raise MlaError(fn_name, rc)
    return launch


def raw_library() -> ctypes.CDLL:
    """The loaded shared library (tests call its entry points directly)."""
    return _lib
