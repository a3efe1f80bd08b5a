"""The C-ABI library on the CPU: it loads, exports what the header declares,
and rejects bad arguments on the host before anything is launched."""
import ctypes
import os
import re

import pytest

from mla_rank_latent_amd import mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")


def test_exports_every_declared_function():
    decl = re.findall(r"^\s*(?:const\s+char\*|size_t|int)\s+(mla_\w+)\s*\(", open(HEADER).read(), re.M)
    assert sorted(decl) == sorted(mla.EXPORTS)
    lib = mla.raw_library()
    for name in decl:
        assert hasattr(lib, name), name


def test_one_hip_runtime_whatever_the_import_order():
    """Importing the binding before torch must not leave a second HIP runtime in
    the process (the library would then query and launch on a runtime that does
    not own torch's tensors and streams)."""
    import subprocess
    import sys
    code = ("from mla_rank_latent_amd import mla\n"
            "import torch\n"
            "maps = set(l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l)\n"
            "print(len(maps))\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    assert out.stdout.strip().splitlines()[-1] == "1", out.stdout


def test_status_strings():
    codes = [0, -1, -2, -3, -4, -5, -6, -7, -8, -9]
    strs = [mla.mla_status_str(c) for c in codes]
    assert len(set(strs)) == len(codes)
    assert mla.mla_status_str(-99) == "unknown status code"


def test_cache_bytes_accounting():
    v2 = mla.dims(128, 128, 64, 512, 5120)
    assert mla.mla_cache_bytes(v2, 1) == 576 * 2       # d_c + d_h^R elements in bf16
    assert mla.mla_cache_bytes(v2, 8192 * 64) == 8192 * 64 * 1152
    f32 = mla.dims(8, 16, 8, 32, 64, dtype="f32")
    assert mla.mla_cache_bytes(f32, 65) == 65 * 40 * 4
    assert mla.mla_cache_bytes(v2, -1) == 0
    bad = mla.dims(128, 128, 64, 512, 5120)
    bad.dtype = 7
    assert mla.mla_cache_bytes(bad, 10) == 0


def test_workspace_query():
    v2 = mla.dims(128, 128, 64, 512, 5120)
    w64 = mla.mla_decode_workspace_bytes(v2, 64, 1, 256)
    # q_lat + (256 + 64) pieces x 128 rows x (512 bf16 latent sums + 2 floats) + plan
    assert w64 >= 64 * 128 * 576 * 2 + 320 * 128 * (512 * 2 + 8)
    assert mla.mla_decode_workspace_bytes(v2, 64, 2, 128) > 0
    assert mla.mla_decode_workspace_bytes(v2, 64, 9, 128) == 0     # sq beyond the bf16 kernels
    assert mla.mla_decode_workspace_bytes(v2, 0, 1, 128) == 0
    odd = mla.dims(128, 96, 64, 512, 5120)
    assert mla.mla_decode_workspace_bytes(odd, 4, 1, 16) == 0      # bf16 widths are fixed


FAKE = 0x10000   # aligned, never dereferenced: every call below fails validation first


def _decode(d, **kw):
    a = dict(q_nope=FAKE, q_rope=FAKE, w_uk=FAKE, w_uv=FAKE, cache=FAKE, num_blocks=16, block_table=FAKE,
             max_blocks=4, seq_lens=FAKE, batch=4, sq=1, scale=0.1, num_splits=8, ws=FAKE, ws_bytes=1 << 40,
             out=FAKE, lse=None, status=None, stream=None)
    a.update(kw)
    return mla.raw_library().mla_decode(ctypes.byref(d), a["q_nope"], a["q_rope"], a["w_uk"], a["w_uv"], a["cache"],
                                        a["num_blocks"], a["block_table"], a["max_blocks"], a["seq_lens"],
                                        a["batch"], a["sq"], a["scale"], a["num_splits"], a["ws"], a["ws_bytes"],
                                        a["out"], a["lse"], a["status"], a["stream"])


def test_decode_argument_errors():
    v2 = mla.dims(128, 128, 64, 512, 5120)
    assert _decode(v2, q_nope=None) == -1
    assert _decode(v2, ws=None) == -1
    assert _decode(v2, batch=0) == -2
    assert _decode(v2, sq=0) == -2
    assert _decode(v2, sq=9) == -6
    assert _decode(v2, num_blocks=0) == -2
    assert _decode(v2, num_splits=-1) == -2
    assert _decode(v2, scale=float("nan")) == -2
    assert _decode(v2, cache=FAKE + 8) == -4
    assert _decode(v2, ws=FAKE + 16) == -4
    assert _decode(v2, ws_bytes=1024) == -5
    assert _decode(v2, batch=70000) == -6
    bad = mla.dims(128, 128, 64, 512, 5120)
    bad.dtype = 3
    assert _decode(bad) == -3
    assert _decode(mla.dims(128, 128, 64, 256, 5120)) == -8
    assert _decode(mla.dims(128, 128, 64, 512, 5120, block_size=32)) == -8
    assert _decode(mla.dims(8, 16, 7, 32, 64, dtype="f32")) == -2       # odd rotary width
    assert _decode(mla.dims(8, 16, 8, 2048, 64, dtype="f32")) == -6


def _prefill(d, fn="mla_prefill", **kw):
    a = dict(q_nope=FAKE, q_rope=FAKE, w_uk=FAKE, w_uv=FAKE, cache=FAKE, num_blocks=16, block_table=FAKE,
             max_blocks=4, seq_lens=FAKE, batch=2, t=100, scale=0.1, ws=FAKE, ws_bytes=1 << 40,
             out=FAKE, lse=None, status=None, stream=None)
    a.update(kw)
    return getattr(mla.raw_library(), fn)(
        ctypes.byref(d), a["q_nope"], a["q_rope"], a["w_uk"], a["w_uv"], a["cache"], a["num_blocks"],
        a["block_table"], a["max_blocks"], a["seq_lens"], a["batch"], a["t"], a["scale"], a["ws"], a["ws_bytes"],
        a["out"], a["lse"], a["status"], a["stream"])


def test_prefill_workspace_and_argument_errors():
    v2 = mla.dims(128, 128, 64, 512, 5120)
    # K^C and V^T of every token slot: 2 x batch x heads x (max_blocks x 64) x 128 bf16
    assert mla.mla_prefill_workspace_bytes(v2, 2, 4) == 2 * 2 * 128 * 256 * 128 * 2
    assert mla.mla_prefill_workspace_bytes(v2, 0, 4) == 0
    assert mla.mla_prefill_workspace_bytes(v2, 2, 0) == 0
    assert mla.mla_prefill_workspace_bytes(v2, 1, (1 << 17) + 1) == 0          # past 2^23 token slots
    assert mla.mla_prefill_workspace_bytes(mla.dims(8, 16, 8, 32, 64, dtype="f32"), 2, 4) == 0
    need = mla.mla_prefill_workspace_bytes(v2, 2, 4)
    for fn in ("mla_prefill", "mla_prefill_expand", "mla_prefill_attend"):
        assert _prefill(v2, fn, q_rope=None) == -1
        assert _prefill(v2, fn, ws=None) == -1
        assert _prefill(v2, fn, t=0) == -2
        assert _prefill(v2, fn, t=257) == -2                  # more queries than token slots
        assert _prefill(v2, fn, scale=float("inf")) == -2
        assert _prefill(v2, fn, scale=0.0) == -2
        assert _prefill(v2, fn, scale=-0.1) == -2
        assert _prefill(v2, fn, batch=0) == -2
        assert _prefill(v2, fn, out=FAKE + 4) == -4
        assert _prefill(v2, fn, ws=FAKE + 128) == -4
        # the phases need the whole batch's workspace; the whole call one sequence's worth
        per_seq = mla.mla_prefill_workspace_bytes(v2, 1, 4)
        assert _prefill(v2, fn, ws_bytes=(per_seq - 1) if fn == "mla_prefill" else need - 1) == -5
        assert _prefill(v2, fn, max_blocks=(1 << 17) + 1, num_blocks=1 << 18) == -6
        assert _prefill(mla.dims(8, 16, 8, 32, 64, dtype="f32"), fn) == -8
        assert _prefill(mla.dims(128, 128, 64, 512, 5120, block_size=32), fn) == -8


def test_layer_workspace_and_argument_errors():
    lib = mla.raw_library()
    v2 = mla.dims(128, 128, 64, 512, 5120)
    n = mla.mla_layer_workspace_bytes(v2, 1536, 64, 1)
    # at least the bf16 compressed query plus one fp32 copy of each projection's output
    assert n >= 64 * 1536 * 2 + 64 * 128 * 128 * 4
    assert n >= 64 * 5120 * 4
    assert mla.mla_layer_workspace_bytes(v2, 1000, 64, 1) == 0                 # d_qlat not a multiple of 64
    assert mla.mla_layer_workspace_bytes(mla.dims(128, 128, 64, 512, 5120 - 32), 1536, 64, 1) == 0
    assert mla.mla_layer_workspace_bytes(mla.dims(8, 16, 8, 32, 64, dtype="f32"), 1536, 1, 1) == 0
    assert mla.mla_layer_workspace_bytes(v2, 1536, 0, 1) == 0
    qc = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 1, FAKE, n, None]
    bad = list(qc)
    bad[0] = None
    assert lib.mla_q_compress(ctypes.byref(v2), 1536, *bad) == -1
    bad = list(qc)
    bad[10] = 1024           # far below what the call needs (every call here must fail before any launch)
    assert lib.mla_q_compress(ctypes.byref(v2), 1536, *bad) == -5
    bad = list(qc)
    bad[3] = FAKE + 2
    assert lib.mla_q_compress(ctypes.byref(v2), 1536, *bad) == -4
    assert lib.mla_q_compress(ctypes.byref(v2), 96, *qc) == -8
    assert lib.mla_q_compress(ctypes.byref(mla.dims(8, 16, 8, 32, 64, dtype="f32")), 1536, *qc) == -8
    op = [FAKE, FAKE, FAKE, 64, 1, FAKE, n, None]
    bad = list(op)
    bad[2] = None
    assert lib.mla_out_project(ctypes.byref(v2), *bad) == -1
    bad = list(op)
    bad[4] = 0
    assert lib.mla_out_project(ctypes.byref(v2), *bad) == -2
    bad = list(op)
    bad[6] = 1024
    assert lib.mla_out_project(ctypes.byref(v2), *bad) == -5


def test_append_and_qproj_argument_errors():
    lib = mla.raw_library()
    v2 = mla.dims(128, 128, 64, 512, 5120)
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 16, 2, 1, None, 0, None, None]
    assert lib.mla_cache_append(ctypes.byref(v2), *args[:4], None, *args[5:]) == -1
    bad_t = list(args)
    bad_t[9] = 0
    assert lib.mla_cache_append(ctypes.byref(v2), *bad_t) == -2
    mis = list(args)
    mis[0] = FAKE + 2
    assert lib.mla_cache_append(ctypes.byref(v2), *mis) == -4
    assert lib.mla_cache_append(ctypes.byref(mla.dims(128, 128, 64, 512, 5000)), *args) == -8
    need = lib.mla_cache_append_workspace_bytes(ctypes.byref(v2), 2, 1)
    assert need == 16 * 2 * 576 * 4                     # sixteen K slices of fp32 partial rows
    assert lib.mla_cache_append_workspace_bytes(ctypes.byref(v2), 0, 1) == 0
    # from 2048 rows the single-GEMM path runs and needs no workspace
    assert lib.mla_cache_append_workspace_bytes(ctypes.byref(v2), 1, 2047) == 16 * 2047 * 576 * 4
    assert lib.mla_cache_append_workspace_bytes(ctypes.byref(v2), 2, 1024) == 0
    assert lib.mla_cache_append_workspace_bytes(ctypes.byref(mla.dims(8, 16, 8, 32, 64, dtype="f32")), 2, 1) == 0
    ws_small = list(args)
    ws_small[10], ws_small[11] = FAKE, need - 1
    assert lib.mla_cache_append(ctypes.byref(v2), *ws_small) == -5
    ws_mis = list(args)
    ws_mis[10], ws_mis[11] = FAKE + 8, need
    assert lib.mla_cache_append(ctypes.byref(v2), *ws_mis) == -4
    q = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 1, None]
    assert lib.mla_q_project(ctypes.byref(v2), *q[:2], None, *q[3:]) == -1
    q2 = list(q)
    q2[6] = 0
    assert lib.mla_q_project(ctypes.byref(v2), *q2) == -2


class _FakeTensor:
    """Just enough of a tensor for the prepared launchers: a device address and a shape."""

    def __init__(self, addr, shape, itemsize=2):
        self.addr, self.shape, self.itemsize = addr, shape, itemsize

    def data_ptr(self):
        return self.addr

    def numel(self):
        n = 1
        for s in self.shape:
            n *= s
        return n

    def element_size(self):
        return self.itemsize


def test_prepared_launchers_check_on_every_call():
    v2 = mla.dims(128, 128, 64, 512, 5120)
    T = _FakeTensor
    q = T(FAKE, (2, 1, 128, 128))
    qr = T(FAKE, (2, 1, 128, 64))
    cache = T(FAKE, (16, 64, 576))
    bt = T(FAKE, (2, 8), 4)
    lens = T(FAKE, (2,), 4)
    ws = T(FAKE, (1024,), 1)            # far too small: the library refuses before launching
    out = T(FAKE, (2, 1, 128, 128))
    with pytest.raises(ValueError):
        mla.prepared_decode("mla_decode_everything", v2, q, qr, q, q, cache, bt, lens, 0.07, ws, out, stream=0)
    for fn in ("mla_decode", "mla_decode_prepare", "mla_decode_attend", "mla_decode_finish"):
        launch = mla.prepared_decode(fn, v2, q, qr, q, q, cache, bt, lens, 0.07, ws, out, num_splits=4, stream=0)
        for _ in range(2):
            with pytest.raises(mla.MlaError) as err:
                launch()
            assert err.value.code == -5
    h = T(FAKE, (2, 0, 5120))           # no tokens: rejected as bad dims
    append = mla.prepared_cache_append(v2, h, q, q, bt, bt, cache, stream=0)
    with pytest.raises(mla.MlaError) as err:
        append()
    assert err.value.code == -2


def test_fp8_cache_entry_points_on_the_host():
    """The FP8 cache type: its byte accounting, the quantise entry point's argument errors,
    append's required workspace, and which entry points take it (every call below fails
    validation before anything is launched)."""
    lib = mla.raw_library()
    v2 = mla.dims(128, 128, 64, 512, 5120)
    f8 = mla.dims(128, 128, 64, 512, 5120, dtype="bf16_fp8")
    page = mla.MLA_FP8_PAGE_BYTES
    assert page == 64 * (512 + 128 + 4)
    assert mla.mla_cache_bytes(f8, 1) == page and mla.mla_cache_bytes(f8, 64) == page
    assert mla.mla_cache_bytes(f8, 65) == 2 * page and mla.mla_cache_bytes(f8, 0) == 0
    assert mla.mla_cache_bytes(f8, 8192 * 64) == 8192 * 64 * 644   # 644 B per token against 1152

    def quant(d, src=FAKE, dst=FAKE, nb=4):
        return lib.mla_cache_quantize(ctypes.byref(d), src, dst, nb, None)
    assert quant(v2) == -3                      # the destination type must be the FP8 cache
    assert quant(f8, src=None) == -1
    assert quant(f8, dst=None) == -1
    assert quant(f8, nb=0) == -2
    assert quant(f8, dst=FAKE + 4) == -4
    assert quant(f8, src=FAKE + 8) == -4
    assert quant(f8, nb=1 << 25) == -6
    assert quant(mla.dims(128, 128, 64, 256, 5120, dtype="bf16_fp8")) == -8

    # append: staging rows (bf16, rounded up to 256 B) + the split path's partial products
    need = lib.mla_cache_append_workspace_bytes(ctypes.byref(f8), 2, 1)
    assert need == 2304 + 16 * 2 * 576 * 4
    assert lib.mla_cache_append_workspace_bytes(ctypes.byref(f8), 2, 1024) == 2048 * 1152   # GEMM path: staging only
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 16, 2, 1, None, 0, None, None]
    assert lib.mla_cache_append(ctypes.byref(f8), *args) == -5        # the workspace is required
    small = list(args)
    small[10], small[11] = FAKE, need - 1
    assert lib.mla_cache_append(ctypes.byref(f8), *small) == -5

    # decode takes the FP8 cache (same checks as bf16); prefill does not
    assert _decode(f8, ws_bytes=1024) == -5
    assert _decode(f8, sq=9) == -6
    assert _decode(f8, cache=FAKE + 8) == -4
    assert mla.mla_decode_workspace_bytes(f8, 64, 1, 256) == mla.mla_decode_workspace_bytes(v2, 64, 1, 256)
    assert _prefill(f8) == -8
    assert mla.mla_prefill_workspace_bytes(f8, 2, 4) == 0
    # the layer's projections take its bf16 tensors
    assert mla.mla_layer_workspace_bytes(f8, 1536, 64, 1) == mla.mla_layer_workspace_bytes(v2, 1536, 64, 1)


def test_prepared_launchers_keep_their_tensors_alive():
    """Every prepared launcher holds the tensors whose addresses it marshalled: a caller that
    drops its own references must not leave the launcher with freed memory.  The tensors
    are released once the launcher itself goes."""
    import gc
    import weakref
    v2 = mla.dims(128, 128, 64, 512, 5120)
    T = _FakeTensor

    def tensors(n):
        return [T(FAKE + 256 * i, (2, 1, 128, 128)) for i in range(n)]

    makers = {
        "q_compress": (8, lambda t: mla.prepared_q_compress(v2, 1536, t[0], t[1], t[2], t[3], t[4], t[5], t[6], t[7],
                                                            stream=0)),
        "out_project": (4, lambda t: mla.prepared_out_project(v2, t[0], t[1], t[2], t[3], stream=0)),
        "prefill": (10, lambda t: mla.prepared_prefill("mla_prefill", v2, t[0], t[1], t[2], t[3], t[4], t[5], t[6],
                                                       0.07, t[7], t[8], lse=t[9], stream=0)),
        "cache_append": (7, lambda t: mla.prepared_cache_append(v2, t[0], t[1], t[2], t[3], t[4], t[5], t[6],
                                                                stream=0)),
        "decode": (10, lambda t: mla.prepared_decode("mla_decode", v2, t[0], t[1], t[2], t[3], t[4], t[5], t[6],
                                                     0.07, t[7], t[8], lse=t[9], stream=0)),
    }
    for name, (n, make) in makers.items():
        ts = tensors(n)
        refs = [weakref.ref(t) for t in ts]
        launch = make(ts)
        del ts
        gc.collect()
        assert all(r() is not None for r in refs), name
        del launch
        gc.collect()
        assert all(r() is None for r in refs), name


def test_noalloc_decode_rejects_before_any_device_call():
    """mla_decode_noalloc checks its arguments, and that the shape's workspace fits its scratch
    array, on the host before it touches a device (these calls run without a GPU)."""
    lib = mla.raw_library()
    v2 = mla.dims(128, 128, 64, 512, 5120)

    def call(batch, sq, num_splits, q=FAKE, out=FAKE):
        return lib.mla_decode_noalloc(ctypes.byref(v2), q, FAKE, FAKE, FAKE, FAKE, 64, FAKE, 16, FAKE, batch, sq,
                                      0.07, num_splits, out, None, None, None)

    assert call(4, 1, 8, q=None) == -1
    assert call(4, 1, 8, out=None) == -1
    assert call(4, 9, 8) == -6                     # more query tokens than the kernels take
    need = mla.mla_decode_workspace_bytes(v2, 4096, 1, 64)
    assert need > mla.MLA_NOALLOC_SCRATCH_BYTES
    assert call(4096, 1, 64) == -9                 # its workspace would not fit the scratch array
    assert "scratch" in mla.mla_status_str(-9)
    # the decode benchmark's shape fits (batch 64, 128 heads, one query token, 256 ranges)
    assert mla.mla_decode_workspace_bytes(v2, 64, 1, 256) <= mla.MLA_NOALLOC_SCRATCH_BYTES


def test_decode_step_rejects_before_any_launch():
    """mla_decode_step checks the append's and decode's arguments and its workspace on the host
    before anything is launched (these calls run without a GPU)."""
    lib = mla.raw_library()
    v2 = mla.dims(128, 128, 64, 512, 5120)
    n = mla.mla_decode_step_workspace_bytes(v2, 2, 1, 8)
    assert n >= mla.mla_decode_workspace_bytes(v2, 2, 1, 8) + mla.mla_cache_append_workspace_bytes(v2, 2, 1)
    assert mla.mla_decode_step_workspace_bytes(mla.dims(128, 128, 64, 512, 5120, dtype="bf16_fp8"), 2, 1, 8) == 0
    assert mla.mla_decode_step_workspace_bytes(v2, 2, 9, 8) == 0

    def args(**kw):
        f = dict(h=FAKE, w_dkv=FAKE, w_kr=FAKE, positions=FAKE, q_nope=FAKE, q_rope=FAKE, w_uk=FAKE, w_uv=FAKE,
                 cache=FAKE, num_blocks=64, block_table=FAKE, max_blocks=16, seq_lens=FAKE, batch=2, sq=1,
                 softmax_scale=0.07, num_splits=8, workspace=FAKE, workspace_bytes=n, out=FAKE, lse=None, status=None)
        f.update(kw)
        return mla.MlaStepArgs(**f)

    def call(a, d=v2, phases=7):
        return lib.mla_decode_step(ctypes.byref(d), ctypes.byref(a), phases, None)

    assert lib.mla_decode_step(ctypes.byref(v2), None, 7, None) == -1
    assert call(args(h=None)) == -1
    assert call(args(q_nope=None)) == -1
    assert call(args(workspace=None)) == -1
    assert call(args(), phases=0) == -2 and call(args(), phases=8) == -2
    assert call(args(sq=0)) == -2
    assert call(args(sq=9)) == -6
    assert call(args(h=FAKE + 4)) == -4
    assert call(args(out=FAKE + 4)) == -4
    assert call(args(workspace=FAKE + 128)) == -4
    assert call(args(workspace_bytes=n - 1)) == -5
    assert call(args(), d=mla.dims(128, 128, 64, 512, 5120, dtype="bf16_fp8")) == -8
    assert call(args(), d=mla.dims(8, 16, 8, 32, 64, dtype="f32")) == -8
