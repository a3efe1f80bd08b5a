"""Benchmark of the MLA decode hot path on one MI355X.

One step = one pass of the whole hot path over one batch: append of the new
token of every sequence (down-projection, RoPE, paged write), then decode
(absorbed queries, split-KV latent attention, log-sum-exp merge, W^UV
up-projection).  Default workload: batch 64, every sequence at context 8192
after the append, 128 heads, DeepSeek-V2 widths, bf16 cache in 64-token
blocks with a randomly permuted block table (seeded synthetic data).

Prints one JSON line.  ``value`` is the whole step's algorithmic HBM
throughput (bytes every step must move / step time).  ``roofline`` rates the
dominant kernel (the split-KV attention) against the MI355X HBM peak, timed
with HIP events around each of its launches on the stream it runs on.
``cpu_baseline`` times the fp64 oracle on the host over a bounded sample of
the same workload.

``--workload v2_b64_ctx8192_paged_append_fp8`` runs the same step with the
cache in FP8 pages (E4M3 codes, a per-token power-of-two scale, bf16 rotary
key: 644 B per token), quantised on the GPU from the generated bf16 cache
before the timed region; its algorithmic bytes count 644 B per cached and
appended token.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, vendor figure
ROOT = os.path.dirname(os.path.abspath(__file__))


FP8_SUFFIX = "_fp8"   # a decode workload with its cache in FP8 pages
_COMMON_SOURCES = ("mla_rank_latent_amd/csrc/attn_common.h", "mla_rank_latent_amd/csrc/device_util.h",
                   "mla_rank_latent_amd/csrc/mla_internal.h")
# The counter profile of each decode workload's attention kernel (HBM traffic from FETCH_SIZE and
# WRITE_SIZE, MFMA busy cycles), and the sources it was taken from.
_BF16_SOURCES = ("mla_rank_latent_amd/csrc/attn_bf16.hip",) + _COMMON_SOURCES
COUNTER_PROFILES = {
    "v2_b64_ctx8192_paged_append": ("attn_bf16_b64_ctx8192_counters.md", _BF16_SOURCES),
    "v2_b1_ctx4096": ("attn_bf16_b1_ctx4096_counters.md", _BF16_SOURCES),
    "v2_b4_longctx_128k": ("attn_bf16_b4_longctx_counters.md", _BF16_SOURCES),
    "v2_b128_ragged_sq2": ("attn_bf16_b128_ragged_sq2_counters.md", _BF16_SOURCES),
    "v2_b64_ctx8192_paged_append_fp8": ("attn_fp8_b64_ctx8192_counters.md",
                                        ("mla_rank_latent_amd/csrc/attn_fp8.hip",) + _COMMON_SOURCES),
}


def code_text(text: str) -> str:
    """C++/HIP source without its comments and with whitespace runs collapsed: what the
    compiler sees, so that a comment edit does not retire a counter profile."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def sources_sha256(sources) -> str:
    """sha256 over the code (comments and whitespace aside) of the given source files."""
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode("utf-8"))
    return h.hexdigest()


def measured_counters(workload: str) -> dict:
    """Figures per attention launch from the committed counter profile of this workload:
    ``traffic`` (HBM bytes, FETCH_SIZE and WRITE_SIZE scaled by a copy kernel's reading) and
    ``mfma_busy`` (rocprofv3's MfmaUtil / 100: SQ_VALU_MFMA_BUSY_CYCLES summed over the SIMDs, over
    the largest GRBM_GUI_ACTIVE times the SIMD count; mean of the timed dispatches).  Empty when
    there is no profile or the attention sources changed since the counters were taken."""
    if workload not in COUNTER_PROFILES:
        return {}
    name, sources = COUNTER_PROFILES[workload]
    try:
        text = open(os.path.join(ROOT, "profiles", name), encoding="utf-8").read()
    except OSError:
        return {}
    fields = dict(re.findall(r"^- ([a-z0-9_]+): (\S+)$", text, flags=re.M))
    if fields.get("workload") != workload or fields.get("attention_sources_sha256") != sources_sha256(sources):
        return {}
    out = {}
    if "traffic_bytes_per_launch" in fields:
        out["traffic"] = int(fields["traffic_bytes_per_launch"])
    if "mfma_busy_frac" in fields:
        out["mfma_busy"] = float(fields["mfma_busy_frac"])
    return out


def host_info() -> dict:
    """The host's CPU model, numpy's BLAS backend and the threads it uses."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo", encoding="utf-8"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas, threads = "unknown", os.cpu_count() or 1
    try:
        import numpy  # noqa: F401  (loads the BLAS library threadpoolctl inspects)
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            blas = f"{info[0].get('internal_api')} {info[0].get('version')}"
            threads = max(i.get("num_threads", 1) for i in info)
    except Exception:
        pass
    return {"cpu_model": model, "blas": blas, "threads": int(threads)}


MALL_BYTES = 256 * 1024 * 1024   # MI355X last-level (Infinity) cache


def rotation_copies(rotate: int, step_bytes: int) -> int:
    """Input copies a timed run cycles through.  rotate > 0: that many.  0 (auto): enough that
    between two uses of one copy the other copies move at least twice the last-level cache,
    so no step finds what it reads still cached from an earlier step."""
    if rotate > 0:
        return rotate
    k = 1
    while (k - 1) * step_bytes < 2 * MALL_BYTES:
        k += 1
    return max(k, 2)


def workload_bytes_flops(spec, seq_lens, fp8: bool = False):
    """Algorithmic bytes and flops of one step, with their parts.  fp8: the cache holds, per token, d_c
    E4M3 codes, the bf16 rotary key and one fp32 scale (644 B for DeepSeek-V2's widths)."""
    H, dn, dr, dc, d = spec.n_heads, spec.d_nope, spec.d_rope, spec.d_latent, spec.d_model
    R = dc + dr
    e = 2 if spec.dtype == "bf16" else 4
    row = dc + 2 * dr + 4 if fp8 else R * e                 # cache bytes per token
    tokens = int(sum(int(L) for L in seq_lens))
    B, S = spec.batch, spec.sq
    cache = tokens * row                                    # every cached row read once
    weights_dec = 2 * H * dn * dc * e                       # W^UK and W^UV
    q_bytes = B * S * H * (dn + dr) * e
    out_bytes = B * S * H * dn * e
    append_bytes = 0
    append_flops = 0
    if spec.append:
        append_bytes = (R * d + B * S * d) * e + B * S * row   # W^DKV, W^KR, h, written rows
        append_flops = 2 * B * S * R * d
    # scores over [c | k^R] (576) and the latent weighted sum (512) per visible token and query row
    vis = 0
    for L in seq_lens:
        for s in range(S):
            vis += max(0, int(L) - S + s + 1)
    attn_flops = 2 * H * vis * (R + dc)
    proj_flops = 2 * 2 * B * S * H * dn * dc                # absorption and up-projection
    total_bytes = cache + weights_dec + q_bytes + out_bytes + append_bytes
    total_flops = attn_flops + proj_flops + append_flops
    return dict(bytes=total_bytes, flops=total_flops, cache_bytes=cache, attn_flops=attn_flops, tokens=tokens,
                row_bytes=row)


def prefill_flops(spec, seq_lens):
    """Algorithmic flops of one prefill step: the append of the t new rows, the expansion of
    every context token into per-head K^C and V, and causal attention (scores over 192
    features and values of 128 per visible (query, key) pair and head)."""
    H, dn, dr, dc, d = spec.n_heads, spec.d_nope, spec.d_rope, spec.d_latent, spec.d_model
    T = spec.sq
    tokens = int(sum(int(L) for L in seq_lens))
    pairs = 0
    for L in seq_lens:
        L = int(L)
        pairs += sum(max(0, L - T + s + 1) for s in range(T))
    append = 2 * spec.batch * T * (dc + dr) * d
    expand = 2 * 2 * tokens * H * dn * dc
    attn = 2 * H * pairs * (dn + dr + dn)
    return dict(total=append + expand + attn, append=append, expand=expand, attn=attn, pairs=pairs)


def cpu_baseline_prefill(x, budget_s: float):
    """Time the fp64 oracle on the prefill workload: the appended rows, then whole heads
    (every query of the sequence) until ``budget_s`` is spent; TFLOP/s of the same
    algorithmic flops (the append counted once, expansion and attention per head)."""
    import numpy as np
    from mla_rank_latent_amd import synth
    from oracle import mla_oracle
    hi = host_info()
    threads = hi["threads"]
    spec = x["spec"]
    bs = spec.block_size
    L = int(x["seq_lens"][0])
    nblk = (L + bs - 1) // bs
    t0 = time.perf_counter()
    rows = mla_oracle.cache_rows(synth.as_float(x["h"][:1], spec.dtype), synth.as_float(x["w_dkv"], spec.dtype),
                                 synth.as_float(x["w_kr"], spec.dtype), x["positions"][:1], spec.rope_base, spec.dtype)
    sub = synth.as_float(x["pool"][x["block_table"][0, :nblk]], spec.dtype)
    for t, p in enumerate(x["positions"][0]):
        sub[p // bs, p % bs] = rows[0, t]
    spent = time.perf_counter() - t0
    qn, qr = synth.as_float(x["q_nope"][:1], spec.dtype), synth.as_float(x["q_rope"][:1], spec.dtype)
    w_uk, w_uv = synth.as_float(x["w_uk"], spec.dtype), synth.as_float(x["w_uv"], spec.dtype)
    heads = 0
    for hh in range(spec.n_heads):
        t0 = time.perf_counter()
        mla_oracle.decode(qn, qr, w_uk, w_uv, sub, np.arange(nblk)[None, :], [L], x["scale"], bs, heads=[hh])
        spent += time.perf_counter() - t0
        heads += 1
        if spent >= budget_s:
            break
    f = prefill_flops(spec, x["seq_lens"][:1])
    done = f["append"] / spec.batch + (f["expand"] + f["attn"]) / spec.batch * heads / spec.n_heads
    return {"value": round(done / spent / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": hi["cpu_model"], "blas": hi["blas"],
            "sample": f"sequence 0: its {spec.sq} appended rows and {heads} of {spec.n_heads} heads (every query) "
                      f"in {spent:.1f} s; fp64 numpy; TFLOP/s of the same algorithmic flops"}


def run_prefill(args, spec, x) -> int:
    """Prefill leg: one step = append of the t new rows of every sequence, expansion of the
    context into per-head K^C and V, causal attention of the t queries."""
    import torch
    from mla_rank_latent_amd import mla

    def dev(a):
        import numpy as np
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    d = mla.dims(spec.n_heads, spec.d_nope, spec.d_rope, spec.d_latent, spec.d_model, spec.block_size, spec.dtype,
                 spec.rope_base)
    pool, bt, lens = dev(x["pool"]), dev(x["block_table"]), dev(x["seq_lens"])
    w_uk, w_uv = dev(x["w_uk"]), dev(x["w_uv"])
    qn, qr = dev(x["q_nope"]), dev(x["q_rope"])
    h, w_dkv, w_kr, pos = dev(x["h"]), dev(x["w_dkv"]), dev(x["w_kr"]), dev(x["positions"])
    out = torch.empty(spec.batch, spec.sq, spec.n_heads, spec.d_nope, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(spec.batch, spec.sq, spec.n_heads, dtype=torch.float32, device="cuda")
    ws = torch.empty(mla.mla_prefill_workspace_bytes(d, spec.batch, int(bt.shape[1])), dtype=torch.uint8,
                     device="cuda")
    n_ws = mla.mla_cache_append_workspace_bytes(d, int(h.shape[0]), int(h.shape[1]))
    append_ws = torch.empty(n_ws, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    append = mla.prepared_cache_append(d, h, w_dkv, w_kr, pos, bt, pool, workspace=append_ws, stream=stream)
    pargs = (d, qn, qr, w_uk, w_uv, pool, bt, lens, x["scale"], ws, out)
    expand = mla.prepared_prefill("mla_prefill_expand", *pargs, lse=lse, stream=stream)
    attend = mla.prepared_prefill("mla_prefill_attend", *pargs, lse=lse, stream=stream)

    def step(ev_a=None, ev_b=None):
        append()
        expand()
        if ev_a is not None:
            ev_a.record(stream)
        attend()
        if ev_b is not None:
            ev_b.record(stream)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        step(ev_a[i], ev_b[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / args.steps
    ms_attn = sum(a.elapsed_time(b) for a, b in zip(ev_a, ev_b)) / args.steps
    print(f"[bench] {args.steps} steps: {ms_step * 1e3:.1f} us/step (wall {wall / args.steps * 1e6:.1f} us), "
          f"attention {ms_attn * 1e3:.1f} us", file=sys.stderr, flush=True)

    f = prefill_flops(spec, x["seq_lens"])
    step_s = ms_step * 1e-3
    tflops = f["total"] / step_s / 1e12
    attn_tflops = f["attn"] / (ms_attn * 1e-3) / 1e12
    res = {
        "metric": "MLA prefill TFLOP/s (% of bf16 MFMA peak), tokens/s; B=1 ctx=8K 128 heads, every token a query",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic (seeded N(0,1) queries/hidden states, N(0,1/fan_in) weights)",
        "config": {"workload": spec.name, "batch": spec.batch, "context": int(max(x["seq_lens"])),
                   "query_tokens": spec.sq, "heads": spec.n_heads, "d_latent": spec.d_latent,
                   "d_rope": spec.d_rope, "d_nope": spec.d_nope, "d_model": spec.d_model,
                   "block_size": spec.block_size, "paged": spec.paged, "append": spec.append},
        "tokens_per_s": round(spec.batch * spec.sq / step_s, 1),
        "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "step_flops": f["total"],
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "prefill_attn_bf16_kernel", "kernel_us": round(ms_attn * 1e3, 2),
                     "flops_per_launch": f["attn"]},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print(f"[bench] cpu baseline (oracle, ~{args.cpu_budget:.0f} s)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline_prefill(x, args.cpu_budget)
    print(json.dumps(res), flush=True)
    return 0


def layer_extra(spec):
    """Bytes and flops the full layer adds to a decode step: W^DQ, W^UQ, W^QR and W^O,
    and the output u (the hidden states are already counted by the append)."""
    H, dn, dr, d, dq = spec.n_heads, spec.d_nope, spec.d_rope, spec.d_model, spec.d_qlat
    M = spec.batch * spec.sq
    w = (dq * d + H * (dn + dr) * dq + d * H * dn) * 2
    flops = 2 * M * (dq * d + H * (dn + dr) * dq + d * H * dn)
    return dict(bytes=w + M * d * 2, flops=flops)


def run_layer(args, spec, x) -> int:
    """Full-layer decode step: append, compressed queries, decode (three phases), W^O."""
    import torch
    from mla_rank_latent_amd import mla

    def dev(a):
        import numpy as np
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    d = mla.dims(spec.n_heads, spec.d_nope, spec.d_rope, spec.d_latent, spec.d_model, spec.block_size, spec.dtype,
                 spec.rope_base)
    B, S = spec.batch, spec.sq
    pool, bt, lens = dev(x["pool"]), dev(x["block_table"]), dev(x["seq_lens"])
    w_uk, w_uv = dev(x["w_uk"]), dev(x["w_uv"])
    h, w_dkv, w_kr, pos = dev(x["h"]), dev(x["w_dkv"]), dev(x["w_kr"]), dev(x["positions"])
    w_dq, w_uq, w_qr, w_o = dev(x["w_dq"]), dev(x["w_uq"]), dev(x["w_qr_c"]), dev(x["w_o"])
    q_pos = dev(x["q_positions"])
    h_q = h[:, -S:].contiguous()
    qn = torch.empty(B, S, spec.n_heads, spec.d_nope, dtype=torch.bfloat16, device="cuda")
    qr = torch.empty(B, S, spec.n_heads, spec.d_rope, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(B, S, spec.n_heads, spec.d_nope, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, S, spec.n_heads, dtype=torch.float32, device="cuda")
    u = torch.empty(B, S, spec.d_model, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mla.mla_decode_workspace_bytes(d, B, S, args.num_splits), dtype=torch.uint8, device="cuda")
    lws = torch.empty(mla.mla_layer_workspace_bytes(d, spec.d_qlat, B, S), dtype=torch.uint8, device="cuda")
    n_ws = mla.mla_cache_append_workspace_bytes(d, int(h.shape[0]), int(h.shape[1]))
    append_ws = torch.empty(n_ws, dtype=torch.uint8, device="cuda") if n_ws else None
    stream = torch.cuda.current_stream()
    append = mla.prepared_cache_append(d, h, w_dkv, w_kr, pos, bt, pool, workspace=append_ws, stream=stream)
    qcomp = mla.prepared_q_compress(d, spec.d_qlat, h_q, w_dq, w_uq, w_qr, q_pos, qn, qr, lws, stream=stream)
    dec_args = (d, qn, qr, w_uk, w_uv, pool, bt, lens, x["scale"], ws, out)
    phase = {name: mla.prepared_decode(name, *dec_args, lse=lse, num_splits=args.num_splits, stream=stream)
             for name in ("mla_decode_prepare", "mla_decode_attend", "mla_decode_finish")}
    oproj = mla.prepared_out_project(d, out, w_o, u, lws, stream=stream)

    def step(ev_a=None, ev_b=None):
        append()
        qcomp()
        phase["mla_decode_prepare"]()
        if ev_a is not None:
            ev_a.record(stream)
        phase["mla_decode_attend"]()
        if ev_b is not None:
            ev_b.record(stream)
        phase["mla_decode_finish"]()
        oproj()

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        step(ev_a[i], ev_b[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / args.steps
    ms_attn = sum(a.elapsed_time(b) for a, b in zip(ev_a, ev_b)) / args.steps
    print(f"[bench] {args.steps} steps: {ms_step * 1e3:.1f} us/step (wall {wall / args.steps * 1e6:.1f} us), "
          f"attention {ms_attn * 1e3:.1f} us", file=sys.stderr, flush=True)

    wl = workload_bytes_flops(spec, x["seq_lens"])
    ex = layer_extra(spec)
    # decode's bytes (cache, W^UK/W^UV, queries, o) plus the layer's weights and its output u
    step_bytes = wl["bytes"] + ex["bytes"]
    step_flops = wl["flops"] + ex["flops"]
    step_s = ms_step * 1e-3
    gbs = step_bytes / step_s / 1e9
    attn_gbs = wl["cache_bytes"] / (ms_attn * 1e-3) / 1e9
    attn_tflops = wl["attn_flops"] / (ms_attn * 1e-3) / 1e12
    res = {
        "metric": "MLA full-layer decode GB/s (% roofline), tokens/s; B=64 ctx=8K 128 heads, d'_c=1536",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic (seeded N(0,1) cache/hidden states, N(0,1/fan_in) weights)",
        "config": {"workload": spec.name, "batch": B, "context": int(max(x["seq_lens"])), "query_tokens": S,
                   "heads": spec.n_heads, "d_latent": spec.d_latent, "d_rope": spec.d_rope, "d_nope": spec.d_nope,
                   "d_model": spec.d_model, "d_qlat": spec.d_qlat, "block_size": spec.block_size,
                   "paged": spec.paged, "append": spec.append, "num_splits": args.num_splits or "auto"},
        "tflops": round(step_flops / step_s / 1e12, 2),
        "tokens_per_s": round(B * S / step_s, 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "step_bytes": step_bytes,
        "step_flops": step_flops,
        "roofline": {"bound": "hbm", "achieved": round(attn_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(attn_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "attn_bf16_kernel", "kernel_us": round(ms_attn * 1e3, 2),
                     "bytes_per_launch": wl["cache_bytes"], "mfma_tflops": round(attn_tflops, 2)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print(f"[bench] cpu baseline (oracle, ~{args.cpu_budget:.0f} s)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline_layer(x, args.cpu_budget, step_bytes)
    print(json.dumps(res), flush=True)
    return 0


def cpu_baseline_layer(x, budget_s: float, step_bytes: int):
    """The fp64 oracle on whole sequences of the layer workload (appended row, compressed
    queries, decode over all heads, W^O) until ``budget_s`` is spent; GB/s of the step's bytes
    in proportion to the sequences done."""
    import numpy as np
    from mla_rank_latent_amd import synth
    from oracle import mla_oracle
    hi = host_info()
    threads = hi["threads"]
    spec = x["spec"]
    bs = spec.block_size
    f = lambda k: synth.as_float(x[k], spec.dtype)
    w_uk, w_uv, w_dq, w_uq, w_qr, w_o = f("w_uk"), f("w_uv"), f("w_dq"), f("w_uq"), f("w_qr_c"), f("w_o")
    w_dkv, w_kr = f("w_dkv"), f("w_kr")
    done, spent = 0, 0.0
    for b in range(spec.batch):
        L = int(x["seq_lens"][b])
        nblk = (L + bs - 1) // bs
        sub = synth.as_float(x["pool"][x["block_table"][b, :nblk]], spec.dtype)
        t0 = time.perf_counter()
        hb = synth.as_float(x["h"][b:b + 1], spec.dtype)
        rows = mla_oracle.cache_rows(hb, w_dkv, w_kr, x["positions"][b:b + 1], spec.rope_base, spec.dtype)
        for t, p in enumerate(x["positions"][b]):
            sub[p // bs, p % bs] = rows[0, t]
        qn, qr = mla_oracle.layer_queries(hb[:, -spec.sq:], w_dq, w_uq, w_qr, x["q_positions"][b:b + 1],
                                          spec.n_heads, spec.rope_base)
        o, _ = mla_oracle.decode(qn, qr, w_uk, w_uv, sub, np.arange(nblk)[None, :], [L], x["scale"], bs)
        mla_oracle.out_project(o, w_o)
        spent += time.perf_counter() - t0
        done += 1
        if spent >= budget_s:
            break
    value = step_bytes * done / spec.batch / spent / 1e9
    return {"value": round(value, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": hi["cpu_model"], "blas": hi["blas"],
            "sample": f"{done} of {spec.batch} sequences (append, compressed queries, all {spec.n_heads} heads, "
                      f"W^O) in {spent:.1f} s; fp64 numpy, non-absorbed; GB/s of the same algorithmic bytes"}


def cpu_baseline(x, budget_s: float, fp8: bool = False):
    """Time the fp64 oracle (as it stands) on whole sequences of the workload until
    ``budget_s`` of CPU work has been spent; scale to GB/s of the same algorithmic bytes.
    fp8: the oracle also quantises each sequence's blocks (and its appended row) and
    decodes the dequantised values, as the FP8 cache stands for them."""
    import numpy as np
    from mla_rank_latent_amd import synth
    from oracle import mla_oracle
    hi = host_info()
    threads = hi["threads"]
    spec = x["spec"]
    bs = spec.block_size
    qn, qr = synth.as_float(x["q_nope"], spec.dtype), synth.as_float(x["q_rope"], spec.dtype)
    w_uk, w_uv = synth.as_float(x["w_uk"], spec.dtype), synth.as_float(x["w_uv"], spec.dtype)
    done, spent = 0, 0.0
    for b in range(spec.batch):
        L = int(x["seq_lens"][b])
        nblk = (L + bs - 1) // bs
        sub = synth.as_float(x["pool"][x["block_table"][b, :nblk]], spec.dtype)
        t0 = time.perf_counter()
        if fp8:
            codes, scales, rope = mla_oracle.quantize_rows(sub, spec.d_latent)
            sub = mla_oracle.dequantize_rows(codes, scales, rope)
        if spec.append:
            rows = mla_oracle.cache_rows(synth.as_float(x["h"][b:b + 1], spec.dtype),
                                         synth.as_float(x["w_dkv"], spec.dtype), synth.as_float(x["w_kr"], spec.dtype),
                                         x["positions"][b:b + 1], spec.rope_base, spec.dtype)
            if fp8:
                rows = mla_oracle.dequantize_rows(*mla_oracle.quantize_rows(rows, spec.d_latent))
            for t, p in enumerate(x["positions"][b]):
                sub[p // bs, p % bs] = rows[0, t]
        mla_oracle.decode(qn[b:b + 1], qr[b:b + 1], w_uk, w_uv, sub, np.arange(nblk)[None, :], [L], x["scale"], bs)
        spent += time.perf_counter() - t0
        done += 1
        if spent >= budget_s:
            break
    # the sampled sequences are `done` of `batch`; weights are counted in proportion
    wb = workload_bytes_flops(spec, x["seq_lens"], fp8)["bytes"]
    value = wb * done / spec.batch / spent / 1e9
    what = ", FP8 quantise/dequantise included" if fp8 else ""
    return {"value": round(value, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": hi["cpu_model"], "blas": hi["blas"],
            "sample": f"{done} of {spec.batch} sequences (all {spec.n_heads} heads, full context, append included"
                      f"{what}) in {spent:.1f} s; fp64 numpy, non-absorbed; GB/s of the same algorithmic bytes"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", default="v2_b64_ctx8192_paged_append")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--rotate", type=int, default=0,
                    help="input copies cycled through by the steps (0: enough that every step reads cold inputs)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB streaming kernel (to calibrate HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library runs the hot path on a single MI355X and has no "
              f"multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        return 2

    import torch
    from mla_rank_latent_amd import mla, synth

    if args.copy_calibration:
        # a plain streaming kernel of known size (dst = src * 1 over 2^28 floats): it reads 2^30 bytes and
        # writes 2^30 bytes per dispatch; a device-to-device copy_ may run on a DMA engine instead
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_dispatch": 1 << 30, "dispatches": 3}), flush=True)
        return 0

    prefill, layer = synth.prefill_presets(), synth.layer_presets()
    fp8 = args.workload.endswith(FP8_SUFFIX)
    base = args.workload[:-len(FP8_SUFFIX)] if fp8 else args.workload
    spec = {**synth.presets(), **prefill, **layer}[base]
    if fp8 and base not in synth.presets():
        print(f"bench.py: the FP8 cache applies to the decode workloads, not {base}", file=sys.stderr)
        return 2
    print(f"[bench] generating {spec.name} (seed {spec.seed})", file=sys.stderr, flush=True)
    x = synth.make_inputs(spec)
    if args.workload in prefill:
        return run_prefill(args, spec, x)
    if args.workload in layer:
        return run_layer(args, spec, x)

    def dev(a):
        import numpy as np
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    d = mla.dims(spec.n_heads, spec.d_nope, spec.d_rope, spec.d_latent, spec.d_model, spec.block_size,
                 "bf16_fp8" if fp8 else spec.dtype, spec.rope_base)
    wl = workload_bytes_flops(spec, x["seq_lens"], fp8)
    copies = rotation_copies(args.rotate, wl["bytes"])
    print(f"[bench] {copies} input copies in rotation ({wl['bytes'] / 1e6:.1f} MB read per step)", file=sys.stderr,
          flush=True)
    bt, lens = dev(x["block_table"]), dev(x["seq_lens"])
    tdt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
    out = torch.empty(spec.batch, spec.sq, spec.n_heads, spec.d_nope, dtype=tdt, device="cuda")
    lse = torch.empty(spec.batch, spec.sq, spec.n_heads, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    has_append = spec.append
    # a bf16 step that appends its own tokens runs as mla_decode_step (the append's partial
    # products, the absorbed queries and the split plan in one launch); the FP8 cache appends
    # with mla_cache_append, then decodes
    fused = has_append and not fp8
    if fused:
        ws = torch.empty(mla.mla_decode_step_workspace_bytes(d, spec.batch, spec.sq, args.num_splits),
                         dtype=torch.uint8, device="cuda")
    else:
        ws = torch.empty(mla.mla_decode_workspace_bytes(d, spec.batch, spec.sq, args.num_splits), dtype=torch.uint8,
                         device="cuda")
    append_ws = None
    if has_append:
        n_ws = mla.mla_cache_append_workspace_bytes(d, spec.batch, spec.sq)
        append_ws = torch.empty(n_ws, dtype=torch.uint8, device="cuda") if n_ws and not fused else None
        pos = dev(x["positions"])

    # Every copy holds its own cache, queries, weights and hidden states (each step reads one
    # copy, so nothing a step reads is still in the caches from the step before); arguments are
    # marshalled once per copy, so a step costs the host four foreign calls.
    sets = []
    base = None
    for k in range(copies):
        if k == 0:
            pool = dev(x["pool"])
            if fp8:
                # the cache in FP8 pages, quantised on the GPU from the generated bf16 cache
                pages = torch.empty(pool.shape[0], mla.MLA_FP8_PAGE_BYTES, dtype=torch.uint8, device="cuda")
                mla.mla_cache_quantize(d, pool, pages)
                torch.cuda.synchronize()
                pool = pages
            t = dict(pool=pool, w_uk=dev(x["w_uk"]), w_uv=dev(x["w_uv"]), qn=dev(x["q_nope"]), qr=dev(x["q_rope"]))
            if has_append:
                t.update(h=dev(x["h"]), w_dkv=dev(x["w_dkv"]), w_kr=dev(x["w_kr"]))
            base = t
        else:
            t = {key: v.clone() for key, v in base.items()}
        launches = []
        if fused:
            for ph in (mla.MLA_PHASE_PREPARE, mla.MLA_PHASE_ATTEND, mla.MLA_PHASE_FINISH):
                launches.append(mla.prepared_decode_step(d, t["h"], t["w_dkv"], t["w_kr"], pos, t["qn"], t["qr"],
                                                         t["w_uk"], t["w_uv"], t["pool"], bt, lens, x["scale"], ws,
                                                         out, lse=lse, num_splits=args.num_splits, phases=ph,
                                                         stream=stream))
        else:
            if has_append:
                launches.append(mla.prepared_cache_append(d, t["h"], t["w_dkv"], t["w_kr"], pos, bt, t["pool"],
                                                          workspace=append_ws, stream=stream))
            dec_args = (d, t["qn"], t["qr"], t["w_uk"], t["w_uv"], t["pool"], bt, lens, x["scale"], ws, out)
            for name in ("mla_decode_prepare", "mla_decode_attend", "mla_decode_finish"):
                launches.append(mla.prepared_decode(name, *dec_args, lse=lse, num_splits=args.num_splits,
                                                    stream=stream))
        sets.append(launches)
    torch.cuda.synchronize()
    counter = [0]

    def step(ev_a=None, ev_b=None):
        launches = sets[counter[0] % copies]
        counter[0] += 1
        for launch in launches[:-2]:      # append (if not fused into the step), then prepare
            launch()
        if ev_a is not None:
            ev_a.record(stream)
        launches[-2]()                    # attend
        if ev_b is not None:
            ev_b.record(stream)
        launches[-1]()                    # finish
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K whole steps
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        step(ev_a[i], ev_b[i])
    t_end.record(stream)
    enqueued = time.perf_counter() - wall0     # host time to issue the steps (well under the GPU time)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / args.steps
    ms_attn = sum(a.elapsed_time(b) for a, b in zip(ev_a, ev_b)) / args.steps
    print(f"[bench] {args.steps} steps: {ms_step * 1e3:.1f} us/step (wall {wall / args.steps * 1e6:.1f} us), "
          f"attention {ms_attn * 1e3:.1f} us; host issue {enqueued / args.steps * 1e6:.1f} us/step", file=sys.stderr,
          flush=True)

    step_s = ms_step * 1e-3
    gbs = wl["bytes"] / step_s / 1e9
    tflops = wl["flops"] / step_s / 1e12
    tok_s = spec.batch * spec.sq / step_s
    attn_gbs = wl["cache_bytes"] / (ms_attn * 1e-3) / 1e9
    attn_tflops = wl["attn_flops"] / (ms_attn * 1e-3) / 1e12

    # The attention kernel's bound: HBM while its arithmetic intensity (flops per cache byte) is
    # under the chip's ridge point (2.5 PFLOP/s over 8 TB/s = 312.5 flop/B, one query token per
    # sequence), the bf16 MFMA peak above it (two or more query tokens per sequence).
    counters = measured_counters(args.workload)
    kernel_s = ms_attn * 1e-3
    mfma_bound = wl["attn_flops"] / wl["cache_bytes"] > MFMA_BF16_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3
    if mfma_bound:
        roofline = {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(attn_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                    "traffic": counters.get("traffic"), "flops_per_launch": wl["attn_flops"],
                    "hbm_gbs": round(attn_gbs, 2), "hbm_frac": round(attn_gbs / HBM_PEAK_GBS, 4)}
    else:
        roofline = {"bound": "hbm", "achieved": round(attn_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(attn_gbs / HBM_PEAK_GBS, 4), "traffic": counters.get("traffic"),
                    "bytes_per_launch": wl["cache_bytes"], "mfma_tflops": round(attn_tflops, 2),
                    "mfma_frac": round(attn_tflops / MFMA_BF16_PEAK_TFLOPS, 4)}
    roofline.update({"kernel": "attn_fp8_kernel" if fp8 else "attn_bf16_kernel",
                     "kernel_us": round(kernel_s * 1e6, 2),
                     # counter-based share of the matrix cores' cycles spent busy, from the
                     # committed rocprofv3 profile of this kernel (null if the sources changed)
                     "mfma_busy_counter": counters.get("mfma_busy")})
    res = {
        "metric": "MLA decode GB/s + TFLOP/s (% roofline), tokens/s; B=64 ctx=8K 128 heads",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic (seeded N(0,1) cache/queries/hidden states, N(0,1/fan_in) weights)",
        "config": {"workload": args.workload, "batch": spec.batch, "context": int(max(x["seq_lens"])),
                   "query_tokens": spec.sq, "heads": spec.n_heads, "d_latent": spec.d_latent,
                   "d_rope": spec.d_rope, "d_nope": spec.d_nope, "d_model": spec.d_model,
                   "block_size": spec.block_size, "paged": spec.paged, "append": spec.append,
                   "cache": "fp8_e4m3 (per-token power-of-two scale, bf16 k^R)" if fp8 else spec.dtype,
                   "cache_bytes_per_token": wl["row_bytes"], "num_splits": args.num_splits or "auto"},
        "tflops": round(tflops, 2),
        "tokens_per_s": round(tok_s, 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "step_bytes": wl["bytes"],
        "step_flops": wl["flops"],
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print(f"[bench] cpu baseline (oracle, ~{args.cpu_budget:.0f} s)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(x, args.cpu_budget, fp8)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
