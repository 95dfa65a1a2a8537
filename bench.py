"""Benchmark of the MLA attention core on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-extra] [--no-cpu]

A step is one pass of the attention core over one batch of synthetic input:
one mla_attn_prefill call for the prefill workloads, one mla_attn_decode call
(or its variable-length, paged, 2D-mask, rotary or latent-cache form) for the
decode workloads. The headline workload is the chunked prefill (B=1, 64 heads,
2048 new queries over 14336 cached keys, 16384 keys): the largest
configuration that fits one GPU's work. Its K timed steps follow W untimed
ones (and at least RAMP_SECONDS of warm-up, while the clock ramps up) and are
timed as ten trials with HIP events on the stream the library launches on;
`ms_per_step` is the mean over all K, and the trials' median and minimum
are reported beside it. Every other full-size workload is measured the same
way (its own step count, ten trials) and reported under "workloads"; decode
steps are replayed from a HIP graph over enough input copies that the 256 MB
Infinity Cache cannot hold them.

Prints one JSON line. `value` is algorithmic work / time: prefill counts
2*(192+128) flops per visible (query, key) pair, decode counts the bytes the
method must read and write (k_nope and v per head, the shared k_pe once per
sequence, q and out). `roofline` puts the dominant kernel against MI355X's
published peak. `cpu_baseline` times the fp64 oracle on a bounded sample of
the same workload and, on that sample, compares the GPU output with it
(max |err|, relative Frobenius error). `probes` holds what this GPU reaches
on the simplest work of each kind: a plain streaming read at the decodes'
byte counts and bf16 MFMA chains with the shader clock they ran at.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from seeded_inputs import (LATENT_WORKLOADS, MASKED_WORKLOADS, PAGED_WORKLOADS, SHARD_WORKLOADS,  # noqa: E402
                           VARLEN_PREFILL_WORKLOADS, VARLEN_WORKLOADS, WORKLOADS, device_inputs,
                           host_inputs, latent_device_inputs, latent_host_inputs, left_pad_mask,
                           left_pads, paged_device_inputs, paged_layout, varlen_prefill_lens,
                           varlen_seq_lens)

METRIC = "prefill attn TFLOP/s & decode HBM GB/s, 1 MI355X, as fraction of peak"
HEADLINE = "chunked_prefill"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, published
CACHE_BYTES = 256 << 20      # Infinity Cache
TRIALS = 10
RAMP_SECONDS = 0.3           # untimed warm-up lasts at least this long: the clock ramps up under load
ATOL, RTOL = 1e-2, 1e-2      # the parity bar on bf16 outputs

KERNEL_SOURCES = {
    "mla_decode_kernel": "attention_mla_causal_amd/csrc/mla_decode.hip",
    "mla_prefill_kernel": "attention_mla_causal_amd/csrc/mla_prefill.hip",
    "mla_attn_decode_latent": "attention_mla_causal_amd/csrc/mla_latent.hip",
    "mla_rope_apply_kernel": "attention_mla_causal_amd/csrc/mla_rope.hip",
}

EXTRA_ORDER = ("decode_p1000", "batched_decode", "causal_prefill", "chunked_prefill",
               "batched_decode_h8", "chunked_prefill_h8", "varlen_batched_decode",
               "paged_batched_decode", "varlen_prefill", "masked_batched_decode", "masked_prefill",
               "decode_p1000_rope", "rope_chunked_prefill", "latent_decode_p1000",
               "latent_batched_decode")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def sig(x, n=5):
    """x rounded to n significant digits (keeps the JSON line short)."""
    if x is None or not isinstance(x, float) or x == 0.0 or not np.isfinite(x):
        return x
    return float(f"{x:.{n}g}")


# ---------------------------------------------------------------- work counts

def decode_bytes(wl) -> int:
    B, H, S = wl.B, wl.H, wl.S
    return B * (H * S * (128 + 128) * 2 + S * 64 * 2 + H * 192 * 2 + H * 128 * 2)


def varlen_bytes(wl, lens) -> int:
    """Right-padded cache: each sequence's valid rows only (k_nope + v per head,
    the shared rotary key once), plus queries and output."""
    L = int(np.asarray(lens, dtype=np.int64).sum())
    return wl.H * L * (128 + 128) * 2 + L * 64 * 2 + wl.B * wl.H * (192 + 128) * 2


def paged_bytes(wl, lens) -> int:
    """Paged decode with append: cached keys before the new one, the new rows
    read and written once, queries and output."""
    L = int((np.asarray(lens, dtype=np.int64) - 1).clip(min=0).sum())
    row = wl.H * (128 + 128) * 2 + 64 * 2
    return L * row + 2 * wl.B * row + wl.B * wl.H * (192 + 128) * 2


def latent_bytes(wl) -> int:
    """Compressed cache: latent and rotary key of every key (once per sequence),
    kv_b_proj's weight (once per call), queries and output."""
    return wl.B * wl.S * (512 + 64) * 2 + wl.H * 256 * 512 * 2 + wl.B * wl.H * (192 + 128) * 2


def prefill_flops(wl) -> int:
    T, P = wl.T, wl.past_len
    return 2 * wl.B * wl.H * (192 + 128) * (T * P + T * (T + 1) // 2)


def varlen_prefill_flops(H, q_lens, past_lens) -> int:
    n_vis = sum(int(t) * int(p) + int(t) * (int(t) + 1) // 2 for t, p in zip(q_lens, past_lens))
    return 2 * H * (192 + 128) * n_vis


def masked_decode_bytes(wl, pads) -> int:
    """Visible rows only, the mask bytes, queries and output."""
    L = int((wl.S - np.asarray(pads, dtype=np.int64)).clip(min=0).sum())
    return wl.H * L * (128 + 128) * 2 + L * 64 * 2 + wl.B * wl.S + wl.B * wl.H * (192 + 128) * 2


def masked_prefill_flops(wl, pads) -> int:
    """Visible pairs only: query i of sequence b sees keys pads[b] .. past_len + i."""
    i = np.arange(wl.T, dtype=np.int64)
    n_vis = sum(int(np.clip(wl.past_len + i - p + 1, 0, None).sum()) for p in np.asarray(pads))
    return 2 * wl.H * (192 + 128) * n_vis


def rope_apply_bytes(wl) -> int:
    """q_pe (H rows per position) and the new k_pe rows read and written once,
    plus one 256-byte table row per position."""
    return (wl.H + 1) * wl.B * wl.T * 256 + wl.T * 256


# ---------------------------------------------------------------- records

def source_hash(kernel: str) -> str:
    with open(os.path.join(ROOT, KERNEL_SOURCES[kernel]), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    ent = rec.get(kernel, {}).get(workload)
    if not ent or ent.get("source_sha256_16") != source_hash(kernel):
        return None
    return ent.get("hbm_bytes_per_launch")


def blas_info():
    """(library name and version, thread count) of numpy's BLAS."""
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                return f"{i.get('internal_api', '?')} {i.get('version', '')}".strip(), int(i.get("num_threads", 1))
    except Exception:
        pass
    return "unknown", 1


def record(shape, t, work, bound, kernel, traffic, timing):
    """Compact record of one workload: times, rate, roofline."""
    hbm = bound == "hbm"
    unit, scale, peak = ("GB/s", 1e9, HBM_PEAK_GBS) if hbm else ("TFLOP/s", 1e12, MFMA_BF16_PEAK_TFS)
    rate = work / (t["ms_per_step"] * 1e-3) / scale
    return {"shape": shape, "ms_per_step": sig(t["ms_per_step"]), "median_ms": sig(t["median_ms"]),
            "min_ms": sig(t["min_ms"]), "steps": t["steps"], "trials": t["trials"], "timing": timing,
            "value": sig(rate), "unit": unit, ("alg_bytes" if hbm else "alg_flops"): int(work),
            "roofline": {"bound": bound, "kernel": kernel, "achieved": sig(rate), "peak": peak, "unit": unit,
                         "frac": sig(rate / peak, 4), "traffic": sig(traffic)}}


# ---------------------------------------------------------------- timing

def warm_up(fn, warmup):
    """At least `warmup` untimed steps, and at least RAMP_SECONDS of them."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while i < warmup or time.perf_counter() - t0 < RAMP_SECONDS:
        fn(i)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def measure(fn, steps, warmup, graph=False, trials=TRIALS):
    """Warm up, then time exactly `steps` steps as min(trials, steps) trials
    (fn(0), fn(1), ... within each), with HIP events recorded on the current
    stream between trials and a synchronisation on both sides. graph: each
    trial replays a HIP graph holding its steps (captured after the warm-up),
    so the GPU never waits for the Python launcher."""
    import torch
    warm_up(fn, warmup)
    n = max(1, min(trials, steps))
    sizes = [steps // n + (1 if t < steps % n else 0) for t in range(n)]
    runners = {}
    if graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn(0)  # one eager call on the capture stream before capturing
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for k in sorted(set(sizes)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(k):
                    fn(i)
            g.replay()  # untimed: graph upload
            runners[k] = g.replay
        torch.cuda.synchronize()
        warm_up(lambda i: runners[sizes[0]](), 1)
    else:
        for k in set(sizes):
            runners[k] = (lambda k=k: [fn(i) for i in range(k)])
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record()
    for t, k in enumerate(sizes):
        runners[k]()
        ev[t + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [ev[t].elapsed_time(ev[t + 1]) / sizes[t] for t in range(n)]
    return {"ms_per_step": ev[0].elapsed_time(ev[n]) / steps, "median_ms": statistics.median(per),
            "min_ms": min(per), "steps": steps, "trials": n, "wall_ms_per_step": wall * 1e3 / steps}


def to_dev(bits, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def to_host_bits(t):
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def copies_for(nbytes):
    """Input copies a rotation needs so that the Infinity Cache cannot hold them."""
    return 1 if nbytes >= 2 * CACHE_BYTES else min(64, -(-2 * CACHE_BYTES // nbytes) + 1)


# ---------------------------------------------------------------- GPU runners
# Each returns (record, state): state carries what the CPU leg needs (inputs
# on the host or the device, and the GPU output of the last timed step).

def run_decode(wl, steps, warmup, graph=True, rope=False, seed=0):
    import torch
    import attention_mla_causal_amd as mla
    dev = torch.device("cuda:0")
    nbytes = decode_bytes(wl) + (wl.B * 256 if rope else 0)  # rotary: one table row per sequence
    copies = copies_for(nbytes)
    log(f"[bench] {wl.name}{'_rope' if rope else ''}: B={wl.B} H={wl.H} S={wl.S} copies={copies} steps={steps}")
    if wl.B * wl.H * wl.S * 256 * 2 > (1 << 31):
        sets = [device_inputs(wl, dev, seed=seed + c) for c in range(copies)]
        host = None
    else:
        hosts = [host_inputs(wl, seed=seed + c) for c in range(copies)]
        sets = [{k: to_dev(v, dev) for k, v in h.items()} for h in hosts]
        host = hosts[0]
    out = torch.empty((wl.B, wl.H, 1, 128), dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(max(mla.mla_attn_decode_workspace_bytes(wl.B, wl.H, wl.S), 256), dtype=torch.uint8,
                     device=dev)
    table = mla.mla_rope_table(wl.S, device=dev) if rope else None

    def step(i):
        d = sets[i % copies]
        mla.mla_attn_decode(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], wl.past_len,
                            wl.softmax_scale, out=out, workspace=ws, rope_table=table)

    t = measure(step, steps, warmup, graph=graph)
    step(0)  # the output of input set 0, for the CPU leg's comparison
    torch.cuda.synchronize()
    name = wl.name + ("_rope" if rope else "")
    kernel = "mla_decode_rope_kernel" if rope else "mla_decode_kernel"
    rec = record(f"B{wl.B} H{wl.H} S{wl.S}", t, nbytes, "hbm", kernel,
                 measured_traffic("mla_decode_kernel", name), "hip_graph" if graph else "eager")
    rec["input_copies"] = copies
    state = {"host": host, "dev": sets[0], "out": out.clone()}
    del sets
    return rec, state


def run_prefill(wl, steps, warmup, seed=0):
    import torch
    import attention_mla_causal_amd as mla
    dev = torch.device("cuda:0")
    log(f"[bench] {wl.name}: B={wl.B} H={wl.H} T={wl.T} P={wl.past_len} steps={steps}")
    x = host_inputs(wl, seed=seed)
    d = {k: to_dev(v, dev) for k, v in x.items()}
    out = torch.empty((wl.B, wl.H, wl.T, 128), dtype=torch.bfloat16, device=dev)
    need = mla.mla_attn_prefill_workspace_bytes(wl.B, wl.H, wl.T, wl.S)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)

    def step(i):
        mla.mla_attn_prefill(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], wl.past_len,
                             wl.softmax_scale, out=out, workspace=ws)

    t = measure(step, steps, warmup)
    kernel = "mla_prefill_split_kernel" if need else "mla_prefill_kernel"
    rec = record(f"B{wl.B} H{wl.H} T{wl.T} P{wl.past_len} S{wl.S}", t, prefill_flops(wl), "mfma", kernel,
                 measured_traffic("mla_prefill_kernel", wl.name), "eager")
    rec["std"] = sig(wl.std, 4)
    state = {"host": x, "out": out}
    del d
    return rec, state


def run_varlen(wl, steps, warmup, seed=0):
    import torch
    import attention_mla_causal_amd as mla
    dev = torch.device("cuda:0")
    lens = varlen_seq_lens(wl.B, wl.cap, seed=seed)
    log(f"[bench] {wl.name}: B={wl.B} H={wl.H} cap={wl.cap} sum(lens)={int(lens.sum())}")
    d = device_inputs(wl.cache(), dev, seed=seed)
    sl = torch.as_tensor(lens, device=dev)
    out = torch.empty((wl.B, wl.H, 1, 128), dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(max(mla.mla_attn_decode_varlen_workspace_bytes(wl.B, wl.H, wl.cap), 256),
                     dtype=torch.uint8, device=dev)

    def step(i):
        mla.mla_attn_decode_varlen(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], sl, wl.cap,
                                   wl.softmax_scale, out=out, workspace=ws)

    t = measure(step, steps, warmup, graph=True)
    rec = record(f"B{wl.B} H{wl.H} cap{wl.cap} sum_len{int(lens.sum())}", t, varlen_bytes(wl, lens), "hbm",
                 "mla_decode_kernel", measured_traffic("mla_decode_kernel", wl.name), "hip_graph")
    step(0)
    torch.cuda.synchronize()
    return rec, {"dev": d, "out": out.clone(), "lens": lens}


def run_paged(wl, steps, warmup, seed=0):
    import torch
    import attention_mla_causal_amd as mla
    dev = torch.device("cuda:0")
    lens = varlen_seq_lens(wl.B, wl.cap, seed=seed)
    table, nblocks = paged_layout(lens, wl.block_size, seed=seed)
    log(f"[bench] {wl.name}: B={wl.B} H={wl.H} bs={wl.block_size} blocks={nblocks} sum(lens)={int(lens.sum())}")
    d = paged_device_inputs(wl.B, wl.H, nblocks, wl.block_size, dev, seed=seed)
    tb = torch.as_tensor(table, device=dev)
    sl = torch.as_tensor(lens, device=dev)
    out = torch.empty((wl.B, wl.H, 1, 128), dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(max(mla.mla_attn_decode_paged_workspace_bytes(wl.B, wl.H, wl.cap), 256),
                     dtype=torch.uint8, device=dev)
    new = (d["k_nope_new"], d["k_pe_new"], d["v_new"])

    def step(i):
        mla.mla_attn_decode_paged(d["q_nope"], d["q_pe"], d["k_nope_pages"], d["k_pe_pages"], d["v_pages"],
                                  tb, sl, wl.cap, wl.softmax_scale, new=new, out=out, workspace=ws)

    t = measure(step, steps, warmup, graph=True)
    rec = record(f"B{wl.B} H{wl.H} bs{wl.block_size} sum_len{int(lens.sum())} append", t, paged_bytes(wl, lens),
                 "hbm", "mla_decode_kernel", measured_traffic("mla_decode_kernel", wl.name), "hip_graph")
    step(0)
    torch.cuda.synchronize()
    return rec, {"dev": d, "out": out.clone(), "lens": lens, "table": table}


def run_prefill_varlen(wl, steps, warmup, seed=0):
    import torch
    import attention_mla_causal_amd as mla
    dev = torch.device("cuda:0")
    tq, pl = varlen_prefill_lens(wl.B, wl.max_q, wl.max_kv, seed=seed)
    log(f"[bench] {wl.name}: B={wl.B} H={wl.H} max_q={wl.max_q} max_kv={wl.max_kv} q_lens={tq.tolist()}")
    d = device_inputs(wl.padded(), dev, seed=seed)
    ql, pp = torch.as_tensor(tq, device=dev), torch.as_tensor(pl, device=dev)
    out = torch.empty((wl.B, wl.H, wl.max_q, 128), dtype=torch.bfloat16, device=dev)

    def step(i):
        mla.mla_attn_prefill_varlen(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], ql, pp,
                                    wl.softmax_scale, out=out)

    t = measure(step, steps, warmup)
    rec = record(f"B{wl.B} H{wl.H} max_q{wl.max_q} max_kv{wl.max_kv}", t, varlen_prefill_flops(wl.H, tq, pl),
                 "mfma", "mla_prefill_varlen_kernel", measured_traffic("mla_prefill_kernel", wl.name), "eager")
    return rec, {"dev": d, "out": out, "q_lens": tq, "past_lens": pl}


def run_masked(wl, steps, warmup, seed=0):
    import torch
    import attention_mla_causal_amd as mla
    dev = torch.device("cuda:0")
    pads = left_pads(wl, seed=seed)
    mask_np = left_pad_mask(wl.S, pads)
    mask = torch.as_tensor(mask_np, device=dev)
    d = device_inputs(wl, dev, seed=seed)
    log(f"[bench] {wl.name}: B={wl.B} H={wl.H} T={wl.T} S={wl.S} sum(pads)={int(pads.sum())}")
    out = torch.empty((wl.B, wl.H, wl.T, 128), dtype=torch.bfloat16, device=dev)
    if wl.T == 1:
        ws = torch.zeros(max(mla.mla_attn_decode_varlen_workspace_bytes(wl.B, wl.H, wl.S), 256),
                         dtype=torch.uint8, device=dev)

        def step(i):
            mla.mla_attn_decode_masked(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], mask,
                                       wl.past_len, wl.softmax_scale, out=out, workspace=ws)

        t = measure(step, steps, warmup, graph=True)
        rec = record(f"B{wl.B} H{wl.H} S{wl.S} sum_pad{int(pads.sum())}", t, masked_decode_bytes(wl, pads), "hbm",
                     "mla_decode_masked_kernel", measured_traffic("mla_decode_kernel", wl.name), "hip_graph")
    else:
        def step(i):
            mla.mla_attn_prefill_masked(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], mask,
                                        wl.past_len, wl.softmax_scale, out=out)

        t = measure(step, steps, warmup)
        rec = record(f"B{wl.B} H{wl.H} T{wl.T} pads{pads.tolist()}", t, masked_prefill_flops(wl, pads), "mfma",
                     "mla_prefill_masked_kernel", measured_traffic("mla_prefill_kernel", wl.name), "eager")
    return rec, {"dev": d, "out": out, "mask": mask_np, "pads": pads}


def run_rope_apply(wl, steps, warmup, seed=0):
    """The rotary prologue of a prefill step: q_pe [B, H, T, 64] and the new
    keys' k_pe [B, 1, T, 64] rotated in place at past_len + t, one launch."""
    import torch
    import attention_mla_causal_amd as mla
    dev = torch.device("cuda:0")
    nbytes = rope_apply_bytes(wl)
    copies = copies_for(nbytes)
    log(f"[bench] rope prologue of {wl.name}: B={wl.B} H={wl.H} T={wl.T} P={wl.past_len} copies={copies}")
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    sets = [(torch.randn((wl.B, wl.H, wl.T, 64), generator=g, device=dev).to(torch.bfloat16),
             torch.randn((wl.B, 1, wl.T, 64), generator=g, device=dev).to(torch.bfloat16)) for _ in range(copies)]
    table = mla.mla_rope_table(wl.S, device=dev)

    def step(i):
        q, k = sets[i % copies]
        mla.mla_rope_apply_qk(q, k, table, past_len=wl.past_len)

    t = measure(step, steps, warmup, graph=True)
    rec = record(f"B{wl.B} H{wl.H} T{wl.T} P{wl.past_len}", t, nbytes, "hbm", "mla_rope_apply_kernel",
                 measured_traffic("mla_rope_apply_kernel", "rope_" + wl.name), "hip_graph")
    rec["input_copies"] = copies
    del sets
    # one more call on fresh rows, kept for the CPU leg's comparison
    q = torch.randn((wl.B, wl.H, wl.T, 64), generator=g, device=dev).to(torch.bfloat16)
    k = torch.randn((wl.B, 1, wl.T, 64), generator=g, device=dev).to(torch.bfloat16)
    state = {"q_in": to_host_bits(q), "k_in": to_host_bits(k)}
    mla.mla_rope_apply_qk(q, k, table, past_len=wl.past_len)
    torch.cuda.synchronize()
    state.update(q_out=to_host_bits(q), k_out=to_host_bits(k))
    return rec, state


def run_latent(wl, steps, warmup, seed=0):
    import torch
    import attention_mla_causal_amd as mla
    dev = torch.device("cuda:0")
    nbytes = latent_bytes(wl)
    copies = copies_for(nbytes)
    log(f"[bench] {wl.name}: B={wl.B} H={wl.H} S={wl.S} copies={copies}")
    if wl.B * wl.S * 512 * 2 > (1 << 28):
        sets = [latent_device_inputs(wl, dev, seed=seed + c) for c in range(copies)]
        host = None
    else:
        hosts = [latent_host_inputs(wl, seed=seed + c) for c in range(copies)]
        sets = [{k: to_dev(v, dev) for k, v in h.items()} for h in hosts]
        host = hosts[0]
    out = torch.empty((wl.B, wl.H, 1, 128), dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(max(mla.mla_attn_decode_latent_workspace_bytes(wl.B, wl.H, wl.S), 256), dtype=torch.uint8,
                     device=dev)

    def step(i):
        d = sets[i % copies]
        mla.mla_attn_decode_latent(d["q_nope"], d["q_pe"], d["c_kv"], d["k_pe"], d["w_kv_b"], wl.past_len,
                                   wl.softmax_scale, out=out, workspace=ws)

    t = measure(step, steps, warmup, graph=True)
    step(0)
    torch.cuda.synchronize()
    rec = record(f"B{wl.B} H{wl.H} S{wl.S}", t, nbytes, "hbm", "mla_attn_decode_latent",
                 measured_traffic("mla_attn_decode_latent", wl.name), "hip_graph")
    rec["input_copies"] = copies
    state = {"host": host, "dev": sets[0], "out": out.clone()}
    del sets
    return rec, state


# ---------------------------------------------------------------- CPU legs
# The fp64 oracle as it stands, timed on the host's cores over a bounded
# sample of the workload; on that sample the GPU output is compared with it.

class Parity:
    def __init__(self):
        self.n, self.max_err, self.sq_err, self.sq_ref, self.ok = 0, 0.0, 0.0, 0.0, True

    def add(self, gpu, ref):
        from oracle import bf16_bits_to_f64
        g = bf16_bits_to_f64(gpu) if gpu.dtype == np.uint16 else np.asarray(gpu, dtype=np.float64)
        r = np.asarray(ref, dtype=np.float64)
        err = np.abs(g - r)
        self.n += err.size
        self.max_err = max(self.max_err, float(err.max()) if err.size else 0.0)
        self.sq_err += float((err ** 2).sum())
        self.sq_ref += float((r ** 2).sum())
        self.ok = self.ok and bool(np.all(np.isfinite(g))) and bool(np.all(err <= ATOL + RTOL * np.abs(r)))

    def result(self):
        rel = (self.sq_err ** 0.5) / (self.sq_ref ** 0.5) if self.sq_ref > 0 else self.sq_err ** 0.5
        return {"n": self.n, "max_abs_err": sig(self.max_err, 3), "rel_fro": sig(rel, 3), "within_bound": self.ok}


def cpu_record(value, unit, sample, parity=None):
    blas, threads = blas_info()
    r = {"value": sig(value), "unit": unit, "cores": threads, "host_cpus": len(os.sched_getaffinity(0)),
         "blas": blas, "kind": "oracle", "sample": sample}
    if parity is not None:
        r["parity"] = parity.result()
    return r


def _timed(fn):
    t0 = time.perf_counter()
    r = fn()
    return r, time.perf_counter() - t0


def head_order(H):
    """Heads in the order the prefill legs sample them: spread first, then the rest."""
    first = [h for h in (0, H // 3, 2 * H // 3, H - 1) if h < H]
    return list(dict.fromkeys(first + list(range(H))))


def cpu_prefill(wl, state, seconds):
    """Whole heads (every query row) of batch 0, in head_order, until `seconds` pass."""
    from oracle import mla_attention
    x, out = state["host"], to_host_bits(state["out"])
    par, el, heads = Parity(), 0.0, 0
    for h in head_order(wl.H):
        ref, dt = _timed(lambda: mla_attention(x["q_nope"][:1, h:h + 1], x["q_pe"][:1, h:h + 1],
                                               x["k_nope"][:1, h:h + 1], x["k_pe"][:1],
                                               x["v"][:1, h:h + 1], wl.past_len, wl.softmax_scale))
        el += dt
        heads += 1
        par.add(out[:1, h:h + 1], ref)
        if el >= seconds:
            break
    rate = prefill_flops(wl) / (wl.B * wl.H) * heads / el / 1e12
    return cpu_record(rate, "TFLOP/s", f"{heads} of {wl.H} heads of batch 0, all {wl.T} queries, {el:.1f} s", par)


def cpu_decode_whole(wl, state, seconds):
    """The whole decode workload (input set 0), repeated for ~`seconds`."""
    from oracle import mla_attention
    x = state["host"]
    par = Parity()
    reps, el, ref = 0, 0.0, None
    while el < seconds and reps < 1000:
        ref, dt = _timed(lambda: mla_attention(x["q_nope"], x["q_pe"], x["k_nope"], x["k_pe"], x["v"],
                                               wl.past_len, wl.softmax_scale))
        el += dt
        reps += 1
    par.add(to_host_bits(state["out"]), ref)
    return cpu_record(decode_bytes(wl) * reps / el / 1e9, "GB/s",
                      f"whole workload (B={wl.B} H={wl.H} S={wl.S}), {reps} repetitions, {el:.1f} s", par)


def cpu_decode_rope_whole(wl, state, seconds):
    """The pages' decode with the rotary prologue, whole (input set 0): the
    rotary oracle turns the query at position S-1 (the released
    configuration's YaRN table), then the attention oracle runs; repeated
    for ~`seconds`."""
    from oracle import KIMI_K2_ROPE, apply_rope, bf16_bits_to_f64, mla_attention, rope_cos_sin, rope_positions
    x = state["host"]
    par = Parity()

    def oracle():
        cos, sin = rope_cos_sin(wl.S, **KIMI_K2_ROPE)
        q_rot = apply_rope(bf16_bits_to_f64(x["q_pe"]), rope_positions(wl.B, 1, past_len=wl.past_len), cos, sin)
        return mla_attention(x["q_nope"], q_rot, x["k_nope"], x["k_pe"], x["v"], wl.past_len, wl.softmax_scale)

    reps, el, ref = 0, 0.0, None
    while el < seconds and reps < 1000:
        ref, dt = _timed(oracle)
        el += dt
        reps += 1
    par.add(to_host_bits(state["out"]), ref)
    nbytes = decode_bytes(wl) + wl.B * 256
    return cpu_record(nbytes * reps / el / 1e9, "GB/s",
                      f"whole workload (B={wl.B} H={wl.H} S={wl.S}, table included), {reps} repetitions, "
                      f"{el:.1f} s", par)


def sampled_pairs(B, H, n, seed=0):
    """Up to n (b, h) pairs: both ends, one in each eighth of the b*H + h
    range and one of each residue of b*H + h mod 8 (the two ways the decode
    kernels deal (b, h) pairs to the XCDs), then random ones."""
    rng = np.random.default_rng(seed)
    BH = B * H
    eighth = max(BH // 8, 1)
    flat = [0, BH - 1]
    for r in range(8):
        flat.append(min(BH - 1, r * BH // 8 + int(rng.integers(eighth))))
        flat.append(min(BH - 1, 8 * int(rng.integers(eighth)) + r))
    while len(set(flat)) < min(n, BH):
        flat.append(int(rng.integers(BH)))
    return [divmod(f, H) for f in list(dict.fromkeys(flat))[:n]]


def cpu_decode_sampled(wl, state, seconds):
    """Sampled (b, h) pairs of a decode whose inputs live on the device: each
    pair's rows are copied to the host, then the oracle runs on them (timed)."""
    from oracle import mla_attention
    d, out = state["dev"], state["out"]
    par, el, n = Parity(), 0.0, 0
    for b, h in sampled_pairs(wl.B, wl.H, 64):
        xs = {"q_nope": to_host_bits(d["q_nope"][b:b + 1, h:h + 1]), "q_pe": to_host_bits(d["q_pe"][b:b + 1, h:h + 1]),
              "k_nope": to_host_bits(d["k_nope"][b:b + 1, h:h + 1]), "k_pe": to_host_bits(d["k_pe"][b:b + 1]),
              "v": to_host_bits(d["v"][b:b + 1, h:h + 1])}
        ref, dt = _timed(lambda: mla_attention(xs["q_nope"], xs["q_pe"], xs["k_nope"], xs["k_pe"], xs["v"],
                                               wl.past_len, wl.softmax_scale))
        el += dt
        n += 1
        par.add(to_host_bits(out[b:b + 1, h:h + 1]), ref)
        if el >= seconds:
            break
    per_pair = decode_bytes(wl) / (wl.B * wl.H)
    return cpu_record(per_pair * n / el / 1e9, "GB/s", f"{n} of {wl.B * wl.H} (b, h) pairs (rows copied from the "
                      f"device inputs), {el:.1f} s", par)


def _pair_bytes(L, H):
    """Algorithmic bytes of one (b, h) pair of a decode over L keys: its k_nope
    and v rows, its share of the shared rotary rows, query and output."""
    return L * (128 + 128) * 2 + L * 64 * 2 / H + (192 + 128) * 2


def cpu_varlen_decode(wl, state, seconds):
    """The variable-length decode oracle on sampled (b, h) pairs; each pair's
    valid cache rows are copied back from the device inputs."""
    from oracle import mla_decode_varlen_rows
    d, out, lens = state["dev"], state["out"], state["lens"]
    par, el, n, work = Parity(), 0.0, 0, 0.0
    for b, h in sampled_pairs(wl.B, wl.H, 64):
        L = int(lens[b])
        xs = {"q_nope": to_host_bits(d["q_nope"][b:b + 1, h:h + 1]), "q_pe": to_host_bits(d["q_pe"][b:b + 1, h:h + 1]),
              "k_nope": to_host_bits(d["k_nope"][b:b + 1, h:h + 1, :max(L, 1)]),
              "k_pe": to_host_bits(d["k_pe"][b:b + 1, :, :max(L, 1)]),
              "v": to_host_bits(d["v"][b:b + 1, h:h + 1, :max(L, 1)])}
        ref, dt = _timed(lambda: mla_decode_varlen_rows(xs["q_nope"], xs["q_pe"], xs["k_nope"], xs["k_pe"], xs["v"],
                                                        np.array([L]), wl.softmax_scale, [(0, 0)]))
        el += dt
        n += 1
        work += _pair_bytes(L, wl.H)
        par.add(to_host_bits(out[b, h, 0]), ref[0])
        if el >= seconds:
            break
    return cpu_record(work / el / 1e9, "GB/s", f"{n} of {wl.B * wl.H} (b, h) pairs (valid rows copied from the "
                      f"device cache), {el:.1f} s", par)


def cpu_paged_decode(wl, state, seconds):
    """The paged-decode oracle (append, then attend) on sampled (b, h) pairs:
    the blocks a sequence's table names, for that head, are copied back and
    renumbered, with the new token's rows from the call's inputs."""
    import torch
    from oracle import mla_decode_paged
    d, out, lens, table = state["dev"], state["out"], state["lens"], state["table"]
    bs = wl.block_size
    par, el, n, work = Parity(), 0.0, 0, 0.0
    for b, h in sampled_pairs(wl.B, wl.H, 64):
        L = int(lens[b])
        nblk = max((L + bs - 1) // bs, 1)
        idx = torch.as_tensor(np.asarray(table[b, :nblk], dtype=np.int64), device=d["k_pe_pages"].device)
        kn = to_host_bits(d["k_nope_pages"].index_select(0, idx)[:, h:h + 1])
        vv = to_host_bits(d["v_pages"].index_select(0, idx)[:, h:h + 1])
        kp = to_host_bits(d["k_pe_pages"].index_select(0, idx))
        new = (to_host_bits(d["k_nope_new"][b:b + 1, h:h + 1]), to_host_bits(d["k_pe_new"][b:b + 1]),
               to_host_bits(d["v_new"][b:b + 1, h:h + 1]))
        q = (to_host_bits(d["q_nope"][b:b + 1, h:h + 1]), to_host_bits(d["q_pe"][b:b + 1, h:h + 1]))
        local = np.arange(nblk, dtype=np.int32)[None]
        res, dt = _timed(lambda: mla_decode_paged(q[0], q[1], kn, kp, vv, local, np.array([L]), wl.softmax_scale,
                                                  new=new))
        el += dt
        n += 1
        work += _pair_bytes(max(L - 1, 0), wl.H) + 2 * ((128 + 128) * 2 + 64 * 2 / wl.H)
        par.add(to_host_bits(out[b, h, 0]), res[0][0, 0, 0])
        if el >= seconds:
            break
    return cpu_record(work / el / 1e9, "GB/s", f"{n} of {wl.B * wl.H} (b, h) pairs (the sequence's blocks for the "
                      f"head copied from the device pages), {el:.1f} s", par)


def cpu_varlen_prefill(wl, state, seconds):
    """Heads of the longest sequence (device inputs copied back), through the
    padded-batch oracle, until `seconds` pass."""
    from oracle import mla_prefill_varlen
    d, out = state["dev"], state["out"]
    T0, P0 = int(state["q_lens"][0]), int(state["past_lens"][0])
    S0 = T0 + P0
    par, el, heads = Parity(), 0.0, 0
    for h in head_order(wl.H):
        xs = {"q_nope": to_host_bits(d["q_nope"][:1, h:h + 1, :T0]), "q_pe": to_host_bits(d["q_pe"][:1, h:h + 1, :T0]),
              "k_nope": to_host_bits(d["k_nope"][:1, h:h + 1, :S0]), "k_pe": to_host_bits(d["k_pe"][:1, :, :S0]),
              "v": to_host_bits(d["v"][:1, h:h + 1, :S0])}
        ref, dt = _timed(lambda: mla_prefill_varlen(xs["q_nope"], xs["q_pe"], xs["k_nope"], xs["k_pe"], xs["v"],
                                                    np.array([T0]), np.array([P0]), wl.softmax_scale))
        el += dt
        heads += 1
        par.add(to_host_bits(out[:1, h:h + 1, :T0]), ref)
        if el >= seconds:
            break
    rate = varlen_prefill_flops(1, [T0], [P0]) * heads / el / 1e12
    return cpu_record(rate, "TFLOP/s", f"{heads} heads of the longest sequence, {el:.1f} s", par)


def cpu_masked(wl, state, seconds):
    """The 2D-mask oracle on device inputs copied back: decode, sampled (b, h)
    pairs; prefill, 64-query blocks of head 0 of the most padded sequence."""
    from oracle import mla_attention_masked
    d, out, mask, pads = state["dev"], state["out"], state["mask"], state["pads"]
    par, el, n = Parity(), 0.0, 0
    if wl.T == 1:
        for b, h in sampled_pairs(wl.B, wl.H, 64):
            xs = {k: to_host_bits(d[k][b:b + 1] if k == "k_pe" else d[k][b:b + 1, h:h + 1])
                  for k in ("q_nope", "q_pe", "k_nope", "k_pe", "v")}
            ref, dt = _timed(lambda: mla_attention_masked(xs["q_nope"], xs["q_pe"], xs["k_nope"], xs["k_pe"],
                                                          xs["v"], mask[b:b + 1], wl.past_len, wl.softmax_scale))
            el += dt
            n += 1
            par.add(to_host_bits(out[b:b + 1, h:h + 1]), ref)
            if el >= seconds:
                break
        per = masked_decode_bytes(wl, pads) / (wl.B * wl.H)
        return cpu_record(per * n / el / 1e9, "GB/s", f"{n} of {wl.B * wl.H} (b, h) pairs, {el:.1f} s", par)
    b = int(np.argmax(pads))
    rows = 64
    xs = {k: to_host_bits(d[k][b:b + 1] if k == "k_pe" else d[k][b:b + 1, :1]) for k in ("q_nope", "q_pe", "k_nope",
                                                                                        "k_pe", "v")}
    pairs = 0
    for lo in range(wl.T - rows, -1, -rows):  # the last (longest) query rows first
        hi = lo + rows
        S_hi = wl.past_len + hi
        ref, dt = _timed(lambda: mla_attention_masked(
            xs["q_nope"][:, :, lo:hi], xs["q_pe"][:, :, lo:hi], xs["k_nope"][:, :, :S_hi], xs["k_pe"][:, :, :S_hi],
            xs["v"][:, :, :S_hi], mask[b:b + 1, :S_hi], wl.past_len + lo, wl.softmax_scale))
        el += dt
        i = np.arange(lo, hi, dtype=np.int64)
        pairs += int(np.clip(wl.past_len + i - pads[b] + 1, 0, None).sum())
        par.add(to_host_bits(out[b:b + 1, :1, lo:hi]), ref)
        if el >= seconds:
            break
    return cpu_record(2 * 320 * pairs / el / 1e12, "TFLOP/s", f"64-query blocks of head 0, sequence {b} "
                      f"(pad {int(pads[b])}), {el:.1f} s", par)


def cpu_latent(wl, state, seconds):
    """The latent-cache oracle on sampled (b, h) pairs (device inputs copied
    back for the batched decode)."""
    from oracle import mla_decode_latent_rows
    out = state["out"]
    par, el, n = Parity(), 0.0, 0
    if state["host"] is not None:
        x = state["host"]
        sel = lambda b: {k: (x[k] if k == "w_kv_b" else x[k][b:b + 1]) for k in x}  # noqa: E731
    else:
        d = state["dev"]
        w = to_host_bits(d["w_kv_b"])
        sel = lambda b: {**{k: to_host_bits(d[k][b:b + 1]) for k in ("q_nope", "q_pe", "c_kv", "k_pe")},  # noqa: E731
                         "w_kv_b": w}
    cache = {}
    for b, h in sampled_pairs(wl.B, wl.H, 64):
        if b not in cache:
            cache = {b: sel(b)}
        xs = cache[b]
        ref, dt = _timed(lambda: mla_decode_latent_rows(xs["q_nope"], xs["q_pe"], xs["c_kv"], xs["k_pe"],
                                                        xs["w_kv_b"], wl.past_len, wl.softmax_scale, [(0, h)]))
        el += dt
        n += 1
        par.add(to_host_bits(out[b, h, 0]), ref[0])
        if el >= seconds:
            break
    per = latent_bytes(wl) / (wl.B * wl.H)
    return cpu_record(per * n / el / 1e9, "GB/s", f"{n} of {wl.B * wl.H} (b, h) pairs, {el:.1f} s", par)


def cpu_rope(wl, state, seconds):
    """The fp64 rotation oracle on the rows of the GPU's last call (table
    built once), the whole workload repeated for ~`seconds`; the GPU's rotated
    rows are compared with it."""
    from oracle import KIMI_K2_ROPE, apply_rope, bf16_bits_to_f64, rope_cos_sin, rope_positions
    q, k = bf16_bits_to_f64(state["q_in"]), bf16_bits_to_f64(state["k_in"])
    cos, sin = rope_cos_sin(wl.S, **KIMI_K2_ROPE)
    pos = rope_positions(wl.B, wl.T, past_len=wl.past_len)
    n, el, res = 0, 0.0, None
    while el < seconds:
        res, dt = _timed(lambda: (apply_rope(q, pos, cos, sin), apply_rope(k, pos, cos, sin)))
        el += dt
        n += 1
    par = Parity()
    par.add(state["q_out"], res[0])
    par.add(state["k_out"], res[1])
    return cpu_record(rope_apply_bytes(wl) * n / el / 1e9, "GB/s", f"the whole workload {n} times, {el:.1f} s",
                      par)


# ---------------------------------------------------------------- probes

def run_probes():
    """A plain streaming read at the decodes' byte counts (the floor a launch
    moving those bytes cannot beat) and bf16 MFMA chains with the shader clock
    they ran at (what the prefill's instruction reaches on this part)."""
    import torch
    path = os.path.join(ROOT, "attention_mla_causal_amd", "libmla_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it (python attention_mla_causal_amd/build.py)")
    lib = ctypes.CDLL(path)
    lib.mla_probe_stream_read.restype = ctypes.c_int
    lib.mla_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_void_p]
    lib.mla_probe_mfma.restype = ctypes.c_int
    lib.mla_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    stream = lambda: ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)  # noqa: E731
    res = {}

    def read_leg(name, nbytes, copies, steps, grids):
        bufs = [torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device=dev) for _ in range(copies)]
        sink = torch.zeros(max(grids), dtype=torch.int32, device=dev)
        best = None
        for grid in grids:
            for nt in (0, 1):
                def step(i, grid=grid, nt=nt):
                    rc = lib.mla_probe_stream_read(bufs[i % copies].data_ptr(), nbytes, sink.data_ptr(), grid, nt,
                                                   stream())
                    if rc != 0:
                        raise RuntimeError(f"stream read probe failed: {rc}")
                t = measure(step, steps, 10, graph=True)
                if best is None or t["median_ms"] < best[0]["median_ms"]:
                    best = (t, grid, nt)
        t, grid, nt = best
        res[name] = {"bytes": nbytes, "copies": copies, "median_us": sig(t["median_ms"] * 1e3),
                     "min_us": sig(t["min_ms"] * 1e3), "GB/s": sig(nbytes / (t["median_ms"] * 1e-3) / 1e9),
                     "frac": sig(nbytes / (t["median_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "grid": grid,
                     "nontemporal": bool(nt), "timing": "hip_graph"}
        del bufs

    c2 = decode_bytes(WORKLOADS["decode_p1000"]) // 16 * 16
    log("[bench] probes: streaming read")
    read_leg("stream_read_decode_p1000_bytes", c2, copies_for(c2), 200, (256, 512, 1024, 2048))
    read_leg("stream_read_4GiB", 4 << 30, 1, 10, (2048, 4096, 8192))

    log("[bench] probes: MFMA chains")
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    ops = torch.randn(8 * 64 * 8, generator=g, device=dev).to(torch.bfloat16)
    grid, iters = 512, 40000  # iters: a multiple of 8 (about 5 ms at full rate)
    out = torch.empty(grid * 256, dtype=torch.float32, device=dev)
    clocks = torch.zeros(grid * 2, dtype=torch.int64, device=dev)
    for valu, name in ((0, "mfma_bf16_chain"), (1, "mfma_bf16_chain_softmax_mix")):
        def step(i, valu=valu):
            rc = lib.mla_probe_mfma(ops.data_ptr(), grid, iters, valu, out.data_ptr(), clocks.data_ptr(), stream())
            if rc != 0:
                raise RuntimeError(f"MFMA probe failed: {rc}")
        t = measure(step, 10, 3)
        ck = clocks.view(grid, 2).cpu().numpy().astype(np.float64)
        ghz = float(np.median(ck[:, 0] / (ck[:, 1] / 100e6))) / 1e9
        flops = grid * 4 * iters * 4 * 32768
        tfs = flops / (t["median_ms"] * 1e-3) / 1e12
        res[name] = {"TFLOP/s": sig(tfs), "frac": sig(tfs / MFMA_BF16_PEAK_TFS, 4), "sclk_GHz": sig(ghz, 4),
                     "median_ms": sig(t["median_ms"]), "valu_per_mfma": "exp2 + 4 FMA" if valu else "none",
                     "operands": "random bf16, changing every MFMA"}
    return res


# ---------------------------------------------------------------- driver

def run_workload(name, steps, warmup, cpu_seconds, eager=False):
    """One workload: its GPU record, and its CPU leg when cpu_seconds > 0."""
    graph = not eager
    if name in WORKLOADS or name in SHARD_WORKLOADS:
        wl = {**WORKLOADS, **SHARD_WORKLOADS}[name]
        if wl.T == 1:
            rec, st = run_decode(wl, steps, warmup, graph=graph)
            if cpu_seconds > 0:
                rec["cpu_baseline"] = (cpu_decode_whole(wl, st, cpu_seconds) if st["host"] is not None
                                       else cpu_decode_sampled(wl, st, cpu_seconds))
        else:
            rec, st = run_prefill(wl, steps, warmup)
            if cpu_seconds > 0:
                rec["cpu_baseline"] = cpu_prefill(wl, st, cpu_seconds)
        return rec
    if name == "decode_p1000_rope":
        wl = WORKLOADS["decode_p1000"]
        rec, st = run_decode(wl, steps, warmup, graph=graph, rope=True)
        if cpu_seconds > 0:
            rec["cpu_baseline"] = cpu_decode_rope_whole(wl, st, cpu_seconds)
        return rec
    if name == "rope_chunked_prefill":
        rec, st = run_rope_apply(WORKLOADS["chunked_prefill"], steps, warmup)
        if cpu_seconds > 0:
            rec["cpu_baseline"] = cpu_rope(WORKLOADS["chunked_prefill"], st, min(cpu_seconds, 3.0))
        return rec
    if name in VARLEN_WORKLOADS:
        wl = VARLEN_WORKLOADS[name]
        rec, st = run_varlen(wl, steps, warmup)
        if cpu_seconds > 0:
            rec["cpu_baseline"] = cpu_varlen_decode(wl, st, cpu_seconds)
        return rec
    if name in PAGED_WORKLOADS:
        wl = PAGED_WORKLOADS[name]
        rec, st = run_paged(wl, steps, warmup)
        if cpu_seconds > 0:
            rec["cpu_baseline"] = cpu_paged_decode(wl, st, cpu_seconds)
        return rec
    if name in VARLEN_PREFILL_WORKLOADS:
        wl = VARLEN_PREFILL_WORKLOADS[name]
        rec, st = run_prefill_varlen(wl, steps, warmup)
        if cpu_seconds > 0:
            rec["cpu_baseline"] = cpu_varlen_prefill(wl, st, cpu_seconds)
        return rec
    if name in MASKED_WORKLOADS:
        wl = MASKED_WORKLOADS[name]
        rec, st = run_masked(wl, steps, warmup)
        if cpu_seconds > 0:
            rec["cpu_baseline"] = cpu_masked(wl, st, cpu_seconds)
        return rec
    if name in LATENT_WORKLOADS:
        wl = LATENT_WORKLOADS[name]
        rec, st = run_latent(wl, steps, warmup)
        if cpu_seconds > 0:
            rec["cpu_baseline"] = cpu_latent(wl, st, cpu_seconds)
        return rec
    raise KeyError(name)


def extra_steps(name):
    """Timed steps of a non-headline workload: enough for ten trials of a
    measurable span (short decodes replay 20 steps per trial)."""
    short = name in ("decode_p1000", "decode_p1000_rope", "rope_chunked_prefill", "latent_decode_p1000")
    return 200 if short else 20


def compact(rec):
    """The printed form of a non-headline workload (the full record goes to --detail)."""
    r = {"shape": rec["shape"], "ms": rec["ms_per_step"], "med": rec["median_ms"], "min": rec["min_ms"],
         "value": rec["value"], "unit": rec["unit"], "frac": rec["roofline"]["frac"],
         "traffic": rec["roofline"]["traffic"]}
    cb = rec.get("cpu_baseline")
    if cb:
        c = {"value": cb["value"], "unit": cb["unit"]}
        par = cb.get("parity")
        if par:
            c.update({"max_err": par["max_abs_err"], "rel_fro": par["rel_fro"], "ok": par["within_bound"]})
        r["cpu"] = c
    return r


def main():
    names = sorted(set(EXTRA_ORDER))
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE, choices=names)
    ap.add_argument("--no-extra", action="store_true", help="only the headline workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle legs")
    ap.add_argument("--no-probes", action="store_true", help="skip the streaming-read and MFMA probes")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="headline CPU leg budget (others: 4 s)")
    ap.add_argument("--eager", action="store_true",
                    help="time decode steps with plain launches instead of a HIP graph (profiler runs)")
    ap.add_argument("--detail", metavar="PATH", help="also write the full JSON record to PATH")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes three times (counter calibration)")
    args = ap.parse_args()

    if args.copy_calibration:
        import torch
        a = torch.ones(args.copy_calibration, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": args.copy_calibration}))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): the attention "
              "core has no cross-GPU path in this library; heads shard with no communication, so one GPU's "
              "figure is its per-GPU throughput.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.synchronize()

    head = run_workload(args.workload, args.steps, args.warmup, 0 if args.no_cpu else args.cpu_seconds,
                        eager=args.eager)
    cpu = head.pop("cpu_baseline", None)
    workloads = {}
    if not args.no_extra:
        for name in EXTRA_ORDER:
            if name == args.workload:
                continue
            workloads[name] = run_workload(name, extra_steps(name), 10 if extra_steps(name) > 20 else 3,
                                           0 if args.no_cpu else min(args.cpu_seconds, 4.0))
            torch.cuda.empty_cache()
    probes = None if (args.no_probes or args.no_extra) else run_probes()

    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "shape": head["shape"], "timing": head["timing"],
                   "median_ms": head["median_ms"], "min_ms": head["min_ms"], "trials": head["trials"],
                   "warmup_min_seconds": RAMP_SECONDS},
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "workloads": workloads,
        "probes": probes,
    }
    for k in ("std", "input_copies"):
        if k in head:
            line["config"][k] = head[k]
    if args.detail:
        with open(args.detail, "w") as f:
            json.dump(line, f, indent=1)
    line["workloads"] = {k: compact(v) for k, v in workloads.items()}
    if probes:
        line["probes"] = {k: {f: v[f] for f in ("median_us", "GB/s", "frac", "TFLOP/s", "sclk_GHz") if f in v}
                          for k, v in probes.items()}
    print(json.dumps(line, separators=(",", ":")), flush=True)


if __name__ == "__main__":
    main()
