"""Benchmark of the MLA attention core on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-extra]

One step is one pass of the attention core over one batch of synthetic input:
one mla_attn_decode call for the decode workloads, one mla_attn_prefill call
for the prefill workloads. The headline workload is decode exactly as the
"Similarities" page shows it (B=1, 64 heads, 1 query, past_len=1000, S=1001
keys); its K timed steps rotate over enough input copies that the 256 MB
Infinity Cache cannot hold them, and are replayed from a HIP graph so the GPU
never waits on the Python launcher. The other full-size workloads (batched
decode, causal prefill, chunked prefill) are measured in the same run and
reported under "workloads".

Prints one JSON line. `value` is algorithmic work / time: decode counts the
bytes the method must read and write (k_nope and v per head, the shared k_pe
once per sequence, q and out), prefill counts 2*(192+128) flops per visible
(query, key) pair. `roofline` puts the dominant kernel against MI355X's
published peak; `cpu_baseline` times the fp64 oracle on a bounded sample.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from seeded_inputs import (LATENT_WORKLOADS, PAGED_WORKLOADS, SHARD_WORKLOADS, VARLEN_WORKLOADS,  # noqa: E402
                           VARLEN_PREFILL_WORKLOADS, WORKLOADS, MASKED_WORKLOADS,
                           device_inputs, host_inputs, latent_device_inputs, latent_host_inputs,
                           left_pad_mask, left_pads, paged_device_inputs, paged_layout,
                           varlen_prefill_lens, varlen_seq_lens)

METRIC = "prefill attn TFLOP/s & decode HBM GB/s, 1 MI355X, as fraction of peak"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, published
CACHE_BYTES = 256 << 20      # Infinity Cache

KERNEL_SOURCES = {
    "mla_decode_kernel": "attention_mla_causal_amd/csrc/mla_decode.hip",
    "mla_prefill_kernel": "attention_mla_causal_amd/csrc/mla_prefill.hip",
    "mla_attn_decode_latent": "attention_mla_causal_amd/csrc/mla_latent.hip",  # its four launches
    "mla_rope_apply_kernel": "attention_mla_causal_amd/csrc/mla_rope.hip",
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def decode_bytes(wl) -> int:
    B, H, S = wl.B, wl.H, wl.S
    return B * (H * S * (128 + 128) * 2 + S * 64 * 2 + H * 192 * 2 + H * 128 * 2)


def varlen_bytes(wl, lens) -> int:
    """Right-padded cache: each sequence's valid rows only (k_nope + v per head,
    the shared rotary key once), plus queries and output."""
    H = wl.H
    L = int(np.asarray(lens, dtype=np.int64).sum())
    return H * L * (128 + 128) * 2 + L * 64 * 2 + wl.B * H * (192 + 128) * 2


def paged_bytes(wl, lens) -> int:
    """Paged decode with append: cached keys before the new one (k_nope + v per
    head, the shared rotary key once), the new rows read and written once,
    queries and output."""
    H, B = wl.H, wl.B
    L = int((np.asarray(lens, dtype=np.int64) - 1).clip(min=0).sum())
    row = H * (128 + 128) * 2 + 64 * 2
    return L * row + 2 * B * row + B * H * (192 + 128) * 2


def latent_bytes(wl) -> int:
    """Decode over the compressed cache: the latent and rotary key of every key
    (once per sequence), kv_b_proj's weight (once per call), queries, output."""
    B, H, S = wl.B, wl.H, wl.S
    return B * S * (512 + 64) * 2 + H * 256 * 512 * 2 + B * H * (192 + 128) * 2


def latent_flops(wl) -> int:
    """Two contractions per (batch, head, key) over 576 and 512 dims, plus the
    absorb and up-projection matrix-vector products."""
    B, H, S = wl.B, wl.H, wl.S
    return 2 * B * H * S * (576 + 512) + 2 * B * H * 128 * 512 * 2


def prefill_flops(wl) -> int:
    T, P = wl.T, wl.past_len
    n_vis = T * P + T * (T + 1) // 2
    return 2 * wl.B * wl.H * (192 + 128) * n_vis


def varlen_prefill_flops(wl, q_lens, past_lens) -> int:
    """Each sequence's own visible (query, key) pairs; padded rows count nothing."""
    n_vis = sum(int(t) * int(p) + int(t) * (int(t) + 1) // 2 for t, p in zip(q_lens, past_lens))
    return 2 * wl.H * (192 + 128) * n_vis


def masked_decode_bytes(wl, pads) -> int:
    """Visible rows only (k_nope + v per head, the shared rotary key once), the
    mask bytes, queries and output."""
    L = int((wl.S - np.asarray(pads, dtype=np.int64)).clip(min=0).sum())
    return wl.H * L * (128 + 128) * 2 + L * 64 * 2 + wl.B * wl.S + wl.B * wl.H * (192 + 128) * 2


def masked_prefill_flops(wl, pads) -> int:
    """Visible (query, key) pairs only: query i of sequence b sees keys
    pads[b] .. past_len + i."""
    n_vis = 0
    for p in np.asarray(pads, dtype=np.int64):
        i = np.arange(wl.T, dtype=np.int64)
        n_vis += int(np.clip(wl.past_len + i - p + 1, 0, None).sum())
    return 2 * wl.H * (192 + 128) * n_vis


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


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        return int(max(n)) if n else 1
    except Exception:
        return 1


def to_dev(bits, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


RAMP_SECONDS = 0.3  # untimed warm-up lasts at least this long: the GPU clock ramps up under load


def warm_up(fn, warmup):
    """Run at least `warmup` untimed steps, and keep going until RAMP_SECONDS have passed."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while i < warmup or time.perf_counter() - t0 < RAMP_SECONDS:
        fn(i)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def time_graph(fn, steps, warmup):
    """Warm up, capture `steps` calls in one HIP graph, time one replay."""
    import torch
    warm_up(fn, warmup)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(0)  # one eager call on the capture stream before capturing
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(steps):
            fn(i)
    g.replay()  # untimed replay: graph upload
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall * 1e3 / steps


def time_eager(fn, steps, warmup):
    import torch
    warm_up(fn, warmup)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall * 1e3 / steps


def run_decode(wl, steps, warmup, seed=0, graph=True, copies=None, rope=False):
    """rope: the query's rotary part is rotated inside the kernel
    (mla_attn_decode_rope, the released configuration's YaRN table); the
    algorithmic bytes add one 256-byte table row per sequence."""
    import torch
    import attention_mla_causal_amd as mla
    dev = torch.device("cuda:0")
    nbytes = decode_bytes(wl) + (wl.B * 256 if rope else 0)
    if copies is None:
        # enough distinct inputs that the rotation cannot live in the Infinity Cache
        copies = 1 if nbytes >= 2 * CACHE_BYTES else min(64, -(-2 * CACHE_BYTES // nbytes) + 1)
    log(f"[bench] {wl.name}: B={wl.B} H={wl.H} S={wl.S} copies={copies} steps={steps}")
    if wl.B * wl.H * wl.S * 256 * 2 > (1 << 31):
        sets = [device_inputs(wl, dev, seed=seed + c) for c in range(copies)]
        recipe = "device"
    else:
        sets = [{k: to_dev(v, dev) for k, v in host_inputs(wl, seed=seed + c).items()} for c in range(copies)]
        recipe = "host"
    out = torch.empty((wl.B, wl.H, 1, 128), dtype=torch.bfloat16, device=dev)
    need = mla.mla_attn_decode_workspace_bytes(wl.B, wl.H, wl.S)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
    table = mla.mla_rope_table(wl.S, device=dev) if rope else None

    def step(i):
        d = sets[i % copies]
        mla.mla_attn_decode(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], wl.past_len,
                            wl.softmax_scale, out=out, workspace=ws, rope_table=table)

    if graph:
        ms, wall_ms = time_graph(step, steps, warmup)
    else:
        ms, wall_ms = time_eager(step, steps, warmup)
    gbs = nbytes / (ms * 1e-3) / 1e9
    kernel = "mla_decode_rope_kernel" if rope else "mla_decode_kernel"
    name = wl.name + ("_rope" if rope else "")
    res = {
        "workload": name, "B": wl.B, "H": wl.H, "T": 1, "past_len": wl.past_len, "S": wl.S,
        "std": wl.std, "inputs": recipe, "input_copies": copies, "steps": steps,
        "timing": "hip_graph" if graph else "eager",
        "ms_per_step": ms, "wall_ms_per_step": wall_ms, "value": gbs, "unit": "GB/s",
        "algorithmic_bytes": nbytes,
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic("mla_decode_kernel", name)},
    }
    del sets
    torch.cuda.empty_cache()
    return res


def rope_apply_bytes(wl) -> int:
    """Rows of the new tokens' q_pe (H per position) and k_pe (one per
    position), each read and written once (128 bytes each way), plus one
    256-byte table row per position."""
    return (wl.H + 1) * wl.B * wl.T * 256 + wl.T * 256


def run_rope_apply(wl, steps, warmup, seed=0, graph=True):
    """The rotary prologue of a prefill step: q_pe [B, H, T, 64] and the new
    keys' k_pe [B, 1, T, 64] rotated in place at past_len + t, in one launch."""
    import torch
    import attention_mla_causal_amd as mla
    dev = torch.device("cuda:0")
    nbytes = rope_apply_bytes(wl)
    copies = min(64, -(-2 * CACHE_BYTES // nbytes) + 1)
    log(f"[bench] rope prologue of {wl.name}: B={wl.B} H={wl.H} T={wl.T} P={wl.past_len} copies={copies}")
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    sets = [(torch.randn((wl.B, wl.H, wl.T, 64), generator=g, device=dev).to(torch.bfloat16),
             torch.randn((wl.B, 1, wl.T, 64), generator=g, device=dev).to(torch.bfloat16)) for _ in range(copies)]
    table = mla.mla_rope_table(wl.S, device=dev)

    def step(i):
        q, k = sets[i % copies]
        mla.mla_rope_apply_qk(q, k, table, past_len=wl.past_len)

    ms, wall_ms = (time_graph if graph else time_eager)(step, steps, warmup)
    gbs = nbytes / (ms * 1e-3) / 1e9
    name = "rope_" + wl.name
    res = {"workload": name, "B": wl.B, "H": wl.H, "T": wl.T, "past_len": wl.past_len, "S": wl.S,
           "inputs": "device", "input_copies": copies, "steps": steps,
           "timing": "hip_graph" if graph else "eager", "ms_per_step": ms, "wall_ms_per_step": wall_ms,
           "value": gbs, "unit": "GB/s", "algorithmic_bytes": nbytes, "launches_per_step": 1,
           "roofline": {"bound": "hbm", "kernel": "mla_rope_apply_kernel", "achieved": gbs,
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                        "traffic": measured_traffic("mla_rope_apply_kernel", name)}}
    del sets
    torch.cuda.empty_cache()
    return res


def cpu_baseline_rope_apply(wl, seconds, seed=0):
    """The fp64 rotation oracle over the same rows (table built once, not timed)."""
    from oracle import KIMI_K2_ROPE, apply_rope, rope_cos_sin, rope_positions
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((wl.B, wl.H, wl.T, 64))
    k = rng.standard_normal((wl.B, 1, wl.T, 64))
    cos, sin = rope_cos_sin(wl.S, **KIMI_K2_ROPE)
    pos = rope_positions(wl.B, wl.T, past_len=wl.past_len)
    n, t0 = 0, time.perf_counter()
    while True:
        apply_rope(q, pos, cos, sin)
        apply_rope(k, pos, cos, sin)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": rope_apply_bytes(wl) * n / el / 1e9, "unit": "GB/s", "cores": blas_threads(),
            "host_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"the whole workload {n} times, {el:.1f} s"}


def run_varlen(wl, steps, warmup, seed=0, graph=True):
    """mla_attn_decode_varlen on a right-padded cache (inputs drawn on the
    device; the cache is far larger than the Infinity Cache)."""
    import torch
    import attention_mla_causal_amd as mla
    dev = torch.device("cuda:0")
    lens = varlen_seq_lens(wl.B, wl.cap, seed=seed)
    nbytes = varlen_bytes(wl, lens)
    log(f"[bench] {wl.name}: B={wl.B} H={wl.H} cap={wl.cap} sum(lens)={int(lens.sum())} steps={steps}")
    d = device_inputs(wl.cache(), dev, seed=seed)
    sl = torch.as_tensor(lens, device=dev)
    out = torch.empty((wl.B, wl.H, 1, 128), dtype=torch.bfloat16, device=dev)
    need = mla.mla_attn_decode_varlen_workspace_bytes(wl.B, wl.H, wl.cap)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)

    def step(i):
        mla.mla_attn_decode_varlen(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], sl, wl.cap,
                                   wl.softmax_scale, out=out, workspace=ws)

    if graph:
        ms, wall_ms = time_graph(step, steps, warmup)
    else:
        ms, wall_ms = time_eager(step, steps, warmup)
    gbs = nbytes / (ms * 1e-3) / 1e9
    kernel = "mla_decode_kernel"
    res = {
        "workload": wl.name, "B": wl.B, "H": wl.H, "T": 1, "cache_len": wl.cap,
        "sum_seq_lens": int(lens.sum()), "min_seq_len": int(lens.min()), "inputs": "device",
        "steps": steps, "timing": "hip_graph" if graph else "eager",
        "ms_per_step": ms, "wall_ms_per_step": wall_ms, "value": gbs, "unit": "GB/s",
        "algorithmic_bytes": nbytes,
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic(kernel, wl.name)},
    }
    del d
    torch.cuda.empty_cache()
    return res


def run_paged(wl, steps, warmup, seed=0, graph=True):
    """mla_attn_decode_paged with append on a shuffled block layout (inputs
    drawn on the device; every step appends the same rows to the same slots)."""
    import torch
    import attention_mla_causal_amd as mla
    dev = torch.device("cuda:0")
    lens = varlen_seq_lens(wl.B, wl.cap, seed=seed)
    table, nblocks = paged_layout(lens, wl.block_size, seed=seed)
    nbytes = paged_bytes(wl, lens)
    log(f"[bench] {wl.name}: B={wl.B} H={wl.H} block_size={wl.block_size} blocks={nblocks} "
        f"sum(lens)={int(lens.sum())} steps={steps}")
    d = paged_device_inputs(wl.B, wl.H, nblocks, wl.block_size, dev, seed=seed)
    tb = torch.as_tensor(table, device=dev)
    sl = torch.as_tensor(lens, device=dev)
    out = torch.empty((wl.B, wl.H, 1, 128), dtype=torch.bfloat16, device=dev)
    need = mla.mla_attn_decode_paged_workspace_bytes(wl.B, wl.H, wl.cap)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
    new = (d["k_nope_new"], d["k_pe_new"], d["v_new"])

    def step(i):
        mla.mla_attn_decode_paged(d["q_nope"], d["q_pe"], d["k_nope_pages"], d["k_pe_pages"],
                                  d["v_pages"], tb, sl, wl.cap, wl.softmax_scale, new=new, out=out,
                                  workspace=ws)

    if graph:
        ms, wall_ms = time_graph(step, steps, warmup)
    else:
        ms, wall_ms = time_eager(step, steps, warmup)
    gbs = nbytes / (ms * 1e-3) / 1e9
    kernel = "mla_decode_kernel"
    res = {
        "workload": wl.name, "B": wl.B, "H": wl.H, "T": 1, "block_size": wl.block_size,
        "num_blocks": nblocks, "sum_seq_lens": int(lens.sum()), "append": True, "inputs": "device",
        "steps": steps, "timing": "hip_graph" if graph else "eager",
        "ms_per_step": ms, "wall_ms_per_step": wall_ms, "value": gbs, "unit": "GB/s",
        "algorithmic_bytes": nbytes,
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic(kernel, wl.name)},
    }
    del d
    torch.cuda.empty_cache()
    return res


def run_latent(wl, steps, warmup, seed=0, copies=None, graph=True):
    """mla_attn_decode_latent, graph-timed (or eager) over rotating input copies (weights too)."""
    import torch
    import attention_mla_causal_amd as mla
    dev = torch.device("cuda:0")
    nbytes = latent_bytes(wl)
    if copies is None:
        copies = 1 if nbytes >= 2 * CACHE_BYTES else min(64, -(-2 * CACHE_BYTES // nbytes) + 1)
    log(f"[bench] {wl.name}: B={wl.B} H={wl.H} S={wl.S} copies={copies} steps={steps}")
    if wl.B * wl.S * 512 * 2 > (1 << 28):
        sets = [latent_device_inputs(wl, dev, seed=seed + c) for c in range(copies)]
        recipe = "device"
    else:
        sets = [{k: to_dev(v, dev) for k, v in latent_host_inputs(wl, seed=seed + c).items()}
                for c in range(copies)]
        recipe = "host"
    out = torch.empty((wl.B, wl.H, 1, 128), dtype=torch.bfloat16, device=dev)
    need = mla.mla_attn_decode_latent_workspace_bytes(wl.B, wl.H, wl.S)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)

    def step(i):
        d = sets[i % copies]
        mla.mla_attn_decode_latent(d["q_nope"], d["q_pe"], d["c_kv"], d["k_pe"], d["w_kv_b"],
                                   wl.past_len, wl.softmax_scale, out=out, workspace=ws)

    if graph:
        ms, wall_ms = time_graph(step, steps, warmup)
    else:
        ms, wall_ms = time_eager(step, steps, warmup)
    gbs = nbytes / (ms * 1e-3) / 1e9
    tfs = latent_flops(wl) / (ms * 1e-3) / 1e12
    kernel = "mla_attn_decode_latent"  # whole call: absorb, attention, merge, up-projection
    res = {
        "workload": wl.name, "B": wl.B, "H": wl.H, "T": 1, "past_len": wl.past_len, "S": wl.S,
        "inputs": recipe, "input_copies": copies, "steps": steps,
        "timing": "hip_graph" if graph else "eager",
        "ms_per_step": ms, "wall_ms_per_step": wall_ms, "value": gbs, "unit": "GB/s",
        "algorithmic_bytes": nbytes, "algorithmic_flops": latent_flops(wl), "tflops": tfs,
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic(kernel, wl.name)},
    }
    del sets
    torch.cuda.empty_cache()
    return res


def run_prefill(wl, steps, warmup, seed=0):
    import torch
    import attention_mla_causal_amd as mla
    dev = torch.device("cuda:0")
    log(f"[bench] {wl.name}: B={wl.B} H={wl.H} T={wl.T} P={wl.past_len} steps={steps}")
    x = host_inputs(wl, seed=seed)
    d = {k: to_dev(v, dev) for k, v in x.items()}
    out = torch.empty((wl.B, wl.H, wl.T, 128), dtype=torch.bfloat16, device=dev)
    need = mla.mla_attn_prefill_workspace_bytes(wl.B, wl.H, wl.T, wl.S)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)  # key-range split partials

    def step(i):
        mla.mla_attn_prefill(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], wl.past_len,
                             wl.softmax_scale, out=out, workspace=ws)

    ms, wall_ms = time_eager(step, steps, warmup)
    flops = prefill_flops(wl)
    tfs = flops / (ms * 1e-3) / 1e12
    kernel = "mla_prefill_kernel"
    res = {
        "workload": wl.name, "B": wl.B, "H": wl.H, "T": wl.T, "past_len": wl.past_len, "S": wl.S,
        "std": wl.std, "inputs": "host", "steps": steps, "timing": "eager",
        "key_splits": max(1, need and int(need // (wl.B * wl.H * wl.T * 130 * 4)) or 1),
        "ms_per_step": ms, "wall_ms_per_step": wall_ms, "value": tfs, "unit": "TFLOP/s",
        "algorithmic_flops": flops,
        "roofline": {"bound": "mfma", "kernel": kernel, "achieved": tfs, "peak": MFMA_BF16_PEAK_TFS,
                     "unit": "TFLOP/s", "frac": tfs / MFMA_BF16_PEAK_TFS,
                     "traffic": measured_traffic(kernel, wl.name)},
    }
    del d
    torch.cuda.empty_cache()
    return res, x


def run_prefill_varlen(wl, steps, warmup, seed=0):
    """mla_attn_prefill_varlen on a right-padded batch of chunked prefills
    (inputs drawn on the device)."""
    import torch
    import attention_mla_causal_amd as mla
    dev = torch.device("cuda:0")
    tq, pl = varlen_prefill_lens(wl.B, wl.max_q, wl.max_kv, seed=seed)
    flops = varlen_prefill_flops(wl, tq, pl)
    log(f"[bench] {wl.name}: B={wl.B} H={wl.H} max_q={wl.max_q} max_kv={wl.max_kv} "
        f"sum(q_lens)={int(tq.sum())} steps={steps}")
    d = device_inputs(wl.padded(), dev, seed=seed)
    ql = torch.as_tensor(tq, device=dev)
    pp = torch.as_tensor(pl, device=dev)
    out = torch.empty((wl.B, wl.H, wl.max_q, 128), dtype=torch.bfloat16, device=dev)

    def step(i):
        mla.mla_attn_prefill_varlen(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], ql, pp,
                                    wl.softmax_scale, out=out)

    ms, wall_ms = time_eager(step, steps, warmup)
    tfs = flops / (ms * 1e-3) / 1e12
    kernel = "mla_prefill_kernel"
    res = {
        "workload": wl.name, "B": wl.B, "H": wl.H, "max_q_len": wl.max_q, "max_kv_len": wl.max_kv,
        "q_lens": tq.tolist(), "past_lens": pl.tolist(), "std": wl.std, "inputs": "device",
        "steps": steps, "timing": "eager", "ms_per_step": ms, "wall_ms_per_step": wall_ms,
        "value": tfs, "unit": "TFLOP/s", "algorithmic_flops": flops,
        "roofline": {"bound": "mfma", "kernel": "mla_prefill_varlen_kernel", "achieved": tfs,
                     "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s", "frac": tfs / MFMA_BF16_PEAK_TFS,
                     "traffic": measured_traffic(kernel, wl.name)},
    }
    del d
    torch.cuda.empty_cache()
    return res


def run_masked(wl, steps, warmup, seed=0, graph=True):
    """mla_attn_decode_masked / mla_attn_prefill_masked with a left-padding 2D
    mask (inputs drawn on the device). Decode is graph-timed, prefill eager."""
    import torch
    import attention_mla_causal_amd as mla
    dev = torch.device("cuda:0")
    pads = left_pads(wl, seed=seed)
    mask = torch.as_tensor(left_pad_mask(wl.S, pads), device=dev)
    d = device_inputs(wl, dev, seed=seed)
    log(f"[bench] {wl.name}: B={wl.B} H={wl.H} T={wl.T} S={wl.S} sum(pads)={int(pads.sum())} steps={steps}")
    out = torch.empty((wl.B, wl.H, wl.T, 128), dtype=torch.bfloat16, device=dev)
    if wl.T == 1:
        need = mla.mla_attn_decode_varlen_workspace_bytes(wl.B, wl.H, wl.S)
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)

        def step(i):
            mla.mla_attn_decode_masked(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], mask,
                                       wl.past_len, wl.softmax_scale, out=out, workspace=ws)

        ms, wall_ms = (time_graph if graph else time_eager)(step, steps, warmup)
        work = masked_decode_bytes(wl, pads)
        rate, unit, bound, peak, kernel = work / (ms * 1e-3) / 1e9, "GB/s", "hbm", HBM_PEAK_GBS, "mla_decode_masked_kernel"
    else:
        def step(i):
            mla.mla_attn_prefill_masked(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], mask,
                                        wl.past_len, wl.softmax_scale, out=out)

        ms, wall_ms = time_eager(step, steps, warmup)
        work = masked_prefill_flops(wl, pads)
        rate, unit, bound, peak, kernel = (work / (ms * 1e-3) / 1e12, "TFLOP/s", "mfma", MFMA_BF16_PEAK_TFS,
                                           "mla_prefill_masked_kernel")
    res = {
        "workload": wl.name, "B": wl.B, "H": wl.H, "T": wl.T, "past_len": wl.past_len, "S": wl.S,
        "left_pads": pads.tolist() if wl.B <= 8 else f"sum {int(pads.sum())}", "inputs": "device",
        "steps": steps, "timing": "hip_graph" if wl.T == 1 and graph else "eager",
        "ms_per_step": ms, "wall_ms_per_step": wall_ms, "value": rate, "unit": unit,
        ("algorithmic_bytes" if wl.T == 1 else "algorithmic_flops"): work,
        "roofline": {"bound": bound, "kernel": kernel, "achieved": rate, "peak": peak, "unit": unit,
                     "frac": rate / peak, "traffic": measured_traffic(
                         "mla_decode_kernel" if wl.T == 1 else "mla_prefill_kernel", wl.name)},
    }
    del d
    torch.cuda.empty_cache()
    return res


def cpu_baseline_decode(wl, seconds):
    """The fp64 oracle on the whole decode workload, repeated for ~`seconds`."""
    from oracle import mla_attention
    x = host_inputs(wl, seed=0)
    reps, t0 = 0, time.perf_counter()
    while True:
        mla_attention(x["q_nope"], x["q_pe"], x["k_nope"], x["k_pe"], x["v"], wl.past_len, wl.softmax_scale)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 1000:
            break
    per = el / reps
    return {"value": decode_bytes(wl) / per / 1e9, "unit": "GB/s", "cores": blas_threads(),
            "host_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"whole workload (B={wl.B} H={wl.H} S={wl.S}), {reps} repetitions, {el:.1f} s",
            "s_per_step": per}


def cpu_baseline_latent(wl, seconds):
    """The fp64 latent-cache oracle on sampled (batch, head) rows until ~`seconds`
    pass; effective rate = the workload's algorithmic bytes scaled by the share
    of rows done / time."""
    from oracle import mla_decode_latent_rows
    if wl.B * wl.S * 512 * 2 > (1 << 28):
        return None  # the host copy of the batched cache alone would take minutes to draw
    x = latent_host_inputs(wl, seed=0)
    rows, t0 = 0, time.perf_counter()
    while rows < wl.B * wl.H:
        b, h = divmod(rows, wl.H)
        mla_decode_latent_rows(x["q_nope"], x["q_pe"], x["c_kv"], x["k_pe"], x["w_kv_b"], wl.past_len,
                               wl.softmax_scale, [(b, h)])
        rows += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": latent_bytes(wl) * rows / (wl.B * wl.H) / el / 1e9, "unit": "GB/s",
            "cores": blas_threads(), "host_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{rows} of {wl.B * wl.H} (batch, head) rows, {el:.1f} s"}


def cpu_baseline_head_rows(name, run_one, units, work_per_unit, total_work, unit, seconds):
    """Time `run_one(k)` for k = 0, 1, ... (each one unit of the workload,
    doing work_per_unit(k)) until ~`seconds` pass or the units run out;
    effective rate = work done / time, in the workload's unit."""
    done, k, t0 = 0.0, 0, time.perf_counter()
    while k < units:
        run_one(k)
        done += work_per_unit(k)
        k += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    scale = 1e12 if unit == "TFLOP/s" else 1e9
    return {"value": done / el / scale, "unit": unit, "cores": blas_threads(),
            "host_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{name}: {k} of {units} units, {done / total_work:.3%} of the workload, {el:.1f} s"}


def cpu_baseline_varlen_prefill(wl, seconds, seed=0):
    """The fp64 padded-batch oracle, one (sequence, head) at a time from the
    longest sequence on, on host-drawn inputs of the first sequence's shape."""
    from oracle import mla_prefill_varlen
    from seeded_inputs import random_inputs
    tq, pl = varlen_prefill_lens(wl.B, wl.max_q, wl.max_kv, seed=seed)
    T0, P0 = int(tq[0]), int(pl[0])
    x = random_inputs(1, 1, wl.max_q, wl.max_kv - wl.max_q, seed=seed, std=wl.std)
    per = 2 * (192 + 128) * (T0 * P0 + T0 * (T0 + 1) // 2)

    def one(k):
        mla_prefill_varlen(x["q_nope"], x["q_pe"], x["k_nope"], x["k_pe"], x["v"], np.array([T0]),
                           np.array([P0]), wl.softmax_scale)

    return cpu_baseline_head_rows("heads of the longest sequence", one, wl.H, lambda k: per,
                                  varlen_prefill_flops(wl, tq, pl), "TFLOP/s", seconds)


def cpu_baseline_masked(wl, seconds, seed=0):
    """The fp64 2D-mask oracle, one head of the first sequence at a time
    (prefill: its queries in blocks of 64 rows; decode: its one query)."""
    from oracle import mla_attention_masked
    from seeded_inputs import random_inputs
    pads = left_pads(wl, seed=seed)
    mask = left_pad_mask(wl.S, pads)[:1]
    x = random_inputs(1, 1, wl.T, wl.past_len, seed=seed)
    if wl.T == 1:
        per = masked_decode_bytes(wl, pads[:1]) / wl.H

        def one(k):
            mla_attention_masked(x["q_nope"], x["q_pe"], x["k_nope"], x["k_pe"], x["v"], mask,
                                 wl.past_len, wl.softmax_scale)

        return cpu_baseline_head_rows("heads of sequence 0", one, wl.H, lambda k: per,
                                      masked_decode_bytes(wl, pads), "GB/s", seconds)
    rows = 64
    nblk = -(-wl.T // rows)
    p0 = int(pads[0])

    def blk_pairs(k):
        i = np.arange(k * rows, min(wl.T, (k + 1) * rows), dtype=np.int64)
        return 2 * (192 + 128) * int(np.clip(wl.past_len + i - p0 + 1, 0, None).sum())

    def one(k):
        lo, hi = k * rows, min(wl.T, (k + 1) * rows)
        S_hi = wl.past_len + hi
        mla_attention_masked(x["q_nope"][:, :, lo:hi], x["q_pe"][:, :, lo:hi], x["k_nope"][:, :, :S_hi],
                             x["k_pe"][:, :, :S_hi], x["v"][:, :, :S_hi], mask[:, :S_hi],
                             wl.past_len + lo, wl.softmax_scale)

    return cpu_baseline_head_rows("64-query blocks of head 0, sequence 0", one, nblk, blk_pairs,
                                  masked_prefill_flops(wl, pads), "TFLOP/s", seconds)


def cpu_baseline_prefill(wl, x, seconds):
    """The fp64 oracle on the first heads of the workload until ~`seconds` pass;
    effective rate = algorithmic flops of the heads done / time."""
    from oracle import mla_attention
    heads, t0 = 0, time.perf_counter()
    while heads < wl.H:
        h = heads
        mla_attention(x["q_nope"][:, h:h + 1], x["q_pe"][:, h:h + 1], x["k_nope"][:, h:h + 1], x["k_pe"],
                      x["v"][:, h:h + 1], wl.past_len, wl.softmax_scale)
        heads += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per_head_flops = prefill_flops(wl) / (wl.B * wl.H)
    return {"value": per_head_flops * heads * wl.B / el / 1e12, "unit": "TFLOP/s", "cores": blas_threads(),
            "host_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{heads} of {wl.H} heads (batch 0), all {wl.T} queries, {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_p1000",
                    choices=sorted(WORKLOADS) + sorted(SHARD_WORKLOADS) + sorted(LATENT_WORKLOADS)
                    + sorted(VARLEN_WORKLOADS)
                    + sorted(PAGED_WORKLOADS) + sorted(VARLEN_PREFILL_WORKLOADS) + sorted(MASKED_WORKLOADS)
                    + ["decode_p1000_rope", "rope_chunked_prefill"])
    ap.add_argument("--no-extra", action="store_true", help="only the headline workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--extra-steps", type=int, default=20)
    ap.add_argument("--eager", action="store_true",
                    help="time decode with plain launches instead of a HIP graph (profiler runs)")
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
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the attention core has no cross-GPU path in this library; heads shard with no "
              "communication, so per-GPU throughput is the single-GPU figure.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    torch.cuda.synchronize()
    if args.workload == "decode_p1000_rope":
        wl = WORKLOADS["decode_p1000"]
        head = run_decode(wl, args.steps, args.warmup, graph=not args.eager, rope=True)
        cpu = None
    elif args.workload == "rope_chunked_prefill":
        wl = WORKLOADS["chunked_prefill"]
        head = run_rope_apply(wl, args.steps, args.warmup, graph=not args.eager)
        cpu = None
    elif args.workload in MASKED_WORKLOADS:
        wl = MASKED_WORKLOADS[args.workload]
        head = run_masked(wl, args.steps, args.warmup, graph=not args.eager)
        cpu = None
    elif args.workload in VARLEN_PREFILL_WORKLOADS:
        wl = VARLEN_PREFILL_WORKLOADS[args.workload]
        head = run_prefill_varlen(wl, args.steps, args.warmup)
        cpu = None
    elif args.workload in PAGED_WORKLOADS:
        wl = PAGED_WORKLOADS[args.workload]
        head = run_paged(wl, args.steps, args.warmup, graph=not args.eager)
        cpu = None
    elif args.workload in VARLEN_WORKLOADS:
        wl = VARLEN_WORKLOADS[args.workload]
        head = run_varlen(wl, args.steps, args.warmup, graph=not args.eager)
        cpu = None
    elif args.workload in LATENT_WORKLOADS:
        wl = LATENT_WORKLOADS[args.workload]
        head = run_latent(wl, args.steps, args.warmup, graph=not args.eager)
        cpu = None if args.no_cpu else cpu_baseline_latent(wl, args.cpu_seconds)
    elif {**WORKLOADS, **SHARD_WORKLOADS}[args.workload].T == 1:
        wl = {**WORKLOADS, **SHARD_WORKLOADS}[args.workload]
        head = run_decode(wl, args.steps, args.warmup, graph=not args.eager)
        cpu = None if args.no_cpu else cpu_baseline_decode(wl, args.cpu_seconds)
    else:
        wl = {**WORKLOADS, **SHARD_WORKLOADS}[args.workload]
        head, x = run_prefill(wl, args.steps, args.warmup)
        cpu = None if args.no_cpu else cpu_baseline_prefill(wl, x, args.cpu_seconds)
        del x

    workloads = {}
    if not args.no_extra:
        for name in ("decode_p1000", "batched_decode", "causal_prefill", "chunked_prefill"):
            if name == wl.name:
                continue
            w = WORKLOADS[name]
            if w.T == 1:
                r = run_decode(w, args.extra_steps, 3)
            else:
                r, x = run_prefill(w, args.extra_steps, 2)
                if not args.no_cpu:
                    r["cpu_baseline"] = cpu_baseline_prefill(w, x, min(args.cpu_seconds, 5.0))
                del x
            workloads[name] = r
        for name, w in SHARD_WORKLOADS.items():  # one GPU's share of 64 heads over 8 GPUs
            if w.T == 1:
                workloads[name] = run_decode(w, args.extra_steps, 3)
            else:
                workloads[name], x = run_prefill(w, args.extra_steps, 2)
                del x
        for name, w in VARLEN_WORKLOADS.items():
            if name != wl.name:
                workloads[name] = run_varlen(w, args.extra_steps, 3)
        for name, w in PAGED_WORKLOADS.items():
            if name != wl.name:
                workloads[name] = run_paged(w, args.extra_steps, 3)
        for name, w in VARLEN_PREFILL_WORKLOADS.items():
            if name != wl.name:
                workloads[name] = run_prefill_varlen(w, args.extra_steps, 2)
                if not args.no_cpu:
                    workloads[name]["cpu_baseline"] = cpu_baseline_varlen_prefill(w, min(args.cpu_seconds, 5.0))
        for name, w in MASKED_WORKLOADS.items():
            if name != wl.name:
                workloads[name] = run_masked(w, args.extra_steps, 2)
                if not args.no_cpu:
                    workloads[name]["cpu_baseline"] = cpu_baseline_masked(w, min(args.cpu_seconds, 5.0))
        # the rotary prologue: fused into the short decode, and on its own over
        # the chunked prefill's new tokens
        workloads["decode_p1000_rope"] = run_decode(WORKLOADS["decode_p1000"], 200, 20, rope=True)
        workloads["rope_chunked_prefill"] = run_rope_apply(WORKLOADS["chunked_prefill"], 200, 20)
        if not args.no_cpu:
            workloads["rope_chunked_prefill"]["cpu_baseline"] = cpu_baseline_rope_apply(
                WORKLOADS["chunked_prefill"], min(args.cpu_seconds, 3.0))
        for name, w in LATENT_WORKLOADS.items():
            if name == wl.name:
                continue
            workloads[name] = run_latent(w, 200 if w.B == 1 else args.extra_steps, 3)
            if not args.no_cpu:
                workloads[name]["cpu_baseline"] = cpu_baseline_latent(w, min(args.cpu_seconds, 5.0))

    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_min_seconds": RAMP_SECONDS,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {k: head[k] for k in ("workload", "B", "H", "T", "past_len", "S", "std", "inputs",
                                        "timing") if k in head},
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "workloads": workloads,
    }
    if "input_copies" in head:
        line["config"]["input_copies"] = head["input_copies"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
