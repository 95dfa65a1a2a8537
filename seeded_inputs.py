"""Seeded synthetic inputs for the MLA attention core, shared by tests and bench.

This module only draws numbers; it holds none of the attention arithmetic, so
both the fp64 oracle and the HIP library can be fed from it without sharing
any code with each other.

Workloads are shaped like the tensors on the Kimi K2 pages: 64 heads, 128
non-rotary + 64 rotary query/key dims with one rotary key shared by all heads,
128 value dims, bf16. The pages never give the distribution of these
activations, so they are i.i.d. normal draws.

Host recipe (all small and medium workloads):
  SeedSequence(seed).spawn(5) -> one child per tensor, in the order
  q_nope, q_pe, k_nope, k_pe, v; each child spawns one grandchild per batch
  index b; PCG64(grandchild).standard_normal(float32) * std; rounded to bf16
  with round-to-nearest-even on the fp32 bits; kept as uint16 bit patterns.
  Per-batch streams let a test regenerate a single batch of a large workload.

Latent-cache decode workloads (the compressed cache that kv_b_proj expands)
draw q_nope, q_pe, c_kv (the normalised 512-dim latent), k_pe and w_kv_b
(kv_b_proj's weight [64*256, 512]) the same way, in that order, with
std 1 for the activations and 1/sqrt(512) for the weight, so that the
decompressed keys and values have unit variance like the other workloads.
The weight has no batch index: its stream is the tensor child's first
grandchild.

Variable-length decode workloads (a preallocated cache of `cap` rows per
sequence, right-padded) draw the five tensors exactly as a decode workload
with S = cap, plus one length per sequence from PCG64(SeedSequence([seed,
1])): integers uniform in [1, cap], the first sequence set to cap so the
longest sequence fills the cache. The pages give no length mix; a uniform mix
over the cache stands in for a serving batch.

Paged-cache decode (blocks of `block_size` rows named by a table per
sequence): the tensors q_nope, q_pe, k_nope_pages [N,H,bs,128], k_pe_pages
[N,bs,64], v_pages [N,H,bs,128] and the appended token's k_nope_new,
k_pe_new, v_new are drawn in that order, one SeedSequence child each
(standard normal, bf16; on the device, drawn in chunks of at most 64 MiB of
fp32 along the leading index); the block layout gives sequence b ceil(L_b / bs)
blocks taken in order from a PCG64(SeedSequence([seed, 2])) permutation of
all blocks, table entries past a sequence's blocks left at 0.

Device recipe (workloads whose inputs exceed a few GiB of host work, i.e. the
batched decode): torch.Generator on the device seeded with `seed`, then for
each tensor in the same order torch.randn(float32) * std rounded to bf16 by
torch's round-to-nearest-even conversion. Tests copy the sampled slices of
these inputs back to the host for the oracle.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

NOPE, ROPE, VDIM = 128, 64, 128
TENSORS = ("q_nope", "q_pe", "k_nope", "k_pe", "v")


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    past_len: int
    std: float = 1.0
    # 192^-0.5 rounded to fp32; the scale is a 32-bit float at the C ABI.
    softmax_scale: float = float(np.float32(192.0 ** -0.5))

    @property
    def S(self) -> int:
        return self.past_len + self.T

    def shapes(self) -> dict:
        B, H, T, S = self.B, self.H, self.T, self.S
        return {
            "q_nope": (B, H, T, NOPE),
            "q_pe": (B, H, T, ROPE),
            "k_nope": (B, H, S, NOPE),
            "k_pe": (B, 1, S, ROPE),
            "v": (B, H, S, VDIM),
        }


# The five workloads: a tiny prefill, decode exactly as the "Similarities"
# page shows it (64 heads, 1 query, p=1000 -> 1001 keys), a batched decode, a
# causal prefill and a chunked prefill on top of a cache. "N(0,2)" for the
# chunked prefill is read as variance 2 (std sqrt 2).
WORKLOADS = {
    "tiny_prefill": Workload("tiny_prefill", B=1, H=4, T=16, past_len=0),
    "decode_p1000": Workload("decode_p1000", B=1, H=64, T=1, past_len=1000),
    "batched_decode": Workload("batched_decode", B=32, H=64, T=1, past_len=8191),
    "causal_prefill": Workload("causal_prefill", B=1, H=64, T=4096, past_len=0),
    "chunked_prefill": Workload("chunked_prefill", B=1, H=64, T=2048, past_len=14336,
                                std=float(np.sqrt(2.0))),
}


# One GPU's share when the 64 heads are split over 8 GPUs (heads shard with no
# exchange inside attention): the same shapes at H = 8.
SHARD_WORKLOADS = {
    "batched_decode_h8": Workload("batched_decode_h8", B=32, H=8, T=1, past_len=8191),
    "chunked_prefill_h8": Workload("chunked_prefill_h8", B=1, H=8, T=2048, past_len=14336,
                                   std=float(np.sqrt(2.0))),
}


KV_RANK = 512
LATENT_TENSORS = ("q_nope", "q_pe", "c_kv", "k_pe", "w_kv_b")


@dataclass(frozen=True)
class LatentWorkload:
    """Decode over the compressed cache: one query per sequence, S = past_len + 1."""
    name: str
    B: int
    H: int
    past_len: int
    softmax_scale: float = float(np.float32(192.0 ** -0.5))

    @property
    def S(self) -> int:
        return self.past_len + 1

    def shapes(self) -> dict:
        B, H, S = self.B, self.H, self.S
        return {
            "q_nope": (B, H, 1, NOPE),
            "q_pe": (B, H, 1, ROPE),
            "c_kv": (B, S, KV_RANK),
            "k_pe": (B, 1, S, ROPE),
            "w_kv_b": (1, H * (NOPE + VDIM), KV_RANK),  # leading 1: no batch index
        }

    @staticmethod
    def std(tensor: str) -> float:
        return float(1.0 / np.sqrt(KV_RANK)) if tensor == "w_kv_b" else 1.0


# The pages' decode (64 heads, p = 1000) and the batched decode, with the
# cache kept compressed.
LATENT_WORKLOADS = {
    "latent_decode_p1000": LatentWorkload("latent_decode_p1000", B=1, H=64, past_len=1000),
    "latent_batched_decode": LatentWorkload("latent_batched_decode", B=32, H=64, past_len=8191),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    r = np.where(nan, (u >> np.uint32(16)) | np.uint32(0x40), r)
    return r.astype(np.uint16)


def _batch_rng(seed: int, tensor: str, B: int, b: int, names=TENSORS) -> np.random.Generator:
    child = np.random.SeedSequence(seed).spawn(len(names))[names.index(tensor)]
    grand = child.spawn(B)[b]
    return np.random.Generator(np.random.PCG64(grand))


def tensor_batch(shape, tensor: str, b: int, seed: int = 0, std: float = 1.0) -> np.ndarray:
    """One batch slice [shape[1:]] of one tensor as bf16 bits (host recipe)."""
    g = _batch_rng(seed, tensor, shape[0], b)
    x = g.standard_normal(shape[1:], dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x)


def host_inputs(wl: Workload, seed: int = 0, std: float | None = None) -> dict:
    """All five inputs of a workload as uint16 bf16 bit arrays (host recipe)."""
    std = wl.std if std is None else std
    out = {}
    for name, shape in wl.shapes().items():
        arr = np.empty(shape, dtype=np.uint16)
        for b in range(shape[0]):
            arr[b] = tensor_batch(shape, name, b, seed, std)
        out[name] = arr
    return out


def latent_host_inputs(wl: LatentWorkload, seed: int = 0) -> dict:
    """The five latent-decode inputs as uint16 bf16 bit arrays (host recipe)."""
    out = {}
    for name, shape in wl.shapes().items():
        arr = np.empty(shape, dtype=np.uint16)
        for b in range(shape[0]):
            g = _batch_rng(seed, name, shape[0], b, LATENT_TENSORS)
            x = g.standard_normal(shape[1:], dtype=np.float32)
            x *= np.float32(wl.std(name))
            arr[b] = f32_to_bf16_bits(x)
        out[name] = arr[0] if name == "w_kv_b" else arr
    return out


def latent_random_inputs(B, H, past_len, seed=0) -> dict:
    """Host-recipe latent-decode inputs for an arbitrary shape."""
    return latent_host_inputs(LatentWorkload("custom", B, H, past_len), seed)


def latent_device_inputs(wl: LatentWorkload, device, seed: int = 0) -> dict:
    """The five latent-decode inputs drawn on a torch device (device recipe)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = {}
    for name, shape in wl.shapes().items():
        t = torch.empty(shape, dtype=torch.bfloat16, device=device)
        for b in range(shape[0]):
            x = torch.randn(shape[1:], generator=g, dtype=torch.float32, device=device)
            x.mul_(wl.std(name))
            t[b].copy_(x)
            del x
        out[name] = t[0] if name == "w_kv_b" else t
    return out


def random_inputs(B, H, T, past_len, seed=0, std=1.0) -> dict:
    """Host-recipe inputs for an arbitrary shape (edge-case tests)."""
    return host_inputs(Workload("custom", B, H, T, past_len, std), seed)


def device_inputs(wl: Workload, device, seed: int = 0, std: float | None = None) -> dict:
    """All five inputs drawn on a torch device (device recipe), bf16 tensors."""
    import torch

    std = wl.std if std is None else std
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = {}
    for name, shape in wl.shapes().items():
        t = torch.empty(shape, dtype=torch.bfloat16, device=device)
        # draw per batch so the fp32 temporary stays at one batch's size
        for b in range(shape[0]):
            x = torch.randn(shape[1:], generator=g, dtype=torch.float32, device=device)
            if std != 1.0:
                x.mul_(std)
            t[b].copy_(x)
            del x
        out[name] = t
    return out


@dataclass(frozen=True)
class VarlenWorkload:
    """Decode over a preallocated cache of `cap` rows per sequence; sequence b
    uses rows [0, L_b) (right padding)."""
    name: str
    B: int
    H: int
    cap: int
    softmax_scale: float = float(np.float32(192.0 ** -0.5))

    def cache(self) -> Workload:
        """The tensors: a decode workload with S = cap."""
        return Workload(self.name, self.B, self.H, 1, self.cap - 1)


VARLEN_WORKLOADS = {
    "varlen_batched_decode": VarlenWorkload("varlen_batched_decode", B=32, H=64, cap=8192),
}


def varlen_seq_lens(B: int, cap: int, seed: int = 0) -> np.ndarray:
    """Lengths [B] int32, uniform in [1, cap], the first one cap."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 1])))
    lens = g.integers(1, cap + 1, size=B).astype(np.int32)
    if B:
        lens[0] = cap
    return lens


@dataclass(frozen=True)
class VarlenPrefillWorkload:
    """A right-padded batch of chunked prefills: sequence b has T_b new
    queries over P_b cached keys, in slices of max_q query rows and max_kv key
    rows."""
    name: str
    B: int
    H: int
    max_q: int
    max_kv: int
    std: float = 1.0
    softmax_scale: float = float(np.float32(192.0 ** -0.5))

    def padded(self) -> Workload:
        """The tensors: a prefill workload with T = max_q, S = max_kv."""
        return Workload(self.name, self.B, self.H, self.max_q, self.max_kv - self.max_q, self.std)


# Eight chunked-prefill requests batched together, the longest being the
# chunked-prefill workload's own (2048 new queries over 14336 cached keys).
VARLEN_PREFILL_WORKLOADS = {
    "varlen_prefill": VarlenPrefillWorkload("varlen_prefill", B=8, H=64, max_q=2048, max_kv=16384,
                                            std=float(np.sqrt(2.0))),
}


def varlen_prefill_lens(B: int, max_q: int, max_kv: int, seed: int = 0):
    """(q_lens, past_lens) int32 [B]: T_b uniform in [1, max_q], P_b uniform in
    [0, max_kv - max_q]; the first sequence takes both maxima."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 3])))
    tq = g.integers(1, max_q + 1, size=B).astype(np.int32)
    pl = g.integers(0, max_kv - max_q + 1, size=B).astype(np.int32)
    if B:
        tq[0], pl[0] = max_q, max_kv - max_q
    return tq, pl


# The caller's 2D padding mask, left padding: sequence b's first pads[b] key
# positions are padding. A batched decode whose sequences end together (the
# batched-decode shape, lengths as the variable-length decode's), and a batch
# of left-padded prompts prefilled together (pads up to half the prompt).
MASKED_WORKLOADS = {
    "masked_batched_decode": Workload("masked_batched_decode", B=32, H=64, T=1, past_len=8191),
    "masked_prefill": Workload("masked_prefill", B=4, H=64, T=4096, past_len=0),
}


def left_pads(wl: Workload, seed: int = 0) -> np.ndarray:
    """Padding positions per sequence [B] int64. Decode: S - L_b with L_b the
    variable-length decode's lengths (uniform in [1, S], the first S). Prefill:
    uniform in [0, S/2], the first 0."""
    if wl.T == 1:
        return (wl.S - varlen_seq_lens(wl.B, wl.S, seed=seed)).astype(np.int64)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 4])))
    pads = g.integers(0, wl.S // 2 + 1, size=wl.B).astype(np.int64)
    if wl.B:
        pads[0] = 0
    return pads


def left_pad_mask(S: int, pads) -> np.ndarray:
    """The 2D mask [B, S] uint8: 0 on each sequence's padding, 1 after it."""
    return (np.arange(S)[None, :] >= np.asarray(pads)[:, None]).astype(np.uint8)


PAGED_TENSORS = ("q_nope", "q_pe", "k_nope_pages", "k_pe_pages", "v_pages",
                 "k_nope_new", "k_pe_new", "v_new")


def paged_layout(lens, block_size: int, seed: int = 0, spare: int = 0):
    """(block_table int32 [B, max_blocks], num_blocks): sequence b owns
    ceil(L_b / block_size) blocks, taken in order from a seeded permutation of
    all num_blocks = (sum of those) + spare blocks."""
    lens = np.asarray(lens, dtype=np.int64)
    need = [int(-(-L // block_size)) for L in lens]
    num_blocks = max(sum(need) + spare, 1)
    M = max(max(need) if need else 0, 1)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 2])))
    perm = g.permutation(num_blocks)
    table = np.zeros((len(lens), M), dtype=np.int32)
    k = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[k:k + n]
        k += n
    return table, num_blocks


def paged_shapes(B: int, H: int, num_blocks: int, block_size: int) -> dict:
    return {"q_nope": (B, H, 1, NOPE), "q_pe": (B, H, 1, ROPE),
            "k_nope_pages": (num_blocks, H, block_size, NOPE),
            "k_pe_pages": (num_blocks, block_size, ROPE),
            "v_pages": (num_blocks, H, block_size, VDIM),
            "k_nope_new": (B, H, 1, NOPE), "k_pe_new": (B, 1, 1, ROPE), "v_new": (B, H, 1, VDIM)}


def paged_host_inputs(B: int, H: int, num_blocks: int, block_size: int, seed: int = 0) -> dict:
    """The eight paged-decode tensors as uint16 bf16 bit arrays (host recipe)."""
    kids = np.random.SeedSequence(seed).spawn(len(PAGED_TENSORS))
    out = {}
    for name, shape in paged_shapes(B, H, num_blocks, block_size).items():
        g = np.random.Generator(np.random.PCG64(kids[PAGED_TENSORS.index(name)]))
        out[name] = f32_to_bf16_bits(g.standard_normal(shape, dtype=np.float32))
    return out


def paged_device_inputs(B: int, H: int, num_blocks: int, block_size: int, device, seed: int = 0) -> dict:
    """The eight paged-decode tensors drawn on a torch device (device recipe)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = {}
    for name, shape in paged_shapes(B, H, num_blocks, block_size).items():
        t = torch.empty(shape, dtype=torch.bfloat16, device=device)
        per = int(np.prod(shape[1:]))
        step = max(1, (64 << 20) // (4 * per))  # leading-index rows per draw (<= 64 MiB of fp32)
        for i in range(0, shape[0], step):
            n = min(step, shape[0] - i)
            t[i:i + n].copy_(torch.randn((n,) + tuple(shape[1:]), generator=g, dtype=torch.float32,
                                         device=device))
        out[name] = t
    return out


@dataclass(frozen=True)
class PagedWorkload:
    """Decode with append over a paged cache: lengths as the variable-length
    workload (uniform in [1, cap], first at cap), blocks of block_size rows."""
    name: str
    B: int
    H: int
    cap: int
    block_size: int
    softmax_scale: float = float(np.float32(192.0 ** -0.5))


PAGED_WORKLOADS = {
    "paged_batched_decode": PagedWorkload("paged_batched_decode", B=32, H=64, cap=8192, block_size=64),
}
