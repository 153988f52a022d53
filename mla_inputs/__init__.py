"""Seeded synthetic inputs for MLA decode over a paged latent KV cache.

This module only draws random numbers and lays them out. It holds none of the
decode arithmetic (no scores, no softmax, no weighted sums). Both the CPU oracle
and the HIP path are fed from here: the tests and the benchmark draw a case once
and hand the same bytes to each side.

Shapes follow the MLA decode problem: each cached token is one 576-wide latent row
(512 latent dims followed by 64 rope dims). All query heads share the rows, and
the first 512 dims of a row also serve as its value vector. Rows live in 64-token
pages; a per-sequence block table maps logical block j to a physical page.

Draw order for a case (fixed, so a seed names one case): cache_seqlens, page
permutation, q, kv.  Values are N(0, 1) drawn in float32; for bf16 cases they
are rounded to bf16 with round-to-nearest-even here on the host, so both sides
read identical bits.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

D_QK = 576        # latent (512) + rope (64)
D_V = 512         # value width = first 512 dims of each cached row
PAGE = 64         # tokens per page (= tokens per KV block)
SCALE_192 = 192.0 ** -0.5

DTYPE_F32 = "f32"
DTYPE_BF16 = "bf16"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  NaN stays NaN (quiet bit forced).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = (u + 0x7FFF + lsb) >> 16
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Case:
    """One decode problem.  Array layouts (all C-contiguous):

    q:            [B, T, H, 576]   float32 values (exactly representable in `dtype`)
    kv:           [num_pages, 64, 576] float32 values
    q_bits/kv_bits: uint16 bf16 patterns of q/kv when dtype == "bf16", else None
    block_table:  [B, max_blocks] int32, entries past ceil(L/64) hold -1
    cache_seqlens:[B] int32, tokens in the cache (including the T new tokens)
    """
    name: str
    dtype: str
    batch: int
    q_len: int
    num_heads: int
    causal: bool
    scale: float
    cache_seqlens: np.ndarray
    block_table: np.ndarray
    q: np.ndarray
    kv: np.ndarray
    q_bits: np.ndarray | None
    kv_bits: np.ndarray | None
    seed: int

    @property
    def num_pages(self) -> int:
        return int(self.kv.shape[0])

    @property
    def rows(self) -> int:
        return self.q_len * self.num_heads

    def q_array(self) -> np.ndarray:
        """q in its storage dtype: uint16 bf16 bits or float32."""
        return self.q_bits if self.dtype == DTYPE_BF16 else self.q

    def kv_array(self) -> np.ndarray:
        return self.kv_bits if self.dtype == DTYPE_BF16 else self.kv


def _normal(rng: np.random.Generator, shape, dtype: str):
    vals = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == DTYPE_BF16:
        bits = f32_to_bf16_bits(vals)
        return bf16_bits_to_f32(bits).reshape(shape), bits.reshape(shape)
    return vals, None


def make_case(*, batch: int, q_len: int, num_heads: int, seqlens, dtype: str = DTYPE_BF16,
              causal: bool = False, scale: float = SCALE_192, permute_pages: bool = True,
              seed: int = 0, extra_pages: int = 0, name: str = "case",
              seqlen_range: tuple[int, int] | None = None) -> Case:
    """Draw one case.

    seqlens: int (every sequence), a list of ints, or None with `seqlen_range`
    = (lo, hi) for lengths uniform in [lo, hi] (drawn first from the seed).
    extra_pages: unused pool pages appended after the used ones (for poison tests).
    """
    rng = np.random.default_rng(seed)
    if seqlens is None:
        lo, hi = seqlen_range
        lens = rng.integers(lo, hi + 1, size=batch, dtype=np.int64)
    elif np.isscalar(seqlens):
        lens = np.full(batch, int(seqlens), dtype=np.int64)
    else:
        lens = np.asarray(seqlens, dtype=np.int64)
        assert lens.shape == (batch,)
    lens = lens.astype(np.int32)
    nblk = [(int(L) + PAGE - 1) // PAGE for L in lens]
    used = int(sum(nblk))
    num_pages = used + int(extra_pages)
    max_blocks = max(1, max(nblk) if nblk else 1)
    if permute_pages:
        perm = rng.permutation(num_pages).astype(np.int32)
    else:
        perm = np.arange(num_pages, dtype=np.int32)
    bt = np.full((batch, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(batch):
        bt[b, :nblk[b]] = perm[off:off + nblk[b]]
        off += nblk[b]
    q, q_bits = _normal(rng, (batch, q_len, num_heads, D_QK), dtype)
    kv, kv_bits = _normal(rng, (max(num_pages, 1), PAGE, D_QK), dtype)
    return Case(name=name, dtype=dtype, batch=batch, q_len=q_len, num_heads=num_heads,
                causal=bool(causal), scale=float(scale), cache_seqlens=lens, block_table=bt,
                q=q, kv=kv, q_bits=q_bits, kv_bits=kv_bits, seed=seed)


# The five workloads of the decode benchmark.  Seeds are 1000 + index.
CONFIGS = {
    0: dict(name="tiny_fp32_b1_h16_l256", batch=1, q_len=1, num_heads=16, seqlens=256,
            dtype=DTYPE_F32, permute_pages=False),
    1: dict(name="b64_h128_l4096", batch=64, q_len=1, num_heads=128, seqlens=4096,
            dtype=DTYPE_BF16),
    2: dict(name="ragged_b128_h128_l1to8192", batch=128, q_len=1, num_heads=128, seqlens=None,
            seqlen_range=(1, 8192), dtype=DTYPE_BF16),
    3: dict(name="long_b8_h128_l32768", batch=8, q_len=1, num_heads=128, seqlens=32768,
            dtype=DTYPE_BF16),
    4: dict(name="spec_b64_h16_t2_l4096_causal", batch=64, q_len=2, num_heads=16, seqlens=4096,
            dtype=DTYPE_BF16, causal=True),
}


def make_config(index: int, seed: int | None = None) -> Case:
    """Draw workload `index` (0..4) with seed 1000 + index unless given."""
    cfg = dict(CONFIGS[index])
    return make_case(seed=1000 + index if seed is None else seed, **cfg)


def make_sinks(num_heads: int, seed: int, lo: float = -4.0, hi: float = 12.0) -> np.ndarray:
    """Per-head attention-sink logits, float32, uniform on [lo, hi).  The default range
    spans the natural-log sums of exp that N(0, 1) inputs at scale 192^-0.5 give for one
    to 8192 keys (about 2 to 11), so some sinks barely count and some dominate."""
    rng = np.random.default_rng(seed)
    return rng.uniform(lo, hi, size=num_heads).astype(np.float32)


def make_topk_indices(cache_seqlens, q_len: int, topk: int, seed: int, pad_frac: float = 0.0,
                      dup_frac: float = 0.0) -> np.ndarray:
    """Sparse token lists [B, q_len, topk] int32 standing in for a top-k indexer's output
    (which needs trained weights): for each (b, t), min(topk, L_b) distinct positions
    of [0, L_b) in random order, the rest -1.  pad_frac of the entries are then turned
    into -1 and dup_frac into copies of another entry of the same list."""
    rng = np.random.default_rng(seed)
    B = len(cache_seqlens)
    out = np.full((B, q_len, topk), -1, dtype=np.int32)
    for b in range(B):
        L = int(cache_seqlens[b])
        for t in range(q_len):
            k = min(topk, max(L, 0))
            if k:
                out[b, t, :k] = rng.choice(L, size=k, replace=False)
            if pad_frac:
                out[b, t, rng.random(topk) < pad_frac] = -1
            if dup_frac and k:
                src = out[b, t, rng.integers(0, k, size=topk)]
                sel = rng.random(topk) < dup_frac
                out[b, t, sel] = src[sel]
    return out


def poison_unused(case: Case, value=np.nan) -> None:
    """Overwrite every KV slot no query may read (tail slots of each sequence's last
    page and every page not named by a block table) with `value`, in place."""
    used = np.zeros(case.num_pages, dtype=bool)
    for b in range(case.batch):
        L = int(case.cache_seqlens[b])
        nb = (L + PAGE - 1) // PAGE
        for j in range(nb):
            used[case.block_table[b, j]] = True
        if nb and L % PAGE:
            page = case.block_table[b, nb - 1]
            case.kv[page, L % PAGE:, :] = value
    case.kv[~used] = value
    if case.dtype == DTYPE_BF16:
        case.kv_bits = f32_to_bf16_bits(case.kv).reshape(case.kv.shape)
