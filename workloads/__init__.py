"""Seeded synthetic inputs for the selected-index NoPE MLA paged decode.

This module only draws inputs: random latents quantised to FP8 E4M3FN with a
library cast, BF16 queries, shuffled block tables, and selection rows with
the structure of each workload. It holds none of the decode's arithmetic and
imports neither the oracle nor the HIP binding; both sides consume what it
makes.

Workloads (sizes from the pages' GLM-5.3 decode shapes; see the module-level
WORKLOADS table):
  tiny    2 rows, 4 heads, D=64, B=16, seq_lens {100, 173}, 32 pages
  glm     32 rows, 64 heads, D=512, B=64, seq_len 8192, 4096 pages,
          2048 ids = 512 distinct pools of 4 contiguous positions
  long    128 rows, 64 heads, D=512, B=64, seq_len 131072, one 24 GiB pool
          (786432 pages), 2048 distinct ids: 70% pool-aligned runs of 4,
          30% singletons
  verify  64 sequences x 4 consecutive rows = 256 rows, 64 heads, base
          length U[4096, 32768]; the rows of a sequence share 60% of ids
  ragged  256 rows, 16 heads, seq_len log-uniform in [16, 65536]; short
          rows pad with holes, long rows carry 30% repeats and 15% holes
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

FP8_MAX = 448.0  # largest finite E4M3FN magnitude

WORKLOADS = {
    # name: (rows, heads, D, block_size, kpool, width, sm_scale, k_scale, sigma)
    "tiny": dict(rows=2, heads=4, D=64, block_size=16, kpool=4, width=32,
                 sm_scale=1.0 / math.sqrt(64), k_scale=0.05, sigma=1.0),
    "glm": dict(rows=32, heads=64, D=512, block_size=64, kpool=4, width=2048,
                sm_scale=1.0 / math.sqrt(256), k_scale=0.02, sigma=1.0),
    "long": dict(rows=128, heads=64, D=512, block_size=64, kpool=4, width=2048,
                 sm_scale=1.0 / math.sqrt(256), k_scale=0.02, sigma=1.0),
    "verify": dict(rows=256, heads=64, D=512, block_size=64, kpool=4, width=2048,
                   sm_scale=1.0 / math.sqrt(256), k_scale=0.02, sigma=1.0),
    "ragged": dict(rows=256, heads=16, D=512, block_size=64, kpool=4, width=2048,
                   sm_scale=1.0 / math.sqrt(256), k_scale=0.02, sigma=2.0),
}
SEEDS = {"tiny": 1000, "glm": 1001, "long": 1002, "verify": 1003, "ragged": 1004}


@dataclasses.dataclass
class Workload:
    name: str
    rows: int
    heads: int
    D: int
    block_size: int
    kpool: int
    width: int
    bt_stride: int
    cache_stride_bytes: int
    max_seq_len: int
    num_pages: int
    sm_scale: float
    k_scale: float
    v_scale: float
    sigma: float
    seed: int
    q_bits: np.ndarray          # [R, H, D] uint16 (bf16 bit patterns)
    block_tables: np.ndarray    # [R, bt_stride] int32
    seq_lens: np.ndarray        # [R] int32
    sel: np.ndarray             # [R, W] int32
    pool: Optional[np.ndarray] = None  # [num_pages * block_size * token_bytes] uint8, host pools only
    rope: int = 0               # rope-tail bytes each token carries after its D latent bytes

    @property
    def pool_bytes(self) -> int:
        return self.num_pages * self.cache_stride_bytes

    @property
    def token_bytes(self) -> int:
        return self.D + self.rope


# ----------------------------------------------------------------- primitives

def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round-to-nearest-even (torch cast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def fp8_codes_from_f32(x: np.ndarray) -> np.ndarray:
    """float32 -> FP8 E4M3FN codes: clamp to +-448 first (saturate, never NaN),
    then torch's round-to-nearest-even cast."""
    import torch
    t = torch.from_numpy(np.clip(np.ascontiguousarray(x, dtype=np.float32),
                                 -FP8_MAX, FP8_MAX))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def host_pool(rng: np.random.Generator, num_pages: int, block_size: int, D: int,
              sigma: float, k_scale: float) -> np.ndarray:
    """Latents x ~ N(0, sigma^2), stored as fp8(x / k_scale)."""
    n = num_pages * block_size * D
    x = rng.standard_normal(n, dtype=np.float32) * np.float32(sigma / k_scale)
    return fp8_codes_from_f32(x)


def device_pool(num_pages: int, block_size: int, D: int, sigma: float,
                k_scale: float, seed: int, device="cuda"):
    """The same recipe drawn on the GPU in 256 MiB slabs (for pools too large
    to draw on the host). Returns a torch uint8 tensor."""
    import torch
    n = num_pages * block_size * D
    pool = torch.empty(n, dtype=torch.uint8, device=device)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    slab = 1 << 28
    scale = sigma / k_scale
    for s in range(0, n, slab):
        e = min(n, s + slab)
        x = torch.randn(e - s, generator=g, device=device, dtype=torch.float32)
        x.mul_(scale).clamp_(-FP8_MAX, FP8_MAX)
        pool[s:e].copy_(x.to(torch.float8_e4m3fn).view(torch.uint8))
        del x
    return pool


def _shuffle_rows(rng, sel):
    for r in range(sel.shape[0]):
        rng.shuffle(sel[r])
    return sel


def _pool_runs(rng, n_pools_total: int, count: int, kpool: int,
               exclude: Optional[np.ndarray] = None) -> np.ndarray:
    """`count` distinct pools out of [0, n_pools_total), minus `exclude`,
    expanded to their kpool contiguous positions."""
    cand = np.arange(n_pools_total, dtype=np.int64)
    if exclude is not None and exclude.size:
        cand = np.setdiff1d(cand, exclude, assume_unique=False)
    pools = rng.choice(cand, size=count, replace=False)
    pos = (pools[:, None] * kpool + np.arange(kpool)[None, :]).ravel()
    return pos.astype(np.int32), pools


# ------------------------------------------------------------------ workloads

def make(name: str, *, sel_seed: int = 0, with_pool: bool = True) -> Workload:
    """Build a workload on the host. `sel_seed` != 0 redraws the selections
    (and nothing else) so a benchmark can cycle through several batches over
    one cache. Pools of 'long' are never drawn here (use device_pool)."""
    cfg = WORKLOADS[name]
    seed = SEEDS[name]
    rng = np.random.default_rng(seed)
    R, H, D, B, kp, W = (cfg["rows"], cfg["heads"], cfg["D"], cfg["block_size"],
                         cfg["kpool"], cfg["width"])
    sm, ks, sigma = cfg["sm_scale"], cfg["k_scale"], cfg["sigma"]
    srng = np.random.default_rng([seed, sel_seed]) if sel_seed else rng

    q = rng.standard_normal((R, H, D), dtype=np.float32)
    q_bits = bf16_bits_from_f32(q)

    if name == "tiny":
        num_pages = 32
        seq_lens = np.array([100, 173], dtype=np.int32)
        bt = rng.permutation(num_pages).astype(np.int32).reshape(R, 16)
        bt_stride = 16
        sel = np.empty((R, W), dtype=np.int32)
        for r in range(R):
            uniq = srng.choice(seq_lens[r], size=23, replace=False)
            dups = srng.choice(uniq, size=3, replace=True)
            holes = np.full(6, -1)
            sel[r] = np.concatenate([uniq, dups, holes])
        _shuffle_rows(srng, sel)
    elif name == "glm":
        L = 8192
        num_pages = R * (L // B)
        seq_lens = np.full(R, L, dtype=np.int32)
        bt = rng.permutation(num_pages).astype(np.int32).reshape(R, L // B)
        bt_stride = L // B
        sel = np.empty((R, W), dtype=np.int32)
        for r in range(R):
            sel[r], _ = _pool_runs(srng, L // kp, W // kp, kp)
        _shuffle_rows(srng, sel)
    elif name == "long":
        L = 131072
        per_seq = L // B
        num_pages = 786432  # 24 GiB of 32 KiB pages
        seq_lens = np.full(R, L, dtype=np.int32)
        perm = rng.permutation(num_pages)[: R * per_seq]
        bt = perm.astype(np.int32).reshape(R, per_seq)
        bt_stride = per_seq
        sel = np.empty((R, W), dtype=np.int32)
        n_runs = 358
        n_single = W - n_runs * kp  # 616
        for r in range(R):
            runs, pools = _pool_runs(srng, L // kp, n_runs, kp)
            taken = np.zeros(L, dtype=bool)
            taken[runs] = True
            free = np.flatnonzero(~taken)
            singles = srng.choice(free, size=n_single, replace=False)
            sel[r] = np.concatenate([runs, singles.astype(np.int32)])
        _shuffle_rows(srng, sel)
    elif name == "verify":
        seqs, k = 64, 4
        assert R == seqs * k
        base = rng.integers(4096, 32768, size=seqs, endpoint=True)
        pages_per_seq = -(-(base + k) // B)
        num_pages = int(pages_per_seq.sum())
        perm = rng.permutation(num_pages).astype(np.int32)
        bt_stride = int(pages_per_seq.max())
        bt = np.zeros((R, bt_stride), dtype=np.int32)
        seq_lens = np.empty(R, dtype=np.int32)
        sel = np.empty((R, W), dtype=np.int32)
        core_pools, row_pools = 307, 205
        start = 0
        for s in range(seqs):
            n = int(pages_per_seq[s])
            table = perm[start:start + n]
            start += n
            S = int(base[s])
            # pools ending at or before position S (every row may attend them)
            core, core_ids = _pool_runs(srng, (S + 1) // kp, core_pools, kp)
            for j in range(k):
                r = s * k + j
                pos = S + j
                bt[r, :n] = table
                seq_lens[r] = pos + 1
                extra, _ = _pool_runs(srng, (pos + 1) // kp, row_pools, kp,
                                      exclude=core_ids)
                sel[r] = np.concatenate([core, extra])
        _shuffle_rows(srng, sel)
    elif name == "ragged":
        lo, hi = math.log(16), math.log(65536)
        seq_lens = np.floor(np.exp(rng.uniform(lo, hi, size=R))).astype(np.int32)
        seq_lens = np.clip(seq_lens, 16, 65536)
        pages_per_seq = -(-seq_lens // B)
        num_pages = int(pages_per_seq.sum())
        perm = rng.permutation(num_pages).astype(np.int32)
        bt_stride = int(pages_per_seq.max())
        bt = np.zeros((R, bt_stride), dtype=np.int32)
        sel = np.full((R, W), -1, dtype=np.int32)
        start = 0
        for r in range(R):
            n = int(pages_per_seq[r])
            bt[r, :n] = perm[start:start + n]
            start += n
            L = int(seq_lens[r])
            if L < W:
                sel[r, :L] = np.arange(L, dtype=np.int32)
            else:
                uniq = srng.choice(L, size=1127, replace=False).astype(np.int32)
                dups = srng.choice(uniq, size=614, replace=True)
                sel[r] = np.concatenate([uniq, dups, np.full(307, -1, np.int32)])
        _shuffle_rows(srng, sel)
    else:
        raise KeyError(name)

    max_seq_len = int(seq_lens.max())
    wl = Workload(
        name=name, rows=R, heads=H, D=D, block_size=B, kpool=kp, width=W,
        bt_stride=bt_stride, cache_stride_bytes=B * D, max_seq_len=max_seq_len,
        num_pages=num_pages, sm_scale=sm, k_scale=ks, v_scale=ks, sigma=sigma,
        seed=seed, q_bits=q_bits, block_tables=np.ascontiguousarray(bt),
        seq_lens=seq_lens, sel=np.ascontiguousarray(sel))
    if with_pool and name != "long":
        wl.pool = host_pool(np.random.default_rng([seed, 7]), num_pages, B, D,
                            sigma, ks)
    return wl


def with_rope_tail(wl: Workload, rope: int = 64, seed: int = 5) -> Workload:
    """The same workload with tokens that carry a rope tail after the latent
    (the DeepSeek-V4 token of [attend]'s module doc: 512 + 64 bytes): q gains
    `rope` values per head (N(0,1), bf16), the pool is redrawn with the same
    recipe at D + rope bytes per token, pages of block_size such tokens, and
    the softmax scale becomes 1/sqrt(D + rope). Tables and selections are
    unchanged."""
    rng = np.random.default_rng([wl.seed if wl.seed >= 0 else 0, seed])
    R, H = wl.rows, wl.heads
    tail = bf16_bits_from_f32(rng.standard_normal((R, H, rope), dtype=np.float32))
    q_bits = np.concatenate([wl.q_bits, tail], axis=2)
    tb = wl.D + rope
    pool = host_pool(rng, wl.num_pages, wl.block_size, tb, wl.sigma, wl.k_scale)
    return dataclasses.replace(
        wl, name=wl.name + f"+rope{rope}", q_bits=np.ascontiguousarray(q_bits),
        cache_stride_bytes=wl.block_size * tb, sm_scale=1.0 / math.sqrt(tb), pool=pool,
        rope=rope)


def pages_of_rows(wl: Workload, rows) -> np.ndarray:
    """Distinct physical pages the given rows' selected ids live on (inputs
    for copying a sub-pool back to the host)."""
    out = []
    for r in rows:
        ids = wl.sel[r]
        ids = ids[(ids >= 0) & (ids < wl.seq_lens[r])]
        table = wl.block_tables[r if wl.bt_stride else 0]
        out.append(table[ids // wl.block_size])
    return np.unique(np.concatenate(out)) if out else np.zeros(0, np.int32)


def random_case(rng: np.random.Generator, *, rows: int, heads: int, D: int,
                block_size: int, max_len: int, width: int, num_pages: int = 0,
                hole_frac: float = 0.2, dup_frac: float = 0.1,
                oob_frac: float = 0.05, shared_table: bool = False,
                k_scale: float = 0.05, sigma: float = 1.0) -> Workload:
    """Small random case for parity tests: random lengths in [1, max_len],
    shuffled pages, selections mixing valid ids, repeats, -1 holes, other
    negative ids and ids past the row's length."""
    pages_per_row = -(-max_len // block_size)
    bt_stride = 0 if shared_table else pages_per_row
    n_tables = 1 if shared_table else rows
    need = n_tables * pages_per_row
    num_pages = max(num_pages, need)
    perm = rng.permutation(num_pages).astype(np.int32)[:need]
    bt = perm.reshape(n_tables, pages_per_row)
    seq_lens = rng.integers(1, max_len, size=rows, endpoint=True).astype(np.int32)
    sel = np.empty((rows, width), dtype=np.int32)
    for r in range(rows):
        L = int(seq_lens[r])
        v = rng.integers(0, L, size=width)
        u = rng.random(width)
        v = np.where(u < hole_frac, -1, v)
        v = np.where((u >= hole_frac) & (u < hole_frac + oob_frac / 2),
                     rng.integers(L, L + 1000, size=width), v)
        v = np.where((u >= hole_frac + oob_frac / 2) & (u < hole_frac + oob_frac),
                     -rng.integers(2, 1000, size=width), v)
        d = rng.random(width) < dup_frac
        if width > 1:
            v[d] = v[rng.integers(0, width, size=int(d.sum()))]
        sel[r] = v
    q = rng.standard_normal((rows, heads, D), dtype=np.float32)
    pool = host_pool(rng, num_pages, block_size, D, sigma, k_scale)
    return Workload(
        name="random", rows=rows, heads=heads, D=D, block_size=block_size,
        kpool=1, width=width, bt_stride=bt_stride,
        cache_stride_bytes=block_size * D, max_seq_len=int(max_len),
        num_pages=num_pages, sm_scale=1.0 / math.sqrt(D), k_scale=k_scale,
        v_scale=k_scale, sigma=sigma, seed=-1, q_bits=bf16_bits_from_f32(q),
        block_tables=np.ascontiguousarray(bt), seq_lens=seq_lens, sel=sel,
        pool=pool)
