"""GPU parity of the cache writer (the latent_write launch of the page
"metrale_model_arch/glm5next_dsa/layer/decode_k.rs") through the C ABI.

Bar: every FP8 code the GPU writes equals the oracle's, except where the
exact value lies within fp32 rounding of a midpoint between two codes (the
two sides compute in different precision and order); there the GPU code must
be one of the two nearest codes, and such cases must be rare. Bytes outside
the written rows are untouched. A pool written by the GPU writer and read by
the GPU decode matches the oracle decode of the same pool (producer and
consumer agree).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as WL

pytestmark = pytest.mark.gpu

SENTINEL = 0xA5


@pytest.fixture(scope="module")
def H(native):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_harness
    return gpu_harness


def _announce(name, **kw):
    print(f"\n[gpu case] {name} {kw}", flush=True)


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _check_codes(got: np.ndarray, want: np.ndarray, values: np.ndarray):
    """got/want: uint8 codes; values: the oracle's exact pre-quantisation
    values. Returns the number of near-tie mismatches (asserts the rest)."""
    mism = np.nonzero(got != want)[0]
    for i in mism:
        v = values[i]
        a = oracle.fp8_e4m3fn(np.array([got[i], want[i]], dtype=np.uint8))
        lo, hi = min(a), max(a)
        # adjacent codes, the exact value between them and within a few fp32
        # ulps of their midpoint
        assert lo < hi, (i, got[i], want[i], v)
        mid = 0.5 * (lo + hi)
        assert abs(v - mid) <= 1e-6 * max(abs(v), 2.0 ** -9), (i, got[i], want[i], v, mid)
    return len(mism)


def _run_case(H, rng, *, rows, D, B, pages, stride_pad, sigma, inv, eps=1e-6, neg_slots=0):
    stride = B * D + stride_pad
    kv = rng.normal(0.0, sigma, (rows, D))
    w = rng.uniform(0.5, 1.5, D)
    kv_bits, w_bits = _bf16_bits(kv), _bf16_bits(w)
    slots = rng.choice(pages * B, size=rows, replace=False).astype(np.int64)
    if neg_slots:
        slots[rng.choice(rows, size=neg_slots, replace=False)] = -1
    pool_bytes = pages * stride
    host = np.full(pool_bytes, SENTINEL, dtype=np.uint8)
    values = oracle.latent_write(kv_bits, w_bits, slots, host, block_size=B,
                                 cache_stride_bytes=stride_pad and stride, eps=eps,
                                 inv_kv_scale=inv)
    import sparse_attention_decode_row_amd as dsa
    dev = torch.device("cuda")
    pool = torch.full((pool_bytes,), SENTINEL, dtype=torch.uint8, device=dev)
    kv_t = torch.from_numpy(kv_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    w_t = torch.from_numpy(w_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    sl_t = torch.from_numpy(slots).to(dev)
    dsa.latent_write(kv_t, w_t, sl_t, pool, block_size=B, rms_eps=eps, inv_kv_scale=inv,
                     cache_stride_bytes=stride_pad and stride)
    torch.cuda.synchronize()
    got = pool.cpu().numpy()
    written = np.zeros(pool_bytes, dtype=bool)
    ties = 0
    for i, s in enumerate(slots):
        if s < 0:
            continue
        off = (s // B) * stride + (s % B) * D
        written[off:off + D] = True
        ties += _check_codes(got[off:off + D], host[off:off + D], values[i])
    assert np.all(got[~written] == SENTINEL)
    n = int(written.sum())
    return ties, n, host, got, values


@pytest.mark.parametrize("D,B,pad", [(512, 64, 0), (512, 16, 256), (256, 32, 0),
                                     (128, 64, 128), (64, 16, 0), (512, 48, 0), (256, 12, 64)])
def test_writer_matches_oracle(H, D, B, pad):
    rng = np.random.default_rng(100 + D + B)
    _announce("latent_write", D=D, B=B, pad=pad)
    ties, n, *_ = _run_case(H, rng, rows=257, D=D, B=B, pages=40, stride_pad=pad,
                            sigma=1.0, inv=1 / 0.02, neg_slots=9)
    print(f"D {D} B {B}: {n} bytes, {ties} near-tie differences", flush=True)
    assert ties <= max(2, n // 1000)


@pytest.mark.parametrize("rows,D", [(1, 512), (2, 512), (7, 512), (8, 512), (9, 512),
                                    (3, 64), (5, 256)])
def test_writer_small_batches(H, rows, D):
    """Batches that leave waves and workgroups partly filled (two rows per
    wave, eight per workgroup)."""
    rng = np.random.default_rng(400 + rows + D)
    _announce("latent_write small", rows=rows, D=D)
    ties, n, *_ = _run_case(H, rng, rows=rows, D=D, B=16, pages=4, stride_pad=0,
                            sigma=2.0, inv=1 / 0.05, neg_slots=1 if rows >= 7 else 0)
    assert ties <= 2


@pytest.mark.parametrize("sigma,eps", [(2.0 ** -10, 2.0 ** -20), (2.0 ** -8, 3.0 * 2.0 ** -16),
                                       (1e-3, 1e-5)])
def test_writer_eps_comparable_to_mean_square(H, sigma, eps):
    """Rows whose mean square is of the order of rms_eps, so that where eps
    enters the root changes every code: the GPU writer must match the
    oracle's placement (inside the root, unscaled)."""
    rng = np.random.default_rng(int(1e6 * sigma) + 5)
    _announce("latent_write eps", sigma=sigma, eps=eps)
    ties, n, host, got, values = _run_case(H, rng, rows=65, D=512, B=64, pages=4,
                                           stride_pad=0, sigma=sigma, inv=1 / 0.02, eps=eps)
    # (mean square / (mean square + eps) is about 1/2, 1/4 and 1/11 here)
    assert ties <= 2


def test_writer_saturates(H):
    rng = np.random.default_rng(9)
    _announce("latent_write saturation")
    # inv_kv_scale 1e4: most values are far past 448 and must come out +-448
    ties, n, host, got, values = _run_case(H, rng, rows=33, D=512, B=64, pages=4,
                                           stride_pad=0, sigma=1.0, inv=1e4)
    # (the codes already equal the oracle's, which saturates)
    big = int((np.abs(values) >= 448).sum())
    assert big > 1000
    written = got[host != SENTINEL]
    assert int(np.isin(written, [0x7E, 0xFE]).sum()) >= big
    assert not np.any(np.isin(written, [0x7F, 0xFF]))  # never a NaN code
    assert ties == 0


def test_writer_zero_rows_and_all_skipped(H):
    import sparse_attention_decode_row_amd as dsa
    _announce("latent_write degenerate")
    dev = torch.device("cuda")
    pool = torch.full((64 * 512,), SENTINEL, dtype=torch.uint8, device=dev)
    kv = torch.zeros((3, 512), dtype=torch.bfloat16, device=dev)
    w = torch.ones(512, dtype=torch.bfloat16, device=dev)
    dsa.latent_write(kv[:0], w, torch.zeros(0, dtype=torch.int64, device=dev), pool,
                     block_size=64, rms_eps=1e-6, inv_kv_scale=1.0)
    dsa.latent_write(kv, w, torch.full((3,), -1, dtype=torch.int64, device=dev), pool,
                     block_size=64, rms_eps=1e-6, inv_kv_scale=1.0)
    torch.cuda.synchronize()
    assert torch.all(pool == SENTINEL)


def test_written_pool_decodes_like_the_oracle(H):
    """Producer and consumer agree: rows written by the GPU writer, read back
    by the GPU decode, match the oracle decode of the bytes written."""
    import sparse_attention_decode_row_amd as dsa
    rng = np.random.default_rng(77)
    _announce("latent_write -> decode")
    wl = WL.random_case(rng, rows=3, heads=32, D=512, block_size=64, max_len=1500, width=700)
    R = wl.rows
    # every position of every row gets a freshly written latent row
    pages_used = int(wl.pool.size // wl.cache_stride_bytes)
    n_tok = pages_used * wl.block_size
    kv = rng.normal(0.0, 1.0, (n_tok, wl.D))
    w = rng.uniform(0.5, 1.5, wl.D)
    kv_bits, w_bits = _bf16_bits(kv), _bf16_bits(w)
    slots = np.arange(n_tok, dtype=np.int64)
    dev = torch.device("cuda")
    pool = torch.zeros(wl.pool.size, dtype=torch.uint8, device=dev)
    dsa.latent_write(torch.from_numpy(kv_bits.view(np.int16)).to(dev).view(torch.bfloat16),
                     torch.from_numpy(w_bits.view(np.int16)).to(dev).view(torch.bfloat16),
                     torch.from_numpy(slots).to(dev), pool, block_size=wl.block_size,
                     rms_eps=1e-6, inv_kv_scale=1 / wl.k_scale,
                     cache_stride_bytes=wl.cache_stride_bytes)
    torch.cuda.synchronize()
    host_pool = pool.cpu().numpy()
    run = H.run_gpu(wl, k_pool=pool)
    want = H.oracle_rows(wl, range(R), host_pool=host_pool)
    err = H.normwise_err(run.out, want)
    print(f"written pool: max err {err.max():.3e}", flush=True)
    assert err.max() <= H.TOL
