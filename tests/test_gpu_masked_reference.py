"""The on-device dense masked-attention reference (dsa_decode_masked_reference).

First it is pinned to the CPU oracle on small shapes: both compute the same
definition (fp32 on the GPU, fp64 in the oracle), so they agree far inside
the decode's tolerance. It then checks the decode on every row and head of
the full-size workloads, where the CPU oracle only samples rows. Every case
prints its name before it touches the GPU.
"""
import numpy as np
import pytest
import torch

import workloads as WL

pytestmark = pytest.mark.gpu

REF_TOL = 1e-4  # fp32 reference against the fp64 oracle, per (row, head)


@pytest.fixture(scope="module")
def H(native):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_harness
    return gpu_harness


def _announce(name, **kw):
    print(f"\n[gpu case] {name} {kw}", flush=True)


def _reference(H, wl, k_pool, v_pool=None, sel=None, seq_lens=None):
    import sparse_attention_decode_row_amd as dsa
    out = dsa.masked_reference(
        H.q_tensor(wl.q_bits), k_pool, k_pool if v_pool is None else v_pool,
        H.i32(wl.block_tables), H.i32(wl.seq_lens if seq_lens is None else seq_lens),
        H.i32(wl.sel if sel is None else sel), k_scale=wl.k_scale, v_scale=wl.v_scale,
        block_size=wl.block_size, index_kpool=wl.kpool, block_table_stride=wl.bt_stride,
        max_seq_len=wl.max_seq_len, sm_scale=wl.sm_scale,
        cache_stride_bytes=wl.cache_stride_bytes)
    torch.cuda.synchronize()
    return out.double().cpu().numpy()


# ------------------------------------------------ pinned to the CPU oracle

REF_CASES = [
    # seed, rows, heads, D, B, max_len, width, shared table, split V
    (1, 3, 4, 64, 16, 300, 64, False, False),
    (2, 4, 16, 512, 64, 2000, 700, False, False),
    (3, 2, 8, 256, 32, 900, 400, True, False),
    (4, 3, 5, 128, 16, 500, 200, False, True),
]


@pytest.mark.parametrize("case", REF_CASES, ids=[f"ref{c[0]}" for c in REF_CASES])
def test_reference_matches_the_oracle(H, case):
    seed, rows, heads, D, B, max_len, width, shared, split_v = case
    rng = np.random.default_rng(900 + seed)
    wl = WL.random_case(rng, rows=rows, heads=heads, D=D, block_size=B,
                        max_len=max_len, width=width, shared_table=shared)
    _announce("reference vs oracle", seed=seed, rows=rows, heads=heads, D=D)
    v_host = WL.host_pool(rng, wl.num_pages, B, D, 1.0, wl.k_scale) if split_v else None
    got = _reference(H, wl, H.u8(wl.pool), None if v_host is None else H.u8(v_host))
    want = H.oracle_rows(wl, range(rows), host_v_pool=v_host)
    err = H.normwise_err(got, want)
    print(f"reference case {seed} max err {err.max():.3e}")
    assert err.max() <= REF_TOL


def test_reference_tiny_and_empty_rows(H):
    wl = WL.make("tiny")
    _announce("reference tiny + empty rows")
    got = _reference(H, wl, H.u8(wl.pool))
    want = H.oracle_rows(wl, range(wl.rows))
    assert H.normwise_err(got, want).max() <= REF_TOL
    sel = np.full_like(wl.sel, -1)
    sel[0, :3] = [wl.seq_lens[0], wl.seq_lens[0] + 5, -7]  # nothing valid either
    got = _reference(H, wl, H.u8(wl.pool), sel=sel)
    assert np.all(got == 0.0)


# ------------------------------------- the decode on every row, full size

@pytest.mark.parametrize("name", ["glm", "ragged"])
def test_decode_matches_reference_on_every_row(H, name):
    wl = WL.make(name, with_pool=False)
    _announce("decode vs reference, all rows", workload=name, rows=wl.rows, heads=wl.heads)
    pool = WL.device_pool(wl.num_pages, wl.block_size, wl.D, wl.sigma, wl.k_scale,
                          seed=wl.seed)
    run = H.run_gpu(wl, k_pool=pool, with_selection=False)
    ref = _reference(H, wl, pool)
    err = H.normwise_err(run.out, ref)
    print(f"{name}: decode vs reference over {err.size} (row, head) pairs: "
          f"max {err.max():.3e} mean {err.mean():.3e}")
    assert err.max() <= H.TOL


def test_decode_matches_reference_verify_co_scheduled(H):
    wl = WL.make("verify", with_pool=False)
    _announce("decode vs reference, all rows", workload="verify", rows_per_sequence=4)
    pool = WL.device_pool(wl.num_pages, wl.block_size, wl.D, wl.sigma, wl.k_scale,
                          seed=wl.seed)
    run = H.run_gpu(wl, k_pool=pool, with_selection=False, rows_per_sequence=4)
    ref = _reference(H, wl, pool)
    err = H.normwise_err(run.out, ref)
    print(f"verify: decode vs reference over {err.size} (row, head) pairs: "
          f"max {err.max():.3e} mean {err.mean():.3e}")
    assert err.max() <= H.TOL


def test_decode_matches_reference_long_context(H):
    """The long-context workload in the bench's launch configuration: 128
    rows x 64 heads over the 24 GiB pool, every row checked."""
    wl = WL.make("long", with_pool=False)
    _announce("decode vs reference, all rows", workload="long", rows=wl.rows,
              pool_gib=wl.pool_bytes / 2**30)
    pool = WL.device_pool(wl.num_pages, wl.block_size, wl.D, wl.sigma, wl.k_scale,
                          seed=wl.seed)
    run = H.run_gpu(wl, k_pool=pool, with_selection=False)
    ref = _reference(H, wl, pool)
    del pool
    torch.cuda.empty_cache()
    err = H.normwise_err(run.out, ref)
    print(f"long: decode vs reference over {err.size} (row, head) pairs: "
          f"max {err.max():.3e} mean {err.mean():.3e}")
    assert err.max() <= H.TOL
