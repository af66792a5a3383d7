"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar (from the method's contract): per (row, head) the max normwise relative
error of the BF16 output is <= 1e-2; the set of attended ids and their byte
offsets are bit-exact. Every case prints its name before it touches the GPU.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as WL

pytestmark = pytest.mark.gpu

H_ = None


@pytest.fixture(scope="module")
def H(native):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_harness
    return gpu_harness


def _announce(name, **kw):
    print(f"\n[gpu case] {name} {kw}", flush=True)


# ------------------------------------------------------------ workloads

def test_tiny(H):
    wl = WL.make("tiny")
    _announce("tiny", rows=wl.rows, heads=wl.heads, D=wl.D)
    run = H.run_gpu(wl)
    H.check_selection(wl, run)
    want = H.oracle_rows(wl, range(wl.rows))
    err = H.normwise_err(run.out, want)
    print(f"tiny max err {err.max():.3e}")
    assert err.max() <= H.TOL


@pytest.mark.parametrize("in_kernel", [False, True])
def test_glm_full(H, in_kernel):
    wl = WL.make("glm")
    _announce("glm", rows=wl.rows, heads=wl.heads, D=wl.D, W=wl.width, in_kernel=in_kernel)
    run = H.run_gpu(wl, merge_in_kernel=in_kernel)
    print("plan", run.info)
    assert run.info["merges_chunks"] == (2 if in_kernel else 1)
    H.check_selection(wl, run)
    want = H.oracle_rows(wl, range(wl.rows))
    err = H.normwise_err(run.out, want)
    print(f"glm max err {err.max():.3e} mean {err.mean():.3e}")
    assert err.max() <= H.TOL


def test_long_sampled_rows(H):
    wl = WL.make("long", with_pool=False)
    _announce("long", rows=wl.rows, heads=wl.heads, pool_gib=wl.pool_bytes / 2**30)
    pool = WL.device_pool(wl.num_pages, wl.block_size, wl.D, wl.sigma, wl.k_scale,
                          seed=wl.seed)
    run = H.run_gpu(wl, k_pool=pool)
    print("plan", run.info)
    H.check_selection(wl, run)          # every row, bit-exact
    rows = [0, 37, 90, 127]
    sub, view = H.sub_pool_for_rows(wl, pool, rows)
    del pool
    torch.cuda.empty_cache()
    want = H.oracle_rows(view, rows, host_pool=sub)
    err = H.normwise_err(run.out[rows], want)
    print(f"long rows {rows} max err {err.max():.3e}")
    assert err.max() <= H.TOL


def test_verify_sampled_rows(H):
    wl = WL.make("verify", with_pool=False)
    _announce("verify", rows=wl.rows, pages=wl.num_pages)
    pool = WL.device_pool(wl.num_pages, wl.block_size, wl.D, wl.sigma, wl.k_scale,
                          seed=wl.seed)
    run = H.run_gpu(wl, k_pool=pool)
    print("plan", run.info)
    H.check_selection(wl, run)
    rows = [0, 1, 2, 3, 101, 254, 255]
    sub, view = H.sub_pool_for_rows(wl, pool, rows)
    want = H.oracle_rows(view, rows, host_pool=sub)
    err = H.normwise_err(run.out[rows], want)
    print(f"verify rows {rows} max err {err.max():.3e}")
    assert err.max() <= H.TOL


def test_verify_rows_co_scheduled_per_sequence(H):
    """decode_k rows of one sequence co-scheduled on one XCD
    (rows_per_sequence = 4): bit-identical to independent scheduling, and
    the sampled rows match the oracle."""
    wl = WL.make("verify", with_pool=False)
    _announce("verify co-scheduled", rows=wl.rows, rows_per_sequence=4)
    pool = WL.device_pool(wl.num_pages, wl.block_size, wl.D, wl.sigma, wl.k_scale,
                          seed=wl.seed)
    base = H.run_gpu(wl, k_pool=pool)
    run = H.run_gpu(wl, k_pool=pool, rows_per_sequence=4)
    print("plan", run.info)
    assert run.info["rows_per_sequence"] == 4
    H.check_selection(wl, run)
    assert np.array_equal(run.out_bits, base.out_bits)
    rows = [0, 3, 4, 130, 255]
    sub, view = H.sub_pool_for_rows(wl, pool, rows)
    want = H.oracle_rows(view, rows, host_pool=sub)
    err = H.normwise_err(run.out[rows], want)
    print(f"verify co-scheduled rows {rows} max err {err.max():.3e}")
    assert err.max() <= H.TOL


@pytest.mark.parametrize("k,chunk_tokens,heads,D,layout", [
    (3, 64, 40, 128, 0), (5, 0, 40, 128, 0), (2, 64, 16, 128, 0), (4, 0, 12, 128, 0),
    (3, 64, 80, 512, 3), (4, 0, 64, 512, 3)])
def test_co_scheduled_rows_with_padding_and_splits(H, k, chunk_tokens, heads, D, layout):
    """A sequence count that leaves a block of 8 partly empty, with and
    without split chunks, in 16-, 32- and 64-head blocks: same bits as
    independent scheduling, oracle parity on every row."""
    rng = np.random.default_rng(77 + k)
    seqs = 5
    wl = WL.random_case(rng, rows=seqs * k, heads=heads, D=D, block_size=16,
                        width=300, max_len=900)
    _announce("co-scheduled", rows=wl.rows, k=k, chunk_tokens=chunk_tokens, heads=heads,
              layout=layout)
    base = H.run_gpu(wl, chunk_tokens=chunk_tokens, layout=layout)
    run = H.run_gpu(wl, chunk_tokens=chunk_tokens, rows_per_sequence=k, layout=layout)
    H.check_selection(wl, run)
    assert np.array_equal(run.out_bits, base.out_bits)
    want = H.oracle_rows(wl, range(wl.rows))
    err = H.normwise_err(run.out, want)
    print(f"co-scheduled k={k} max err {err.max():.3e} plan {run.info}")
    assert err.max() <= H.TOL


def test_ragged_all_rows(H):
    wl = WL.make("ragged", with_pool=False)
    _announce("ragged", rows=wl.rows, heads=wl.heads, pages=wl.num_pages)
    pool = WL.device_pool(wl.num_pages, wl.block_size, wl.D, wl.sigma, wl.k_scale,
                          seed=wl.seed)
    run = H.run_gpu(wl, k_pool=pool)
    print("plan", run.info)
    H.check_selection(wl, run)
    host = pool.cpu().numpy()
    want = H.oracle_rows(wl, range(wl.rows), host_pool=host)
    err = H.normwise_err(run.out, want)
    print(f"ragged max err {err.max():.3e}")
    assert err.max() <= H.TOL


# -------------------------------------------------- random shapes and splits

CASES = [
    # (seed, rows, heads, D, B, max_len, width, chunk_tokens, shared, split_v)
    (0, 3, 16, 512, 64, 700, 600, 0, False, False),
    (1, 4, 64, 512, 64, 5000, 1500, 128, False, False),
    (2, 2, 32, 512, 16, 900, 1000, 64, False, False),
    (3, 5, 20, 256, 32, 2000, 700, 192, False, False),
    (4, 3, 80, 128, 16, 400, 300, 0, False, False),
    (5, 6, 4, 64, 16, 300, 200, 64, True, False),
    (6, 3, 48, 512, 64, 3000, 2100, 0, False, True),
    (7, 2, 64, 512, 64, 1000, 900, 256, True, True),
    (8, 4, 1, 512, 8, 150, 64, 0, False, False),
    (9, 3, 128, 256, 64, 2600, 2500, 1024, False, False),
    (10, 3, 64, 64, 16, 1200, 900, 64, False, False),
    (11, 2, 40, 256, 32, 3000, 2000, 0, False, True),
    (12, 2, 96, 128, 32, 1500, 1400, 128, True, False),
    (13, 2, 64, 512, 64, 20000, 8192, 0, False, False),   # the planner's split: 64 chunks a row
    (14, 2, 64, 512, 64, 20000, 8192, 2048, False, False),  # four chunks of the largest size
    # page sizes that are not a power of two (the translation divides), and larger pages
    (15, 3, 64, 512, 12, 1500, 1200, 0, False, False),
    (16, 2, 32, 256, 48, 3000, 2000, 256, True, False),
    (17, 3, 64, 512, 128, 5000, 2048, 0, False, False),
    (18, 2, 16, 512, 256, 9000, 2048, 512, False, True),
]


@pytest.mark.parametrize("case", CASES, ids=[f"case{c[0]}" for c in CASES])
def test_random_shapes(H, case):
    seed, rows, heads, D, B, max_len, width, ct, shared, split_v = case
    rng = np.random.default_rng(500 + seed)
    wl = WL.random_case(rng, rows=rows, heads=heads, D=D, block_size=B,
                        max_len=max_len, width=width, shared_table=shared)
    _announce("random", seed=seed, rows=rows, heads=heads, D=D, W=width,
              chunk=ct, shared=shared, split_v=split_v)
    v_host = None
    v_dev = None
    if split_v:
        v_host = WL.host_pool(rng, wl.num_pages, B, D, 1.0, wl.k_scale)
        v_dev = H.u8(v_host)
    run = H.run_gpu(wl, v_pool=v_dev, chunk_tokens=ct)
    H.check_selection(wl, run)
    want = H.oracle_rows(wl, range(rows), host_v_pool=v_host)
    err = H.normwise_err(run.out, want)
    print(f"case {seed}: plan {run.info} max err {err.max():.3e}")
    assert err.max() <= H.TOL
    # without the selection export (the production path: every head block
    # translates through its own branch-free placement when it can)
    plain = H.run_gpu(wl, v_pool=v_dev, chunk_tokens=ct, with_selection=False)
    assert np.array_equal(plain.out_bits, run.out_bits)


@pytest.mark.parametrize("layout", [1, 2, 3])
def test_both_layouts_match_the_oracle(H, layout):
    """32-head, 16-head and 64-head blocks (eight waves each) compute the
    same decode; run each on a split, multi-block shape (96 heads: a partial
    last block in every layout)."""
    rng = np.random.default_rng(40 + layout)
    wl = WL.random_case(rng, rows=5, heads=96, D=512, block_size=64, max_len=4000,
                        width=1800)
    _announce("layout", layout=layout)
    for ct in (0, 384):
        run = H.run_gpu(wl, chunk_tokens=ct, layout=layout)
        assert run.info["layout"] == layout
        H.check_selection(wl, run)
        want = H.oracle_rows(wl, range(wl.rows))
        err = H.normwise_err(run.out, want)
        print(f"layout {layout} chunk {ct}: plan {run.info} max err {err.max():.3e}")
        assert err.max() <= H.TOL


# 64-head blocks: one scoring wave per 16-head group scores the whole tile
CASES64 = [
    # (seed, rows, heads, B, max_len, width, chunk_tokens, split_v)
    (0, 3, 64, 64, 5000, 2048, 0, False),
    (1, 4, 96, 64, 3000, 1500, 192, False),
    (2, 2, 48, 16, 900, 1000, 64, True),
    (3, 5, 128, 32, 2600, 2100, 512, False),
    (4, 2, 17, 64, 700, 600, 0, True),
]


@pytest.mark.parametrize("case", CASES64, ids=[f"h64_{c[0]}" for c in CASES64])
def test_64_head_blocks(H, case):
    seed, rows, heads, B, max_len, width, ct, split_v = case
    rng = np.random.default_rng(900 + seed)
    wl = WL.random_case(rng, rows=rows, heads=heads, D=512, block_size=B,
                        max_len=max_len, width=width)
    _announce("heads64", seed=seed, rows=rows, heads=heads, W=width, chunk=ct,
              split_v=split_v)
    v_host = v_dev = None
    if split_v:
        v_host = WL.host_pool(rng, wl.num_pages, B, 512, 1.0, wl.k_scale)
        v_dev = H.u8(v_host)
    run = H.run_gpu(wl, v_pool=v_dev, chunk_tokens=ct, layout=3)
    assert run.info["layout"] == 3 and run.info["heads_per_block"] == 64
    H.check_selection(wl, run)
    want = H.oracle_rows(wl, range(rows), host_v_pool=v_host)
    err = H.normwise_err(run.out, want)
    print(f"h64 case {seed}: plan {run.info} max err {err.max():.3e}")
    assert err.max() <= H.TOL


@pytest.mark.parametrize("layout", [0, 3])
def test_split_invariance(H, layout):
    """Any chunk size gives the oracle's result (the planner's head blocks,
    and 64-head blocks)."""
    rng = np.random.default_rng(42)
    wl = WL.random_case(rng, rows=3, heads=64, D=512, block_size=64,
                        max_len=6000, width=2048, hole_frac=0.0, dup_frac=0.0,
                        oob_frac=0.0)
    outs = []
    for ct in (0, 64, 192, 512, 2048):
        _announce("split", chunk=ct, layout=layout)
        run = H.run_gpu(wl, chunk_tokens=ct, with_selection=False, layout=layout)
        outs.append(run.out)
    want = H.oracle_rows(wl, range(3))
    for o in outs:
        assert H.normwise_err(o, want).max() <= H.TOL
        assert H.normwise_err(o, outs[0]).max() <= H.TOL


# ------------------------------------------------------------ special cases

@pytest.mark.parametrize("layout", [2, 1, 3])
def test_single_token_is_exact_dequantised_row(H, layout):
    """One selected token (repeated, among holes): the output of every head
    is bf16(v_scale * dec(code)) bit for bit. The latent row holds all 254
    finite codes, so this also checks the FP8 decode exhaustively. Every
    head-block layout."""
    D, B, heads = 512, 64, 64
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    row = np.resize(codes, D)   # 254 codes, repeated to fill the row
    pool = np.zeros(4 * B * D, np.uint8)
    rng = np.random.default_rng(9)
    bt = np.array([[3, 1], [2, 0]], np.int32)
    seq_lens = np.array([100, 128], np.int32)
    sel = np.full((2, 16), -1, np.int32)
    t = [77, 5]
    for r in range(2):
        page = bt[r, t[r] // B]
        base = (page * B + t[r] % B) * D
        pool[base:base + D] = row
        sel[r, ::4] = t[r]
    for vs in (1.0, 0.02):
        wl = WL.Workload(name="single", rows=2, heads=heads, D=D, block_size=B, kpool=4,
                         width=16, bt_stride=2, cache_stride_bytes=B * D,
                         max_seq_len=128, num_pages=4, sm_scale=1 / 16, k_scale=0.02,
                         v_scale=vs, sigma=1.0, seed=0,
                         q_bits=WL.bf16_bits_from_f32(rng.standard_normal((2, heads, D), dtype=np.float32)),
                         block_tables=bt, seq_lens=seq_lens, sel=sel, pool=pool)
        _announce("single token", v_scale=vs, layout=layout)
        run = H.run_gpu(wl, layout=layout)
        assert run.info["layout"] == layout
        dec = torch.from_numpy(row.copy()).view(torch.float8_e4m3fn).float()
        # the output is a weighted sum that starts from +0, so the -0 code
        # comes out as +0 (IEEE: +0 + -0 = +0); the oracle does the same
        want = (dec * torch.tensor(vs, dtype=torch.float32) + 0.0).to(torch.bfloat16)
        want_bits = want.view(torch.int16).numpy().view(np.uint16)
        for r in range(2):
            for h in range(heads):
                assert np.array_equal(run.out_bits[r, h], want_bits), (vs, r, h)


@pytest.mark.parametrize("layout", [2, 1, 3])
def test_empty_selection_rows_are_zero(H, layout):
    rng = np.random.default_rng(10)
    wl = WL.random_case(rng, rows=4, heads=64, D=512, block_size=64, max_len=500,
                        width=300)
    sel = wl.sel.copy()
    seq_lens = wl.seq_lens.copy()
    sel[0] = -1                              # all holes
    sel[1] = seq_lens[1] + np.arange(300)    # all past the end
    seq_lens[2] = 0                          # nothing valid
    for ct in (0, 64):
        _announce("empty rows", chunk=ct, layout=layout)
        run = H.run_gpu(wl, sel=sel, seq_lens=seq_lens, chunk_tokens=ct, layout=layout)
        H.check_selection(wl, run, sel=sel, seq_lens=seq_lens)
        assert np.array_equal(run.out_bits[:3], np.zeros_like(run.out_bits[:3]))
        want = H.oracle_rows(wl, [3], sel=sel, seq_lens=seq_lens)
        assert H.normwise_err(run.out[3:4], want).max() <= H.TOL


def test_seq_lens_are_clamped_to_0_and_max_seq_len(H):
    """A negative seq_lens[r] attends nothing and one above max_seq_len
    attends as if it were max_seq_len (the launch contract: ids are kept
    when 0 <= t < min(max(seq_len, 0), max_seq_len))."""
    rng = np.random.default_rng(16)
    wl = WL.random_case(rng, rows=4, heads=32, D=512, block_size=64, max_len=1000,
                        width=900)
    sel = wl.sel.copy()
    sel[1, :300] = np.arange(700, 1600, 3)     # ids on both sides of max_seq_len
    given = np.array([-5, 1500, 1000, 37], np.int32)
    clamped = np.clip(given, 0, wl.max_seq_len).astype(np.int32)
    for ct in (0, 128):
        _announce("clamped seq_lens", chunk=ct)
        run = H.run_gpu(wl, sel=sel, seq_lens=given, chunk_tokens=ct)
        H.check_selection(wl, run, sel=sel, seq_lens=clamped)
        assert np.array_equal(run.out_bits[0], np.zeros_like(run.out_bits[0]))
        want = H.oracle_rows(wl, [1, 2, 3], sel=sel, seq_lens=clamped)
        assert H.normwise_err(run.out[1:], want).max() <= H.TOL


@pytest.mark.parametrize("k_scale,v_scale", [(1e-6, 1e-20), (0.5, 1e4), (0.05, -3.0)])
def test_extreme_and_negative_scales(H, k_scale, v_scale):
    """Dequantisation scales far from the pool's own: k_scale 1e-6 flattens
    the softmax to uniform, 0.5 sharpens it; v_scale 1e-20 and 1e4 scale the
    output far from 1 (bf16 keeps fp32's exponent range), and a negative
    v_scale flips its sign. Whole rows and rows split into chunks."""
    rng = np.random.default_rng(17)
    base = WL.random_case(rng, rows=3, heads=64, D=512, block_size=64, max_len=2500,
                          width=1200)
    wl = WL.Workload(**{**base.__dict__, "k_scale": k_scale, "v_scale": v_scale})
    want = H.oracle_rows(wl, range(wl.rows))
    for ct in (0, 256):
        _announce("scales", k_scale=k_scale, v_scale=v_scale, chunk=ct)
        run = H.run_gpu(wl, chunk_tokens=ct, with_selection=False)
        assert np.isfinite(run.out).all()
        assert H.normwise_err(run.out, want).max() <= H.TOL


def test_repeats_holes_and_order_do_not_change_the_result(H):
    """The selection is normalised to a sorted set before the attention, so
    the output is bit-identical whatever the repeats, holes and order."""
    rng = np.random.default_rng(11)
    wl = WL.random_case(rng, rows=3, heads=64, D=512, block_size=64, max_len=3000,
                        width=700, hole_frac=0.0, dup_frac=0.0, oob_frac=0.0)
    _announce("invariance clean")
    base = H.run_gpu(wl, with_selection=False)
    W2 = 1400
    sel2 = np.full((3, W2), -1, np.int32)
    for r in range(3):
        row = np.concatenate([wl.sel[r], wl.sel[r][: 400], np.full(250, -1),
                              wl.seq_lens[r] + np.arange(50)]).astype(np.int32)
        rng.shuffle(row)
        sel2[r] = row
    wl2 = WL.Workload(**{**wl.__dict__, "width": W2, "sel": sel2})
    _announce("invariance noisy")
    noisy = H.run_gpu(wl2)
    H.check_selection(wl2, noisy)
    assert np.array_equal(noisy.out_bits, base.out_bits)


@pytest.mark.parametrize("layout", [2, 1, 3])
def test_uniform_softmax_membership_probe(H, layout):
    """q = 0 makes every selected token weigh 1/n. With one-hot V rows
    (token t's latent row is e_t with FP8 1.0, v_scale 1) the output is
    nonzero exactly on the selected set, every nonzero equal to bf16(1/n):
    a duplicate counted twice or a stray token would show."""
    D, B, L = 512, 64, 500
    rng = np.random.default_rng(12)
    pages = -(-L // B)
    bt = rng.permutation(pages).astype(np.int32)[None, :]
    pool = np.zeros(pages * B * D, np.uint8)
    for t in range(L):
        base = (bt[0, t // B] * B + t % B) * D
        pool[base + t] = 0x38   # 1.0
    sel = rng.integers(-3, L + 30, size=(1, 900)).astype(np.int32)
    heads = 64
    wl = WL.Workload(name="probe", rows=1, heads=heads, D=D, block_size=B, kpool=4,
                     width=900, bt_stride=pages, cache_stride_bytes=B * D,
                     max_seq_len=L, num_pages=pages, sm_scale=1.0, k_scale=1.0,
                     v_scale=1.0, sigma=1.0, seed=0,
                     q_bits=np.zeros((1, heads, D), np.uint16), block_tables=bt,
                     seq_lens=np.array([L], np.int32), sel=sel, pool=pool)
    for ct in (0, 64):
        _announce("membership probe", chunk=ct, layout=layout)
        run = H.run_gpu(wl, chunk_tokens=ct, layout=layout)
        S = sorted({int(t) for t in sel[0] if 0 <= t < L})
        inv_n = torch.tensor(1.0 / len(S), dtype=torch.float32).to(torch.bfloat16).float().item()
        for h in range(heads):
            nz = np.flatnonzero(run.out[0, h])
            assert nz.tolist() == S
            np.testing.assert_allclose(run.out[0, h, S], inv_n, rtol=2 ** -7)


def test_two_window_selection_beyond_262144_positions(H):
    """Rows longer than one selection-bitmap window (262144 positions)."""
    rng = np.random.default_rng(13)
    D, B, L = 512, 64, 600_000
    n_pages = 96
    per_row = -(-L // B)
    bt = rng.integers(0, n_pages, size=(2, per_row)).astype(np.int32)
    sel = rng.integers(-10, L + 100, size=(2, 3000)).astype(np.int32)
    sel[:, :500] = rng.integers(262_000, 262_300, size=(2, 500))   # around the window edge
    pool = WL.host_pool(rng, n_pages, B, D, 1.0, 0.02)
    wl = WL.Workload(name="window", rows=2, heads=64, D=D, block_size=B, kpool=4,
                     width=3000, bt_stride=per_row, cache_stride_bytes=B * D,
                     max_seq_len=L, num_pages=n_pages, sm_scale=1 / 16, k_scale=0.02,
                     v_scale=0.02, sigma=1.0, seed=0,
                     q_bits=WL.bf16_bits_from_f32(rng.standard_normal((2, 64, D), dtype=np.float32)),
                     block_tables=bt, seq_lens=np.array([L, 400_000], np.int32), sel=sel,
                     pool=pool)
    _announce("two windows", L=L)
    run = H.run_gpu(wl)
    H.check_selection(wl, run)
    want = H.oracle_rows(wl, [0, 1])
    assert H.normwise_err(run.out, want).max() <= H.TOL


@pytest.mark.parametrize("D,B,L", [(512, 16, 300_000), (64, 16, 100_000)])
def test_block_table_beyond_the_lds_copy(H, D, B, L):
    """Rows whose block-table row is longer than the part the kernel copies
    into LDS (16384 entries at D = 512, 2048 at D = 64): pages past it are
    read from global memory. The D = 64 row also spans several bitmap
    windows (32768 positions each)."""
    rng = np.random.default_rng(17 + D)
    n_pages = 64
    per_row = -(-L // B)
    bt = rng.integers(0, n_pages, size=(2, per_row)).astype(np.int32)
    sel = rng.integers(-5, L + 50, size=(2, 1500)).astype(np.int32)
    sel[:, :300] = rng.integers(L - 40_000, L, size=(2, 300))   # pages past the copy
    pool = WL.host_pool(rng, n_pages, B, D, 1.0, 0.02)
    wl = WL.Workload(name="bt_tail", rows=2, heads=24, D=D, block_size=B, kpool=4,
                     width=1500, bt_stride=per_row, cache_stride_bytes=B * D,
                     max_seq_len=L, num_pages=n_pages, sm_scale=1 / 16, k_scale=0.02,
                     v_scale=0.02, sigma=1.0, seed=0,
                     q_bits=WL.bf16_bits_from_f32(rng.standard_normal((2, 24, D), dtype=np.float32)),
                     block_tables=bt, seq_lens=np.array([L, L - 7], np.int32), sel=sel,
                     pool=pool)
    _announce("block table tail", D=D, B=B, L=L)
    run = H.run_gpu(wl)
    H.check_selection(wl, run)
    want = H.oracle_rows(wl, [0, 1])
    assert H.normwise_err(run.out, want).max() <= H.TOL


def test_padded_page_stride(H):
    rng = np.random.default_rng(14)
    wl = WL.random_case(rng, rows=3, heads=64, D=512, block_size=16, max_len=800,
                        width=500)
    # re-lay the pool with a 4 KiB gap after every page
    stride = wl.block_size * wl.D + 4096
    pages = wl.pool.reshape(wl.num_pages, -1)
    big = np.full((wl.num_pages, stride), 0x7F, np.uint8)   # gaps hold NaN codes
    big[:, : pages.shape[1]] = pages
    wl2 = WL.Workload(**{**wl.__dict__, "cache_stride_bytes": stride,
                         "pool": big.ravel()})
    _announce("padded stride", stride=stride)
    run = H.run_gpu(wl2)
    H.check_selection(wl2, run)
    want = H.oracle_rows(wl2, range(3))
    assert H.normwise_err(run.out, want).max() <= H.TOL


@pytest.mark.parametrize("layout", [0, 3])
def test_deterministic(H, layout):
    """Two launches of the GLM workload give the same bits (the planner's
    32-head blocks in four chunks, and 64-head blocks in eight)."""
    wl = WL.make("glm")
    _announce("determinism", layout=layout)
    pool = H.u8(wl.pool)
    a = H.run_gpu(wl, k_pool=pool, with_selection=False, layout=layout)
    b = H.run_gpu(wl, k_pool=pool, with_selection=False, layout=layout)
    assert np.array_equal(a.out_bits, b.out_bits)


@pytest.mark.parametrize("layout,in_kernel", [(1, False), (1, True), (2, False), (2, True),
                                              (3, False)])   # 64-head blocks: combine kernel only
def test_many_chunk_merges_repeated_on_one_workspace(H, layout, in_kernel):
    """The split merge under load: 64-token chunks (up to 32 per row), 30
    launches on one workspace without re-initialising it, merged by the
    combine kernel or inside the decode kernel (most workgroups publish and
    the last per row and head block merges). Every launch must give the same
    bits (the counters reset themselves, the merge order is fixed whichever
    chunk arrives last) and the first must match the oracle."""
    import sparse_attention_decode_row_amd as dsa
    rng = np.random.default_rng(31 + layout)
    wl = WL.random_case(rng, rows=6, heads=64, D=512, block_size=64, max_len=3000,
                        width=2048)
    _announce("many-chunk merges, repeated", layout=layout, in_kernel=in_kernel)
    plan = H.plan_for(wl, chunk_tokens=64, layout=layout, merge_in_kernel=in_kernel)
    assert plan.info()["merges_chunks"] == (2 if in_kernel else 1)
    info = plan.info()
    print("plan", info)
    assert info["chunks_per_row"] >= 16
    q, pool = H.q_tensor(wl.q_bits), H.u8(wl.pool)
    bt, sl, sel = H.i32(wl.block_tables), H.i32(wl.seq_lens), H.i32(wl.sel)
    ws = plan.new_workspace()
    outs = []
    for _ in range(30):
        out = torch.full_like(q, float("nan"))
        plan.launch(q, pool, pool, bt, sl, sel, wl.k_scale, wl.v_scale, out, ws)
        outs.append(out)
    torch.cuda.synchronize()
    bits = [o.view(torch.int16).cpu().numpy() for o in outs]
    for i, b in enumerate(bits[1:], 1):
        assert np.array_equal(b, bits[0]), f"launch {i} differs from launch 0"
    want = H.oracle_rows(wl, range(wl.rows))
    err = H.normwise_err(outs[0].float().cpu().numpy().astype(np.float64), want)
    print(f"many-chunk merges: max err {err.max():.3e}")
    assert err.max() <= H.TOL
    plan.close()


def test_timed_out_merge_poisons_the_workspace_until_reinit(H):
    """The split merge's bounded wait, forced from the host: the published
    count of one (row, head block) is preset far below zero, so its merger
    gives up after its time limit while every kernel still ends normally.
    That block's output must be NaN and the rest correct; the workspace's
    status word then poisons every later launch on it, until
    dsa_decode_workspace_init zeroes it, after which the output is right
    again."""
    rng = np.random.default_rng(78)
    wl = WL.random_case(rng, rows=4, heads=64, D=512, block_size=64, max_len=3000,
                        width=2048)
    _announce("timed-out merge, sticky status")
    plan = H.plan_for(wl, chunk_tokens=512, layout=1, merge_in_kernel=True)
    info = plan.info()
    R, HB, C = wl.rows, info["head_blocks"], info["chunks_per_row"]
    assert C >= 2 and HB == 2
    q, pool = H.q_tensor(wl.q_bits), H.u8(wl.pool)
    bt, sl, sel = H.i32(wl.block_tables), H.i32(wl.seq_lens), H.i32(wl.sel)
    ws = plan.new_workspace()
    counters = ws.narrow(0, info["counters_offset"], 8 * R * HB).view(torch.int32)
    status = ws.narrow(0, info["status_offset"], 4).view(torch.int32)
    bad_row, bad_hb = 1, 1
    counters[R * HB + bad_row * HB + bad_hb] = -(1 << 30)

    def launch():
        out = torch.full_like(q, float("nan"))
        plan.launch(q, pool, pool, bt, sl, sel, wl.k_scale, wl.v_scale, out, ws)
        torch.cuda.synchronize()
        return out.float().cpu().numpy().astype(np.float64)

    want = H.oracle_rows(wl, range(R))
    first = launch()
    bad = np.zeros((R, wl.heads), dtype=bool)
    bad[bad_row, 32 * bad_hb:32 * (bad_hb + 1)] = True
    assert np.isnan(first[bad]).all()
    assert np.isfinite(first[~bad]).all()
    err = H.normwise_err(np.where(bad[..., None], want, first), want)
    assert err.max() <= H.TOL
    assert int(status.item()) == 1
    c = counters.cpu().numpy()
    assert (c[:R * HB] == 0).all()                                   # arrivals reset
    assert c[R * HB + bad_row * HB + bad_hb] == -(1 << 30)           # publishes owed came in
    assert (np.delete(c[R * HB:], bad_row * HB + bad_hb) == 0).all()
    second = launch()
    assert np.isnan(second).all(), "a poisoned workspace must poison every output"
    plan.workspace_init(ws)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    third = launch()
    assert np.isfinite(third).all()
    assert H.normwise_err(third, want).max() <= H.TOL
    plan.close()


# ------------------------------------------------------------ launch errors

def test_launch_rejects_bad_arguments(H):
    import sparse_attention_decode_row_amd as dsa
    wl = WL.make("tiny")
    _announce("launch errors")
    plan = H.plan_for(wl)
    q = H.q_tensor(wl.q_bits)
    pool = H.u8(wl.pool)
    bt, sl, sel = H.i32(wl.block_tables), H.i32(wl.seq_lens), H.i32(wl.sel)
    out = torch.empty_like(q)
    ws = torch.empty(plan.workspace_bytes + 512, dtype=torch.uint8, device=q.device)
    plan.workspace_init(ws)
    with pytest.raises(dsa.DsaDecodeError) as e:
        plan.launch(q, pool, pool, bt, sl, sel, 0.05, 0.05, out, ws,
                    workspace_bytes=plan.workspace_bytes - 1)
    assert e.value.status == dsa.DSA_DECODE_ERR_WORKSPACE
    with pytest.raises(dsa.DsaDecodeError) as e:
        plan.launch(q, pool, pool, bt, sl, sel, 0.05, 0.05, out, ws.data_ptr() + 8,
                    workspace_bytes=plan.workspace_bytes)
    assert e.value.status == dsa.DSA_DECODE_ERR_WORKSPACE
    with pytest.raises(dsa.DsaDecodeError) as e:
        plan.launch(q.data_ptr() + 2, pool, pool, bt, sl, sel, 0.05, 0.05, out, ws)
    assert e.value.status == dsa.DSA_DECODE_ERR_INVALID
    with pytest.raises(dsa.DsaDecodeError) as e:
        plan.launch(q, pool, pool, bt, sl, 0, 0.05, 0.05, out, ws)
    assert e.value.status == dsa.DSA_DECODE_ERR_INVALID
    with pytest.raises(dsa.DsaDecodeError) as e:
        plan.launch(q, pool, pool, bt, sl, sel, float("nan"), 0.05, out, ws)
    assert e.value.status == dsa.DSA_DECODE_ERR_INVALID
    host_plan = dsa.Plan(num_rows=2, num_q_heads=4, kv_lora_rank=64, block_size=16,
                         index_kpool=4, sel_width=32, block_table_stride=16,
                         max_seq_len=173, sm_scale=0.125, device=-1)
    with pytest.raises(dsa.DsaDecodeError) as e:
        host_plan.launch(q, pool, pool, bt, sl, sel, 0.05, 0.05, out, ws)
    assert e.value.status == dsa.DSA_DECODE_ERR_INVALID
    # nothing was launched: out is untouched by the refused calls
    plan.launch(q, pool, pool, bt, sl, sel, 0.05, 0.05, out, ws)
    torch.cuda.synchronize()
    # the read-back hook needs a plan that exports the selection
    with pytest.raises(dsa.DsaDecodeError) as e:
        plan.read_selection(ws, counts=torch.empty(2, dtype=torch.int32, device=q.device))
    assert e.value.status == dsa.DSA_DECODE_ERR_INVALID
    assert "EXPORT_SELECTION" in str(e.value)


def test_plan_on_gfx950_device(H):
    import sparse_attention_decode_row_amd as dsa
    _announce("device plan")
    p = dsa.Plan(num_rows=128, num_q_heads=64, kv_lora_rank=512, block_size=64,
                 index_kpool=4, sel_width=2048, block_table_stride=2048,
                 max_seq_len=131072, sm_scale=1 / 16, device=0)
    info = p.info()
    assert info["device"] == 0 and info["num_cus"] >= 1
    props = torch.cuda.get_device_properties(0)
    assert props.gcnArchName.startswith("gfx950")


@pytest.mark.parametrize("layout", [2, 1, 3])
def test_score_far_above_the_first_tiles_max(H, layout):
    """Late tokens whose scores exceed every earlier one by hundreds of
    log2 units, twice (a token at position 500, then a larger one at 900,
    in different 16-token blocks of their tiles): the weights must stay
    finite and the result match the oracle (the softmax is then essentially
    one-hot on the last of them). Every head-block layout, whole rows and
    rows split into chunks."""
    D, B, L, heads = 512, 64, 1024, 64
    rng = np.random.default_rng(15)
    pages = L // B
    bt = rng.permutation(pages).astype(np.int32)[None, :]
    pool = WL.fp8_codes_from_f32(rng.standard_normal(pages * B * D, dtype=np.float32) * 0.5)
    for pos, code in ((500, 0x7D), (900, 0x7E)):   # 416, then 448, in every column
        base = (bt[0, pos // B] * B + pos % B) * D
        pool[base:base + D] = code
    q = np.zeros((1, heads, D), np.float32)
    q[0, :, :] = 8.0                      # large |q|: scores spread far
    q[0, 1::2, :] = 6.0                   # heads differ in how far
    wl = WL.Workload(name="spread", rows=1, heads=heads, D=D, block_size=B, kpool=4,
                     width=L, bt_stride=pages, cache_stride_bytes=B * D, max_seq_len=L,
                     num_pages=pages, sm_scale=1 / 16, k_scale=0.02, v_scale=0.02,
                     sigma=1.0, seed=0, q_bits=WL.bf16_bits_from_f32(q),
                     block_tables=bt, seq_lens=np.array([L], np.int32),
                     sel=np.arange(L, dtype=np.int32)[None, :], pool=pool)
    want = H.oracle_rows(wl, [0])
    for ct in (0, 256):
        _announce("score spread", layout=layout, chunk=ct)
        run = H.run_gpu(wl, chunk_tokens=ct, layout=layout)
        assert run.info["layout"] == layout
        assert np.isfinite(run.out).all()
        assert H.normwise_err(run.out, want).max() <= H.TOL
