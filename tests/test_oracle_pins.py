"""Pins of the CPU oracle against things other than itself.

Page citations:
  [attend]   "spark_model/layers/glm5next_dsa/attend.rs"
  [decode_k] "metrale_model_arch/glm5next_dsa/layer/decode_k.rs"
  [build]    "spark_model/layers/glm5next_dsa/build.rs"

What pins what:
  * FP8 decode: torch's float8_e4m3fn -> float32 cast on all 256 codes, plus
    landmark values of the OCP E4M3FN format.
  * Selection normalisation: Python set semantics.
  * Page translation: a logically contiguous cache scattered into pages, and
    hand-worked offsets (tests/golden/page_translation.txt).
  * The whole decode: a float64 dense masked-attention brute force over the
    logical (unpaged) latents with a set-membership mask, which [attend]
    (module doc, "Why this is not the masked kernel") states is exactly
    equivalent; closed forms (single token, uniform softmax, two-token
    logistic weights); a hand-worked example (tests/golden/worked_example_d2.txt);
    invariances (repeats, holes, order, page relabelling).
"""
import math
import os

import numpy as np
import pytest
import torch

import workloads as WL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ helpers

def torch_fp8_to_f64(codes: np.ndarray) -> np.ndarray:
    """Library decode (torch), independent of the oracle's decoder."""
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def masked_dense_attention(q_bits, lat_k, lat_v, sel_row, seq_len, sm_scale,
                           k_scale, v_scale):
    """Dense attention over every logical position < seq_len with a
    set-membership mask: a position takes part iff it occurs in the
    selection row (the masked-kernel semantics). lat_k / lat_v: [L, D] FP8
    codes in logical position order (no paging). Returns [H, D] float64, or
    zeros when nothing is selected."""
    q = torch_bf16_to_f64(q_bits)                       # [H, D]
    K = k_scale * torch_fp8_to_f64(lat_k[:seq_len])     # [L, D]
    V = v_scale * torch_fp8_to_f64(lat_v[:seq_len])
    mask = np.isin(np.arange(seq_len), np.asarray(sel_row))
    if not mask.any():
        return np.zeros_like(q)
    scores = sm_scale * (q @ K.T)                       # [H, L]
    scores = np.where(mask[None, :], scores, -np.inf)
    scores = scores - scores.max(axis=1, keepdims=True)
    w = np.exp(scores)
    w = w / w.sum(axis=1, keepdims=True)
    return w @ V


def logical_case(rng, *, rows, heads, D, B, max_len, width, separate_v=False,
                 shared_table=False, extra_pages=3):
    """Build latents in logical order first, then scatter them into a paged
    pool through a random block table. Returns everything the oracle needs
    plus the logical arrays the brute force reads."""
    pages_per_row = -(-max_len // B)
    n_tables = 1 if shared_table else rows
    num_pages = n_tables * pages_per_row + extra_pages
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = perm[: n_tables * pages_per_row].reshape(n_tables, pages_per_row)
    stride = 0 if shared_table else pages_per_row
    # unused bytes hold the NaN code: a stray read poisons the result
    pool_k = np.full(num_pages * B * D, 0x7F, dtype=np.uint8)
    pool_v = np.full(num_pages * B * D, 0x7F, dtype=np.uint8) if separate_v else pool_k
    seq_lens = rng.integers(1, max_len, size=rows, endpoint=True).astype(np.int32)
    if shared_table:
        seq_lens[:] = seq_lens.max()
    lat_k, lat_v = [], []
    if shared_table:
        Lk = WL.fp8_codes_from_f32(rng.standard_normal((max_len, D), dtype=np.float32) * 20)
        Lv = WL.fp8_codes_from_f32(rng.standard_normal((max_len, D), dtype=np.float32) * 20) if separate_v else Lk
    for r in range(rows):
        if not shared_table:
            Lk = WL.fp8_codes_from_f32(rng.standard_normal((max_len, D), dtype=np.float32) * 20)
            Lv = WL.fp8_codes_from_f32(rng.standard_normal((max_len, D), dtype=np.float32) * 20) if separate_v else Lk
        lat_k.append(Lk)
        lat_v.append(Lv)
        table = bt[0 if shared_table else r]
        for t in range(int(seq_lens[r])):
            base = (int(table[t // B]) * B + t % B) * D
            pool_k[base:base + D] = Lk[t]
            if separate_v:
                pool_v[base:base + D] = Lv[t]
    sel = np.empty((rows, width), dtype=np.int32)
    for r in range(rows):
        L = int(seq_lens[r])
        v = rng.integers(0, L, size=width)
        u = rng.random(width)
        v = np.where(u < 0.2, -1, v)
        v = np.where((u >= 0.2) & (u < 0.25), rng.integers(L, L + 50, size=width), v)
        v = np.where((u >= 0.25) & (u < 0.28), -rng.integers(2, 50, size=width), v)
        dup = rng.random(width) < 0.15
        v[dup] = v[rng.integers(0, width, size=int(dup.sum()))]
        sel[r] = v
    q_bits = WL.bf16_bits_from_f32(rng.standard_normal((rows, heads, D), dtype=np.float32))
    return dict(q_bits=q_bits, pool_k=pool_k, pool_v=pool_v, bt=bt, stride=stride,
                seq_lens=seq_lens, sel=sel, lat_k=lat_k, lat_v=lat_v, B=B, D=D)


def run_oracle(oracle_mod, c, sm, ks, vs, **kw):
    return oracle_mod.decode(c["q_bits"], c["pool_k"], c["pool_v"], c["bt"],
                             c["seq_lens"], c["sel"], block_size=c["B"],
                             bt_stride=c["stride"],
                             cache_stride_bytes=c["B"] * c["D"], sm_scale=sm,
                             k_scale=ks, v_scale=vs, **kw)


# --------------------------------------------------------------- FP8 / BF16

def test_fp8_decode_matches_torch_cast_on_every_code(oracle_mod):
    codes = np.arange(256, dtype=np.uint8)
    got = oracle_mod.fp8_e4m3fn(codes)
    want = torch_fp8_to_f64(codes)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


@pytest.mark.parametrize("code,value", [
    (0x38, 1.0),                 # exponent field 7 = bias, mantissa 0
    (0x40, 2.0),
    (0x7E, 448.0),               # largest finite magnitude
    (0xFE, -448.0),
    (0x08, 2.0 ** -6),           # smallest normal
    (0x07, 7 * 2.0 ** -9),       # largest subnormal
    (0x01, 2.0 ** -9),           # smallest subnormal
    (0x00, 0.0),
    (0x3C, 1.5),
    (0xB8, -1.0),
])
def test_fp8_format_landmarks(oracle_mod, code, value):
    assert oracle_mod.fp8_e4m3fn(np.array([code], np.uint8))[0] == value


def test_fp8_negative_zero(oracle_mod):
    v = oracle_mod.fp8_e4m3fn(np.array([0x80], np.uint8))[0]
    assert v == 0.0 and math.copysign(1.0, v) == -1.0


def test_bf16_decode_matches_torch(oracle_mod):
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 1 << 16, size=4000).astype(np.uint16)
    got = oracle_mod.bf16(bits)
    want = torch_bf16_to_f64(bits)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


# ------------------------------------------------------------ selection set

@pytest.mark.parametrize("seed", range(6))
def test_select_row_is_the_python_set(oracle_mod, seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(1, 3000))
    W = int(rng.integers(1, 600))
    row = rng.integers(-5, L + 40, size=W).astype(np.int32)
    row[rng.random(W) < 0.2] = -1
    if W > 3:
        row[: W // 3] = row[W // 3: 2 * (W // 3)]  # repeats
    want = sorted({int(t) for t in row if 0 <= t < L})
    got = oracle_mod.select_row(row, L)
    assert got.tolist() == want


def test_select_row_degenerate(oracle_mod):
    assert oracle_mod.select_row(np.full(8, -1, np.int32), 10).size == 0
    assert oracle_mod.select_row(np.array([3, 3, 3], np.int32), 10).tolist() == [3]
    assert oracle_mod.select_row(np.array([5, 9, 10, 11], np.int32), 10).tolist() == [5, 9]
    assert oracle_mod.select_row(np.array([0, 1], np.int32), 0).size == 0


# ---------------------------------------------------------- page translation

def test_token_offset_golden(oracle_mod):
    n = 0
    with open(os.path.join(GOLDEN, "page_translation.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            head, table = line.split("|")
            B, D, stride, pos, want = (int(x) for x in head.split())
            bt = np.array([int(x) for x in table.split()], np.int32)
            assert oracle_mod.token_offset(bt, pos, B, stride, D) == want
            n += 1
    assert n == 6


def test_token_offset_recovers_logical_layout(oracle_mod):
    rng = np.random.default_rng(11)
    B, D, L = 8, 16, 77
    pages = -(-L // B)
    bt = rng.permutation(pages + 4)[:pages].astype(np.int32)
    logical = rng.integers(0, 256, size=(L, D)).astype(np.uint8)
    pool = np.zeros((pages + 4) * B * D, np.uint8)
    for t in range(L):
        base = (int(bt[t // B]) * B + t % B) * D
        pool[base:base + D] = logical[t]
    for t in range(L):
        off = oracle_mod.token_offset(bt, t, B, B * D, D)
        assert np.array_equal(pool[off:off + D], logical[t])


# --------------------------------------------------- whole decode: pins

def test_worked_example_golden(oracle_mod):
    vals = {}
    with open(os.path.join(GOLDEN, "worked_example_d2.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, *rest = line.split()
                vals[k] = rest
    pool = np.array([int(x, 16) for x in vals["pool_hex"]], np.uint8)
    bt = np.array([[int(x) for x in vals["block_table"]]], np.int32)
    sl = np.array([int(vals["seq_len"][0])], np.int32)
    sel = np.array([[int(x) for x in vals["selection"]]], np.int32)
    q = np.array([[[int(x, 16) for x in vals["q_bf16_hex"]]]], np.uint16)
    out = oracle_mod.decode(q, pool, None, bt, sl, sel,
                            block_size=int(vals["block_size"][0]), bt_stride=2,
                            cache_stride_bytes=4,
                            sm_scale=float(vals["sm_scale"][0]),
                            k_scale=float(vals["k_scale"][0]),
                            v_scale=float(vals["v_scale"][0]))
    assert oracle_mod.select_row(sel[0], sl[0]).tolist() == [int(x) for x in vals["expected_set"]]
    want = np.array([float(x) for x in vals["expected_out"]])
    np.testing.assert_allclose(out[0, 0], want, rtol=1e-15, atol=0)
    # and the same numbers from the logistic closed form
    w0 = 1.0 / (1.0 + math.exp(0.5))
    w2 = 1.0 / (1.0 + math.exp(-0.5))
    np.testing.assert_allclose(out[0, 0], [0.25 * w0, 0.5 * w2], rtol=1e-15)


@pytest.mark.parametrize("seed,D,heads,B,max_len,width,separate_v,shared", [
    (0, 2, 1, 2, 9, 6, False, False),
    (1, 16, 3, 4, 60, 40, False, False),
    (2, 64, 4, 16, 173, 32, False, False),
    (3, 16, 8, 8, 200, 300, True, False),
    (4, 32, 2, 16, 120, 64, False, True),
    (5, 64, 16, 64, 300, 128, True, True),
])
def test_decode_equals_dense_masked_bruteforce(oracle_mod, seed, D, heads, B,
                                               max_len, width, separate_v, shared):
    rng = np.random.default_rng(100 + seed)
    rows = 3
    c = logical_case(rng, rows=rows, heads=heads, D=D, B=B, max_len=max_len,
                     width=width, separate_v=separate_v, shared_table=shared)
    sm, ks, vs = 1.0 / math.sqrt(D), 0.05, 0.03
    got = run_oracle(oracle_mod, c, sm, ks, vs)
    for r in range(rows):
        want = masked_dense_attention(c["q_bits"][r], c["lat_k"][r], c["lat_v"][r],
                                      c["sel"][r], int(c["seq_lens"][r]), sm, ks, vs)
        np.testing.assert_allclose(got[r], want, rtol=1e-11, atol=1e-13)


def test_tiny_workload_equals_dense_masked_bruteforce(oracle_mod):
    wl = WL.make("tiny")
    got = oracle_mod.decode(wl.q_bits, wl.pool, None, wl.block_tables, wl.seq_lens,
                            wl.sel, block_size=wl.block_size, bt_stride=wl.bt_stride,
                            cache_stride_bytes=wl.cache_stride_bytes,
                            sm_scale=wl.sm_scale, k_scale=wl.k_scale,
                            v_scale=wl.v_scale)
    pages = wl.pool.reshape(wl.num_pages, wl.block_size, wl.D)
    for r in range(wl.rows):
        L = int(wl.seq_lens[r])
        # logical view: the page of block j is table[j], the page's slots in order
        lat = pages[wl.block_tables[r]].reshape(-1, wl.D)[:L]
        want = masked_dense_attention(wl.q_bits[r], lat, lat, wl.sel[r], L,
                                      wl.sm_scale, wl.k_scale, wl.v_scale)
        np.testing.assert_allclose(got[r], want, rtol=1e-11, atol=1e-13)


def test_single_token_returns_its_dequantised_latent(oracle_mod):
    rng = np.random.default_rng(3)
    c = logical_case(rng, rows=2, heads=5, D=64, B=16, max_len=50, width=10)
    for r in range(2):
        t = int(rng.integers(0, c["seq_lens"][r]))
        c["sel"][r] = -1
        c["sel"][r, ::3] = t   # one id, repeated, among holes
    vs = 0.037
    got = run_oracle(oracle_mod, c, 0.125, 0.05, vs)
    for r in range(2):
        t = int(c["sel"][r, 0])
        want = vs * torch_fp8_to_f64(c["lat_v"][r][t])
        for h in range(5):
            assert np.array_equal(got[r, h], want)   # p = exp(0) = 1, l = 1: exact


def test_zero_query_gives_mean_of_selected_values(oracle_mod):
    rng = np.random.default_rng(4)
    c = logical_case(rng, rows=3, heads=2, D=16, B=4, max_len=40, width=30)
    c["q_bits"][:] = 0
    vs = 0.5
    got = run_oracle(oracle_mod, c, 0.25, 0.05, vs)
    for r in range(3):
        ids = sorted({int(t) for t in c["sel"][r] if 0 <= t < c["seq_lens"][r]})
        want = vs * torch_fp8_to_f64(c["lat_v"][r][ids]).mean(axis=0) if ids else np.zeros(16)
        for h in range(2):
            np.testing.assert_allclose(got[r, h], want, rtol=1e-13, atol=1e-15)


def test_equal_keys_give_mean_of_selected_values(oracle_mod):
    rng = np.random.default_rng(6)
    D, B, L = 16, 4, 12
    lat_k = np.tile(WL.fp8_codes_from_f32(rng.standard_normal(D, dtype=np.float32) * 9), (L, 1))
    lat_v = WL.fp8_codes_from_f32(rng.standard_normal((L, D), dtype=np.float32) * 9)
    bt = np.array([[2, 0, 1]], np.int32)
    pool_k = np.zeros(3 * B * D, np.uint8)
    pool_v = np.zeros(3 * B * D, np.uint8)
    for t in range(L):
        base = (int(bt[0, t // B]) * B + t % B) * D
        pool_k[base:base + D] = lat_k[t]
        pool_v[base:base + D] = lat_v[t]
    sel = np.array([[1, 5, 5, -1, 11, 7]], np.int32)
    q = WL.bf16_bits_from_f32(rng.standard_normal((1, 3, D), dtype=np.float32))
    got = oracle_mod.decode(q, pool_k, pool_v, bt, np.array([L], np.int32), sel,
                            block_size=B, bt_stride=3, cache_stride_bytes=B * D,
                            sm_scale=0.3, k_scale=0.05, v_scale=0.2)
    want = 0.2 * torch_fp8_to_f64(lat_v[[1, 5, 7, 11]]).mean(axis=0)
    for h in range(3):
        np.testing.assert_allclose(got[0, h], want, rtol=1e-13)


def test_two_tokens_follow_the_logistic_weights(oracle_mod):
    D, B = 4, 2
    # token 0 latent (a, 0, 0, 0), token 1 latent (b, 0, 1, 0); q = (x, 0, 0, 0)
    codes = {0: [0x40, 0, 0, 0], 1: [0x3C, 0, 0x38, 0]}  # 2.0 ; 1.5, 1.0
    pool = np.zeros(2 * B * D, np.uint8)
    bt = np.array([[1]], np.int32)
    for t, c in codes.items():
        base = (1 * B + t) * D
        pool[base:base + D] = c
    x = 3.0
    q = WL.bf16_bits_from_f32(np.array([[[x, 0, 0, 0]]], np.float32))
    sm, ks, vs = 0.7, 0.25, 1.0
    out = oracle_mod.decode(q, pool, None, bt, np.array([2], np.int32),
                            np.array([[0, 1]], np.int32), block_size=B,
                            bt_stride=1, cache_stride_bytes=B * D, sm_scale=sm,
                            k_scale=ks, v_scale=vs)
    delta = sm * ks * x * (2.0 - 1.5)           # s_0 - s_1
    w0 = 1.0 / (1.0 + math.exp(-delta))
    w1 = 1.0 - w0
    np.testing.assert_allclose(out[0, 0], [w0 * 2.0 + w1 * 1.5, 0.0, w1 * 1.0, 0.0],
                               rtol=1e-14, atol=1e-16)


def test_empty_selection_gives_zero(oracle_mod):
    rng = np.random.default_rng(8)
    c = logical_case(rng, rows=2, heads=3, D=16, B=4, max_len=20, width=7)
    c["sel"][0] = -1
    c["sel"][1] = c["seq_lens"][1] + np.arange(7)   # all past the end
    got = run_oracle(oracle_mod, c, 0.25, 0.05, 0.05)
    assert np.array_equal(got, np.zeros_like(got))
    assert not np.signbit(got).any()


# ------------------------------------------------------------- invariances

def _base_case(seed):
    rng = np.random.default_rng(seed)
    return rng, logical_case(rng, rows=3, heads=4, D=32, B=8, max_len=90, width=40)


def test_invariant_to_repeats_holes_and_order(oracle_mod):
    rng, c = _base_case(21)
    ref = run_oracle(oracle_mod, c, 0.2, 0.05, 0.05)
    c2 = dict(c)
    sel = c["sel"]
    extra = np.concatenate([sel, sel[:, ::-1], np.full((3, 9), -1, np.int32),
                            c["seq_lens"][:, None] + np.arange(4)[None, :]], axis=1)
    for r in range(3):
        rng.shuffle(extra[r])
    c2["sel"] = np.ascontiguousarray(extra.astype(np.int32))
    got = run_oracle(oracle_mod, c2, 0.2, 0.05, 0.05)
    assert np.array_equal(got, ref)   # same set, same order of summation


def test_invariant_to_physical_page_relabelling(oracle_mod):
    rng, c = _base_case(22)
    ref = run_oracle(oracle_mod, c, 0.2, 0.05, 0.05)
    B, D = c["B"], c["D"]
    num_pages = c["pool_k"].size // (B * D)
    relabel = rng.permutation(num_pages).astype(np.int32)   # old page p -> new page relabel[p]
    pages = c["pool_k"].reshape(num_pages, B * D)
    new_pool = np.empty_like(pages)
    new_pool[relabel] = pages
    c2 = dict(c)
    c2["pool_k"] = new_pool.ravel()
    c2["pool_v"] = c2["pool_k"]
    c2["bt"] = relabel[c["bt"]]
    got = run_oracle(oracle_mod, c2, 0.2, 0.05, 0.05)
    assert np.array_equal(got, ref)


def test_thread_count_does_not_change_the_result(oracle_mod):
    _, c = _base_case(23)
    a = run_oracle(oracle_mod, c, 0.2, 0.05, 0.05, num_threads=1)
    b = run_oracle(oracle_mod, c, 0.2, 0.05, 0.05, num_threads=4)
    assert np.array_equal(a, b)


def test_oracle_rejects_bad_geometry(oracle_mod):
    _, c = _base_case(24)
    with pytest.raises(ValueError):
        oracle_mod.decode(c["q_bits"], c["pool_k"], None, c["bt"], c["seq_lens"],
                          c["sel"], block_size=0, bt_stride=c["stride"],
                          cache_stride_bytes=256, sm_scale=1.0, k_scale=1.0,
                          v_scale=1.0)
