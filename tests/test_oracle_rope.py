"""Pins of the oracle's decode over cache tokens that carry a rope tail after
the latent (dsa_oracle_decode_qkv), against things other than itself.

Page citation: [attend] "spark_model/layers/glm5next_dsa/attend.rs", module
doc section "NoPE, and why no common/ kernel would do" (a DeepSeek-V4 token
carries a 64-wide rope tail after the 512-wide latent; one prior kernel
silently took that tail from the next token) and decode_attention's comment
on the score scale (DeepSeek-V4 scales by 1/sqrt(576) for that reason).
Reading taken here: a token is 576 FP8 E4M3FN bytes, the latent then the
already rotated tail, both under k_scale; q has 576 values per head; the
scores run over all 576, the values and the output over the first 512.

What pins what:
  * The whole decode: a float64 dense masked-attention brute force over the
    logical (unpaged) 576-byte tokens, with the selection as a membership
    mask, on random shapes (and a small 80 = 64 + 16 token).
  * Closed forms: one selected token returns its first 512 bytes
    dequantised; two adjacent tokens of one page, with a query that reads
    only the tail, follow the logistic weights of their own tails. Taking a
    token's tail from the next token's first 64 bytes gives another result.
  * A query whose tail is zero reproduces the NoPE decode of the first 512
    bytes of every token.
"""
import math

import numpy as np
import pytest
import torch

import workloads as WL


def f64_fp8(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def f64_bf16(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def fp8(x):
    return WL.fp8_codes_from_f32(np.asarray(x, dtype=np.float32))


def brute(q_bits, lat, sel_row, seq_len, dv, sm, ks, vs):
    """Dense masked attention over logical tokens lat [L, Dqk] (FP8 codes):
    scores over every byte, values over the first dv."""
    q = f64_bf16(q_bits)                       # [H, Dqk]
    K = ks * f64_fp8(lat[:seq_len])            # [L, Dqk]
    V = vs * f64_fp8(lat[:seq_len, :dv])       # [L, dv]
    mask = np.isin(np.arange(seq_len), np.asarray(sel_row))
    if not mask.any():
        return np.zeros((q.shape[0], dv))
    s = sm * (q @ K.T)
    s = np.where(mask[None, :], s, -np.inf)
    w = np.exp(s - s.max(axis=1, keepdims=True))
    return (w / w.sum(axis=1, keepdims=True)) @ V


def paged(rng, *, rows, heads, dqk, B, max_len, width, pad=0, scale=20.0):
    """Logical tokens scattered into a shuffled paged pool (pages of
    B * dqk + pad bytes; unused bytes hold the NaN code)."""
    ppr = -(-max_len // B)
    num_pages = rows * ppr + 2
    stride = B * dqk + pad
    bt = rng.permutation(num_pages).astype(np.int32)[:rows * ppr].reshape(rows, ppr)
    pool = np.full(num_pages * stride, 0x7F, dtype=np.uint8)
    seq_lens = rng.integers(1, max_len, size=rows, endpoint=True).astype(np.int32)
    lats = []
    for r in range(rows):
        lat = fp8(rng.standard_normal((max_len, dqk)) * scale)
        lats.append(lat)
        for t in range(int(seq_lens[r])):
            off = int(bt[r, t // B]) * stride + (t % B) * dqk
            pool[off:off + dqk] = lat[t]
    sel = np.empty((rows, width), dtype=np.int32)
    for r in range(rows):
        L = int(seq_lens[r])
        v = rng.integers(0, L, size=width)
        u = rng.random(width)
        v = np.where(u < 0.2, -1, v)
        v = np.where((u >= 0.2) & (u < 0.25), rng.integers(L, L + 50, size=width), v)
        dup = rng.random(width) < 0.15
        v[dup] = v[rng.integers(0, width, size=int(dup.sum()))]
        sel[r] = v
    q_bits = WL.bf16_bits_from_f32(rng.standard_normal((rows, heads, dqk)).astype(np.float32))
    return dict(q=q_bits, pool=pool, bt=bt, stride=stride, seq_lens=seq_lens, sel=sel,
                lats=lats, B=B)


@pytest.mark.parametrize("seed,dqk,dv,heads,B,max_len,width,pad", [
    (1, 576, 512, 4, 16, 150, 64, 0),
    (2, 576, 512, 2, 64, 300, 200, 576),
    (3, 80, 64, 3, 8, 90, 40, 16),
])
def test_rope_decode_equals_dense_masked_bruteforce(oracle_mod, seed, dqk, dv, heads, B,
                                                    max_len, width, pad):
    rng = np.random.default_rng(700 + seed)
    c = paged(rng, rows=3, heads=heads, dqk=dqk, B=B, max_len=max_len, width=width, pad=pad)
    sm, ks, vs = 1.0 / math.sqrt(dqk), 0.05, 0.03
    got = oracle_mod.decode(c["q"], c["pool"], None, c["bt"], c["seq_lens"], c["sel"],
                            block_size=B, bt_stride=c["bt"].shape[1],
                            cache_stride_bytes=c["stride"], sm_scale=sm, k_scale=ks,
                            v_scale=vs, v_dim=dv)
    assert got.shape == (3, heads, dv)
    for r in range(3):
        want = brute(c["q"][r], c["lats"][r], c["sel"][r], int(c["seq_lens"][r]), dv,
                     sm, ks, vs)
        np.testing.assert_allclose(got[r], want, rtol=1e-11, atol=1e-13)


def test_rope_single_token_returns_its_latent(oracle_mod):
    rng = np.random.default_rng(11)
    c = paged(rng, rows=2, heads=3, dqk=576, B=16, max_len=40, width=12)
    vs = 0.041
    toks = []
    for r in range(2):
        t = int(rng.integers(0, c["seq_lens"][r]))
        toks.append(t)
        c["sel"][r] = -1
        c["sel"][r, ::4] = t
    got = oracle_mod.decode(c["q"], c["pool"], None, c["bt"], c["seq_lens"], c["sel"],
                            block_size=16, bt_stride=c["bt"].shape[1],
                            cache_stride_bytes=c["stride"], sm_scale=0.05, k_scale=0.05,
                            v_scale=vs, v_dim=512)
    for r in range(2):
        want = vs * f64_fp8(c["lats"][r][toks[r], :512])
        for h in range(3):
            np.testing.assert_array_equal(got[r, h], want)


def test_rope_tail_belongs_to_its_own_token(oracle_mod):
    # Tokens 0 and 1 are adjacent rows of one page. q reads tail element 0
    # only; token 0's tail starts with a = 2, token 1's with c = -1, and token
    # 1's latent starts with b = 4 (its value row is 4 e_0 + e_1; token 0's is
    # e_0). With sm_scale 1, k_scale 1/2: s_0 = 1, s_1 = -1/2, so
    #   out_0 = v_scale (p_0 + 4 p_1), out_1 = v_scale p_1, p_1 = 1/(1 + e^1.5).
    # A tail read from the next token's first bytes (b instead of a) would
    # give s_0 = 2.
    B, dqk = 4, 576
    row0 = np.zeros(dqk, np.float32)
    row1 = np.zeros(dqk, np.float32)
    row0[0], row0[512] = 1.0, 2.0
    row1[0], row1[1], row1[512] = 4.0, 1.0, -1.0
    pool = np.zeros(B * dqk, np.uint8)
    pool[0:dqk] = fp8(row0)
    pool[dqk:2 * dqk] = fp8(row1)
    q = np.zeros((1, 2, dqk), np.float32)
    q[0, :, 512] = 1.0
    vs = 0.25
    got = oracle_mod.decode(WL.bf16_bits_from_f32(q), pool, None, np.zeros((1, 1), np.int32),
                            np.array([2], np.int32), np.array([[1, 0]], np.int32),
                            block_size=B, bt_stride=1, cache_stride_bytes=B * dqk,
                            sm_scale=1.0, k_scale=0.5, v_scale=vs, v_dim=512)
    p1 = 1.0 / (1.0 + math.exp(1.5))
    p0 = 1.0 - p1
    want = np.zeros(512)
    want[0] = vs * (p0 + 4.0 * p1)
    want[1] = vs * p1
    for h in range(2):
        np.testing.assert_allclose(got[0, h], want, rtol=1e-14, atol=0)


def test_zero_tail_query_is_the_nope_decode_of_the_latents(oracle_mod):
    rng = np.random.default_rng(13)
    c = paged(rng, rows=3, heads=4, dqk=576, B=16, max_len=120, width=60)
    q = c["q"].copy()
    q[:, :, 512:] = 0                      # bf16 +0
    kw = dict(block_size=16, bt_stride=c["bt"].shape[1], sm_scale=0.07, k_scale=0.05,
              v_scale=0.03)
    got = oracle_mod.decode(q, c["pool"], None, c["bt"], c["seq_lens"], c["sel"],
                            cache_stride_bytes=c["stride"], v_dim=512, **kw)
    # the same latents as 512-byte tokens
    pages = c["pool"].reshape(-1, 16, 576)[:, :, :512].reshape(-1)
    nope = oracle_mod.decode(q[:, :, :512], pages, None, c["bt"], c["seq_lens"], c["sel"],
                             cache_stride_bytes=16 * 512, **kw)
    np.testing.assert_allclose(got, nope, rtol=1e-13, atol=1e-15)
