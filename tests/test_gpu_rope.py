"""GPU parity of the decode over cache tokens that carry a rope tail after
the latent (qk_rope_dim 64: the 512 + 64 = 576-byte DeepSeek-V4 token named
in the module doc of the page "spark_model/layers/glm5next_dsa/attend.rs",
section "NoPE, and why no common/ kernel would do", and in decode_attention's
comment on the score scale). The scores run over all 576 bytes of each
token's own row, the values and the output over the first 512.

Compared with the CPU oracle (dsa_oracle_decode_qkv, pinned separately) at
the 1e-2 normwise bar per (row, head), on the GLM-shaped workload (32 rows x
64 heads, 2048 selected of 8192 positions) with 576-byte tokens, on random
shapes in both head-block layouts with forced splits, and bit-exact for a
single selected token."""
import numpy as np
import pytest
import torch

import workloads as WL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def H(native):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_harness
    return gpu_harness


def _announce(name, **kw):
    print(f"\n[gpu case] {name} {kw}", flush=True)


@pytest.mark.parametrize("in_kernel", [False, True])
def test_glm_shaped_with_rope_tail(H, in_kernel):
    wl = WL.with_rope_tail(WL.make("glm"))
    assert wl.token_bytes == 576
    _announce("glm + rope tail", rows=wl.rows, heads=wl.heads, in_kernel=in_kernel)
    run = H.run_gpu(wl, merge_in_kernel=in_kernel)
    print("plan", run.info)
    assert run.info["qk_rope_dim"] == 64 and run.info["chunk_tokens"] <= 2048
    H.check_selection(wl, run)
    want = H.oracle_rows(wl, range(wl.rows))
    err = H.normwise_err(run.out, want)
    print(f"glm+rope max err {err.max():.3e} mean {err.mean():.3e}")
    assert err.max() <= H.TOL


@pytest.mark.parametrize("seed,heads,layout,ct,shared,B", [
    (1, 16, 0, 0, False, 64),
    (2, 40, 1, 0, False, 64),
    (3, 64, 2, 256, False, 64),
    (4, 24, 1, 64, True, 64),
    (5, 128, 0, 1024, False, 64),
    (6, 32, 1, 2048, False, 64),   # one workgroup takes 2048 tokens: the tail ring wraps ten times
    (7, 16, 2, 2048, True, 64),
    (8, 64, 0, 0, False, 12),      # pages of 12 and 128 tokens of 576 bytes
    (9, 32, 1, 128, True, 128),
])
def test_random_shapes_with_rope_tail(H, seed, heads, layout, ct, shared, B):
    rng = np.random.default_rng(900 + seed)
    wide = ct == 2048
    base = WL.random_case(rng, rows=5, heads=heads, D=512, block_size=B,
                          max_len=6000 if wide else 3000, width=2048 if wide else 1500,
                          shared_table=shared)
    wl = WL.with_rope_tail(base, seed=seed)
    _announce("rope random", seed=seed, heads=heads, layout=layout, ct=ct, shared=shared, B=B)
    run = H.run_gpu(wl, chunk_tokens=ct, layout=layout)
    H.check_selection(wl, run)
    want = H.oracle_rows(wl, range(wl.rows))
    err = H.normwise_err(run.out, want)
    print(f"rope random max err {err.max():.3e}", flush=True)
    assert err.max() <= H.TOL


def test_single_token_with_rope_tail_is_exact(H):
    """One selected token: the output is v_scale times its latent, rounded
    to bf16, whatever its tail and the query hold."""
    rng = np.random.default_rng(77)
    base = WL.random_case(rng, rows=4, heads=32, D=512, block_size=64, max_len=500,
                          width=16, hole_frac=0.0, dup_frac=0.0, oob_frac=0.0)
    wl = WL.with_rope_tail(base, seed=9)
    sel = np.full_like(wl.sel, -1)
    toks = [int(rng.integers(0, wl.seq_lens[r])) for r in range(wl.rows)]
    for r, t in enumerate(toks):
        sel[r, ::5] = t
    _announce("rope single token")
    run = H.run_gpu(wl, sel=sel)
    for r, t in enumerate(toks):
        page = wl.block_tables[r][t // wl.block_size]
        off = page * wl.cache_stride_bytes + (t % wl.block_size) * wl.token_bytes
        lat = torch.from_numpy(wl.pool[off:off + wl.D].copy()).view(torch.float8_e4m3fn)
        want = (lat.to(torch.float32) * wl.v_scale).to(torch.bfloat16)
        want_bits = want.view(torch.int16).numpy().view(np.uint16)
        for h in range(wl.heads):
            np.testing.assert_array_equal(run.out_bits[r, h], want_bits)


def test_rope_tail_needs_one_buffer(H):
    import sparse_attention_decode_row_amd as dsa
    rng = np.random.default_rng(3)
    wl = WL.with_rope_tail(WL.random_case(rng, rows=2, heads=16, D=512, block_size=64,
                                          max_len=200, width=32))
    _announce("rope separate V refused")
    plan = H.plan_for(wl)
    q, pool = H.q_tensor(wl.q_bits), H.u8(wl.pool)
    other = H.u8(wl.pool)
    out = torch.empty((wl.rows, wl.heads, wl.D), dtype=torch.bfloat16, device=q.device)
    ws = plan.new_workspace()
    with pytest.raises(dsa.DsaDecodeError) as e:
        plan.launch(q, pool, other, H.i32(wl.block_tables), H.i32(wl.seq_lens),
                    H.i32(wl.sel), wl.k_scale, wl.v_scale, out, ws)
    assert e.value.status == dsa.DSA_DECODE_ERR_INVALID
    plan.close()
