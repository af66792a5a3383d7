"""The decode entry point that allocates nothing (dsa_decode_launch_static),
for callers that cannot allocate device memory: it runs the same kernels as
dsa_decode_launch with the library's static scratch in place of a caller
workspace. Checked through the C ABI against dsa_decode_launch on two calls
in a row, the second with a smaller input (the scratch then holds what the
first call left), then a third in 64-head blocks, all split into several
chunks per row so that the arrival counters and the partials are used; and
against the oracle."""
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


def _both(H, wl, **plan_kw):
    """(static-scratch output, workspace output, plan info) for one workload."""
    plan = H.plan_for(wl, **plan_kw)
    q, pool = H.q_tensor(wl.q_bits), H.u8(wl.pool)
    bt, sl, sel = H.i32(wl.block_tables), H.i32(wl.seq_lens), H.i32(wl.sel)
    out_s = torch.full_like(q, float("nan"))
    out_w = torch.full_like(q, float("nan"))
    plan.launch_static(q, pool, pool, bt, sl, sel, wl.k_scale, wl.v_scale, out_s)
    ws = plan.new_workspace()
    plan.launch(q, pool, pool, bt, sl, sel, wl.k_scale, wl.v_scale, out_w, ws)
    torch.cuda.synchronize()
    info = plan.info()
    plan.close()
    return out_s, out_w, info


def test_static_scratch_matches_the_workspace_entry_point(H):
    rng = np.random.default_rng(2024)
    big = WL.random_case(rng, rows=32, heads=64, D=512, block_size=64, max_len=8192,
                         width=2048)
    small = WL.random_case(rng, rows=5, heads=24, D=256, block_size=32, max_len=3000,
                           width=900)
    wide = WL.random_case(rng, rows=4, heads=80, D=512, block_size=64, max_len=4000,
                          width=1500)
    for name, wl, kw in (("first, split into chunks", big, {}),
                         ("second, smaller, 128-token chunks", small, {"chunk_tokens": 128}),
                         ("third, 64-head blocks, 256-token chunks", wide,
                          {"layout": 3, "chunk_tokens": 256})):
        print(f"\n[gpu case] launch_static {name}: rows {wl.rows} heads {wl.heads} "
              f"D {wl.D}", flush=True)
        out_s, out_w, info = _both(H, wl, **kw)
        print("plan", info, flush=True)
        assert info["chunks_per_row"] > 1
        a = out_s.view(torch.int16).cpu().numpy()
        b = out_w.view(torch.int16).cpu().numpy()
        assert np.array_equal(a, b), "static scratch and caller workspace differ"
        want = H.oracle_rows(wl, range(wl.rows))
        err = H.normwise_err(out_s.float().cpu().numpy().astype(np.float64), want)
        print(f"max err {err.max():.3e}", flush=True)
        assert err.max() <= H.TOL


def test_static_scratch_refuses_what_it_cannot_hold(H):
    import sparse_attention_decode_row_amd as dsa
    print("\n[gpu case] launch_static refusals", flush=True)
    dev = torch.device("cuda")
    # 32 chunks per row of 256 rows: about 1 GiB of partials
    p = dsa.Plan(num_rows=256, num_q_heads=64, kv_lora_rank=512, block_size=64,
                 index_kpool=4, sel_width=2048, block_table_stride=128,
                 max_seq_len=8192, sm_scale=1 / 16, chunk_tokens=64, device=0)
    assert p.workspace_bytes > 32 << 20
    x = torch.zeros(1 << 20, dtype=torch.uint8, device=dev)
    with pytest.raises(dsa.DsaDecodeError) as e:
        p.launch_static(x, x, x, x, x, x, 0.02, 0.02, x)
    assert e.value.status == dsa.DSA_DECODE_ERR_WORKSPACE
    assert "static" in str(e.value)
    p.close()
    p = dsa.Plan(num_rows=2, num_q_heads=4, kv_lora_rank=64, block_size=16, index_kpool=4,
                 sel_width=32, block_table_stride=16, max_seq_len=173, sm_scale=0.125,
                 export_selection=True, device=0)
    with pytest.raises(dsa.DsaDecodeError) as e:
        p.launch_static(x, x, x, x, x, x, 0.02, 0.02, x)
    assert e.value.status == dsa.DSA_DECODE_ERR_INVALID
    p.close()
    torch.cuda.synchronize()
