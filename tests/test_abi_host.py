"""Host-side tests of the C ABI (no GPU): the library loads and exports what
include/dsa_decode.h declares, the planner's validation rules and the split
decomposition. Rules cited from the pages:
  [attend]   "spark_model/layers/glm5next_dsa/attend.rs" (DsaDecodePaging::validate,
             decode_attention's guards, Glm5NextDsaDecodeKernel::resolve)
  [decode_k] "metrale_model_arch/glm5next_dsa/layer/decode_k.rs" (block-table
             capacity check)
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa_decode.h")

GOOD = dict(num_rows=128, num_q_heads=64, kv_lora_rank=512, block_size=64,
            index_kpool=4, sel_width=2048, block_table_stride=2048,
            max_seq_len=131072, sm_scale=1 / 16)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_decode_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("dsa_decode_plan", "dsa_decode_launch", "dsa_decode_workspace_bytes",
                 "dsa_decode_plan_destroy", "dsa_decode_last_error"):
        assert must in names


def test_library_exports_every_declared_symbol(native):
    lib = ctypes.CDLL(native.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in include/dsa_decode.h but not exported"
    assert set(native.EXPORTED_SYMBOLS) == set(declared_functions())


def test_version(native):
    assert native.lib().dsa_decode_version() == 400


def plan(native, **kw):
    args = dict(GOOD)
    args.update(kw)
    return native.Plan(device=-1, **args)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(num_rows=0), -1, "degenerate launch"),
    (dict(num_q_heads=0), -1, "degenerate launch"),
    (dict(block_size=0), -1, "block_size must be > 0"),
    (dict(index_kpool=0), -1, "index_kpool must be > 0"),
    (dict(block_size=64, index_kpool=6), -1, "not a multiple of index_kpool 6"),
    (dict(num_kv_heads=2), -1, "single latent KV head"),
    (dict(kv_lora_rank=576), -2, "not compiled in"),
    (dict(kv_lora_rank=32), -2, "not compiled in"),
    (dict(sel_width=0), -1, "sel_width must be > 0"),
    (dict(max_seq_len=0), -1, "max_seq_len must be > 0"),
    (dict(block_table_stride=-1), -1, "block_table_stride must be >= 0"),
    (dict(cache_stride_bytes=1000), -1, "smaller than one page"),
    (dict(cache_stride_bytes=64 * 512 + 8), -1, "not a multiple of the token's 512 bytes"),
    (dict(cache_stride_bytes=64 * 512 + 256), -1, "not a multiple of the token's 512 bytes"),
    (dict(qk_rope_dim=32), -2, "qk_rope_dim 32 is not compiled in"),
    (dict(qk_rope_dim=64, kv_lora_rank=256), -2, "kv_lora_rank 512 only"),
    (dict(qk_rope_dim=64, cache_stride_bytes=64 * 512), -1, "smaller than one page"),
    (dict(qk_rope_dim=64, cache_stride_bytes=64 * 576 + 512), -1,
     "not a multiple of the token's 576 bytes"),
    (dict(qk_rope_dim=64, chunk_tokens=4096), -1, "up to 2048"),
    (dict(flags=8), -1, "unknown flags"),
    (dict(block_table_stride=100), -1, "block-table entries per row"),
    (dict(sm_scale=float("inf")), -1, "sm_scale must be finite"),
    (dict(chunk_tokens=100), -1, "chunk_tokens"),
    (dict(chunk_tokens=4096), -1, "chunk_tokens"),
    (dict(rows_per_sequence=-1), -1, "rows_per_sequence"),
    (dict(num_rows=10, rows_per_sequence=4), -1, "divides num_rows 10"),
    (dict(layout=3, kv_lora_rank=256), -2, "64-head blocks"),
    (dict(layout=3, qk_rope_dim=64), -2, "64-head blocks"),
    (dict(layout=3, flags=2), -2, "64-head blocks"),
])
def test_plan_rejects(native, kw, status, needle):
    with pytest.raises(native.DsaDecodeError) as e:
        plan(native, **kw)
    assert e.value.status == status
    assert needle in str(e.value)
    assert needle in native.last_error()


def test_plan_rejects_bad_device_argument(native):
    with pytest.raises(native.DsaDecodeError) as e:
        native.Plan(device=-5, **GOOD)
    assert e.value.status == -1


def test_no_gpu_means_device_error(native):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(native.DsaDecodeError) as e:
        native.Plan(device=0, **GOOD)
    assert e.value.status == native.DSA_DECODE_ERR_DEVICE


def test_rope_tail_plans(native):
    # 576-byte tokens: pages of block_size such tokens by default; a
    # workgroup takes up to 2048 of them like 512-byte tokens (the tails sit
    # in a three-slot ring beside the tile buffers), so the long-context
    # shape keeps one workgroup per (row, head block)
    p = plan(native, qk_rope_dim=64).info()
    assert p["qk_rope_dim"] == 64
    assert p["chunk_tokens"] == 2048 and p["chunks_per_row"] == 1
    assert p["merges_chunks"] == 0 and p["workgroups"] == 256
    q = plan(native, qk_rope_dim=64, cache_stride_bytes=64 * 576 * 2).info()
    assert q["chunks_per_row"] == 1
    # a forced split and the in-kernel merge's lead stay within 2048 tokens
    m = plan(native, qk_rope_dim=64, num_rows=32, max_seq_len=8192, block_table_stride=128,
             merge_in_kernel=True).info()
    assert m["chunks_per_row"] > 1 and m["chunk_tokens"] + m["chunk_lead"] <= 2048


def test_masked_reference_refuses_rope_tail(native):
    P = native.Params(2, 4, 1, 512, 64, 4, 32, 16, 0, 1000, 0.1, 0, 0, 0, 0, 64,
                      (ctypes.c_int32 * 2)(0, 0))
    rc = native.lib().dsa_decode_masked_reference(ctypes.byref(P), 1, 1, 1, 1, 1, 1,
                                                  0.05, 0.05, 1, None)
    assert rc == native.DSA_DECODE_ERR_UNSUPPORTED
    assert "rope" in native.last_error()


def test_shared_table_skips_capacity_rule(native):
    p = plan(native, block_table_stride=0)
    assert p.workspace_bytes > 0


def test_capacity_rule_boundary(native):
    # exactly enough entries: 2048 * 64 = 131072 positions
    plan(native, block_table_stride=2048, max_seq_len=131072)
    with pytest.raises(native.DsaDecodeError):
        plan(native, block_table_stride=2048, max_seq_len=131073)


@pytest.mark.parametrize("kw,chunks,ct", [
    (dict(), 1, 2048),                                        # 128 rows x 2 head blocks
    (dict(num_rows=32, max_seq_len=8192, block_table_stride=128), 4, 512),
    (dict(num_rows=256, max_seq_len=32768, block_table_stride=512), 1, 2048),
    (dict(num_rows=256, max_seq_len=32768, block_table_stride=512, layout=2), 1, 2048),
    (dict(num_rows=2, num_q_heads=4, kv_lora_rank=64, block_size=16,
          sel_width=32, block_table_stride=16, max_seq_len=173), 1, 64),
    (dict(chunk_tokens=192), 11, 192),
    (dict(num_rows=1, sel_width=100, max_seq_len=50, block_table_stride=1), 1, 64),
])
def test_split_plan(native, kw, chunks, ct):
    info = plan(native, **kw).info()
    assert info["chunks_per_row"] == chunks
    assert info["chunk_tokens"] == ct
    assert info["merges_chunks"] == (chunks > 1)
    rows = kw.get("num_rows", 128)
    # one row's chunks are grouped on one XCD: rows padded to a multiple of
    # 8, times the chunks and the head blocks (unsplit rows: the same)
    assert info["workgroups"] == (rows + 7) // 8 * 8 * chunks * info["head_blocks"]
    heads = kw.get("num_q_heads", 64)
    small = kw.get("layout", 0) == 2 or heads <= 16
    # 64-head blocks when one block per row still fills the 256 CUs
    large = (not small and kw.get("layout", 0) == 0 and heads > 32
             and kw.get("kv_lora_rank", 512) == 512 and rows * -(-heads // 64) >= 256)
    assert info["layout"] == (2 if small else 3 if large else 1)
    assert info["heads_per_block"] == (16 if small else 64 if large else 32)
    assert info["head_blocks"] == (heads + info["heads_per_block"] - 1) // info["heads_per_block"]
    assert info["device"] == -1


def test_layouts(native):
    h32 = plan(native, layout=1).info()
    h16 = plan(native, layout=2).info()
    assert (h32["heads_per_block"], h32["head_blocks"], h32["workgroups"]) == (32, 2, 256)
    assert (h16["heads_per_block"], h16["head_blocks"], h16["workgroups"]) == (16, 4, 512)
    # the planner picks 32-head blocks unless the heads fit one 16-head group
    assert plan(native).info()["layout"] == 1
    assert plan(native, num_q_heads=16).info()["layout"] == 2
    assert plan(native, num_q_heads=17).info()["layout"] == 1
    # 64-head blocks: one block per row, the rows split in two to fill the chip
    h64 = plan(native, layout=3).info()
    assert (h64["heads_per_block"], h64["head_blocks"], h64["layout"]) == (64, 1, 3)
    assert (h64["chunks_per_row"], h64["workgroups"]) == (2, 256)
    with pytest.raises(native.DsaDecodeError) as e:
        plan(native, layout=4)
    assert e.value.status == native.DSA_DECODE_ERR_INVALID


def test_chunk_lead(native):
    # split rows: chunk 0 takes one more 128-token tile so that it finishes
    # last and merges; a forced split keeps equal chunks
    assert plan(native).info()["chunk_lead"] == 0          # one chunk per row
    assert plan(native, chunk_tokens=192).info()["chunk_lead"] == 0
    # merged by the combine kernel: equal chunks
    comb = plan(native, num_rows=32, max_seq_len=8192, block_table_stride=128).info()
    assert comb["chunk_tokens"] == 512 and comb["chunk_lead"] == 0
    assert comb["chunks_per_row"] == 4 and comb["merges_chunks"] == 1
    # merged in the kernel by chunk 0, which takes one more tile pair
    split = plan(native, num_rows=32, max_seq_len=8192, block_table_stride=128,
                 merge_in_kernel=True).info()
    assert split["chunk_tokens"] == 512 and split["chunk_lead"] == 128
    assert split["merges_chunks"] == 2
    small = plan(native, num_rows=8, max_seq_len=8192, block_table_stride=128,
                 merge_in_kernel=True).info()
    assert small["chunks_per_row"] == 16 and small["chunk_tokens"] == 128
    assert small["chunk_lead"] == 0                         # a lead must be below the chunk
    # the ranges still cover every rank a row can have
    for info in (plan(native).info(), comb, split, small):
        assert info["chunks_per_row"] * info["chunk_tokens"] + info["chunk_lead"] >= 2048
        assert info["chunk_tokens"] + info["chunk_lead"] <= 2048


def test_workspace_layout(native):
    R, W, C, HB, HPB, D = 32, 2048, 4, 2, 32, 512
    core = 4 + 2 * R * HB * 4 + R * HB * C * HPB * D * 4 + R * HB * C * HPB * 2 * 4
    export = R * W * 4 + R * W * 8 + R * 4
    for flag, need in ((False, core), (True, core + export)):
        p = plan(native, num_rows=32, max_seq_len=8192, block_table_stride=128,
                 export_selection=flag)
        assert need <= p.workspace_bytes <= need + 7 * 256
        info = p.info()
        assert info["flags"] == (1 if flag else 0)
        assert info["status_offset"] == 0 and info["counters_offset"] == 256
    p1 = plan(native)
    assert p1.info()["chunks_per_row"] == 1        # no partials, no export
    assert p1.workspace_bytes <= 4 * 256 + 2 * 128 * 2 * 4
    p2 = plan(native, export_selection=True)
    assert p2.workspace_bytes <= 128 * 2048 * 12 + 128 * 12 + 6 * 256


def test_head_blocks(native):
    assert plan(native, num_q_heads=64, layout=1).info()["head_blocks"] == 2
    assert plan(native, num_q_heads=65, layout=1).info()["head_blocks"] == 3
    assert plan(native, num_q_heads=128, layout=1).info()["head_blocks"] == 4
    assert plan(native, num_q_heads=64, layout=2).info()["head_blocks"] == 4
    assert plan(native, num_q_heads=40, layout=2).info()["head_blocks"] == 3
    assert plan(native, num_q_heads=16).info()["head_blocks"] == 1
    assert plan(native, num_q_heads=8).info()["heads_per_block"] == 16


def test_host_only_plan_cannot_launch(native):
    p = plan(native)
    with pytest.raises(native.DsaDecodeError) as e:
        p.launch(1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 0.02, 0.02,
                 1 << 20, 1 << 20, workspace_bytes=p.workspace_bytes, stream=0)
    assert e.value.status == native.DSA_DECODE_ERR_INVALID
    assert "host-only" in str(e.value)


def test_binding_refuses_without_library(monkeypatch, native):
    import sparse_attention_decode_row_amd as pkg
    monkeypatch.setattr(pkg, "_lib", None)
    monkeypatch.setattr(pkg, "library_path", lambda: "/nonexistent/libdsa_decode.so")
    with pytest.raises(RuntimeError, match="not built"):
        pkg.lib()


# ------------------------------------------------------------ cache writer

def _writer(native, **kw):
    args = dict(kv_a=None, weight=None, slots=None, num_rows=0, kv_lora_rank=512,
                block_size=64, cache_stride_bytes=0, rms_eps=1e-6, inv_kv_scale=50.0,
                k_pool=None, stream=None)
    args.update(kw)
    return native.lib().dsa_decode_latent_write(*args.values())


def test_writer_zero_rows_is_a_no_op(native):
    assert _writer(native) == 0


@pytest.mark.parametrize("kw,status,needle", [
    (dict(kv_lora_rank=96), -2, "not compiled"),
    (dict(block_size=0), -1, "block_size"),
    (dict(cache_stride_bytes=64 * 512 - 16), -1, "cache_stride_bytes"),
    (dict(cache_stride_bytes=64 * 512 + 8), -1, "cache_stride_bytes"),
    (dict(rms_eps=-1.0), -1, "rms_eps"),
    (dict(inv_kv_scale=0.0), -1, "inv_kv_scale"),
    (dict(inv_kv_scale=float("inf")), -1, "inv_kv_scale"),
    (dict(num_rows=-1), -1, "num_rows"),
    (dict(num_rows=4), -1, "NULL"),
    (dict(num_rows=4, kv_a=8, weight=16, slots=16, k_pool=16), -1, "aligned"),
])
def test_writer_rejects(native, kw, status, needle):
    assert _writer(native, **kw) == status
    assert needle in native.last_error()


def test_rows_per_sequence_grid(native):
    """Co-scheduled decode_k rows: the grid covers whole blocks of 8
    sequences, each sequence's rows x chunks units in consecutive rounds."""
    base = dict(num_rows=256, max_seq_len=32768, block_table_stride=512, layout=1)
    plain = plan(native, **base).info()
    assert plain["rows_per_sequence"] == 1
    grouped = plan(native, rows_per_sequence=4, **base).info()
    assert grouped["rows_per_sequence"] == 4
    # 64 sequences fill 8 blocks exactly: the same grid as without grouping
    assert grouped["workgroups"] == plain["workgroups"]
    assert grouped["chunks_per_row"] == plain["chunks_per_row"]
    assert grouped["workspace_bytes"] == plain["workspace_bytes"]
    # 5 sequences of 3 rows: one block of 8 sequences, padded
    odd = plan(native, num_rows=15, rows_per_sequence=3, max_seq_len=32768,
               block_table_stride=512, layout=1).info()
    assert odd["workgroups"] == 8 * 3 * odd["chunks_per_row"] * odd["head_blocks"]
    assert plan(native, rows_per_sequence=1, **base).info()["workgroups"] == plain["workgroups"]


def test_rows_per_sequence_mapping_is_a_bijection():
    """The kernel's workgroup -> (row, chunk) map for grouped units (the
    rows of a co-scheduled sequence, or the chunks of a split row), restated
    here: every unit is hit exactly once, the units of a sequence share an
    XCD (id mod 8) and head blocks of one unit are 8 ids apart."""
    for seqs, k, chunks, hb in [(64, 4, 1, 2), (5, 3, 2, 1), (9, 2, 3, 4), (1, 5, 1, 1),
                                (32, 1, 4, 2), (13, 1, 3, 2), (3, 1, 11, 4)]:
        G = k * chunks
        blocks = -(-seqs // 8)
        grid = blocks * 8 * G * hb
        seen = {}
        for bid in range(grid):
            h = (bid >> 3) % hb
            lin = (bid // (8 * hb)) * 8 + (bid & 7)
            rnd, x = lin >> 3, lin & 7
            blk, i = divmod(rnd, G)
            rc = (blk * 8 + x) * G + i
            if rc >= seqs * k * chunks:
                continue
            assert (rc, h) not in seen
            seen[(rc, h)] = bid
        assert len(seen) == seqs * k * chunks * hb
        for (rc, h), bid in seen.items():
            s = rc // G
            assert bid % 8 == s % 8
            if h > 0:
                assert seen[(rc, h - 1)] == bid - 8


def _reference_call(native, *, rows=2, heads=4, D=64, width=8, **kw):
    """The masked reference with host tensors standing in for device buffers:
    every check these cases reach runs before anything is read."""
    import torch
    args = dict(k_scale=0.05, v_scale=0.05, block_size=16, index_kpool=4,
                block_table_stride=16, max_seq_len=256, sm_scale=0.125)
    args.update(kw)
    q = torch.zeros((rows, heads, D), dtype=torch.bfloat16)
    pool = torch.zeros(64, dtype=torch.uint8)
    bt = torch.zeros((rows, 16), dtype=torch.int32)
    sl = torch.zeros(rows, dtype=torch.int32)
    sel = torch.zeros((rows, width), dtype=torch.int32)
    out = torch.zeros((rows, heads, D), dtype=torch.float32)
    return native.masked_reference(q, pool, pool, bt, sl, sel, out=out, stream=0, **args)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(block_size=0), -1, "block_size must be > 0"),
    (dict(D=576), -2, "not compiled in"),
    (dict(k_scale=float("nan")), -1, "k_scale and v_scale must be finite"),
    (dict(max_seq_len=1 << 22, block_table_stride=1 << 18, width=2048), -1, "bytes of LDS"),
])
def test_masked_reference_rejects(native, kw, status, needle):
    with pytest.raises(native.DsaDecodeError) as e:
        _reference_call(native, **kw)
    assert e.value.status == status
    assert needle in str(e.value)


def test_masked_reference_without_gpu_is_a_device_error(native):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(native.DsaDecodeError) as e:
        _reference_call(native)
    assert e.value.status == native.DSA_DECODE_ERR_DEVICE


def test_planner_invariants_over_random_geometries(native):
    """Property test of the planner (host-only plans): for any valid
    geometry the chunks cover every rank a row can have, no workgroup's
    row table exceeds its 2048 LDS entries, the grid covers every (row,
    chunk, head block) unit in whole rounds of 8 (whole blocks of 8
    sequences when rows are co-scheduled), and the workspace holds the
    status word and counters plus, when rows are split, every partial."""
    from hypothesis import given, settings, strategies as st

    @settings(max_examples=300, deadline=None)
    @given(rows=st.integers(1, 300), heads=st.integers(1, 200),
           D=st.sampled_from([64, 128, 256, 512]), B=st.sampled_from([4, 16, 64]),
           width=st.integers(1, 5000), L=st.integers(1, 300000),
           ct=st.integers(0, 32), layout=st.integers(0, 3), k=st.integers(0, 6))
    def check(rows, heads, D, B, width, L, ct, layout, k):
        if k > 1 and rows % k:
            k = 1
        if layout == 3 and D != 512:
            layout = 0  # 64-head blocks are compiled for the 512-wide latent
        stride = -(-L // B)
        p = native.Plan(device=-1, num_rows=rows, num_q_heads=heads, kv_lora_rank=D,
                        block_size=B, index_kpool=4 if B % 4 == 0 else 1, sel_width=width,
                        block_table_stride=stride, max_seq_len=L, sm_scale=0.1,
                        chunk_tokens=64 * ct, layout=layout, rows_per_sequence=k)
        info = p.info()
        wmax = min(width, L)
        C, T, lead, HB = (info["chunks_per_row"], info["chunk_tokens"], info["chunk_lead"],
                          info["head_blocks"])
        assert T % 64 == 0 and 64 <= T <= 2048
        assert C * T + lead >= wmax                  # every rank is in some chunk
        assert T + lead <= 2048                      # chunk 0's row table fits
        assert (C - 1) * T + lead < max(wmax, 1) or C == 1   # no chunk is always empty
        assert HB == -(-heads // info["heads_per_block"])
        assert info["heads_per_block"] == {1: 32, 2: 16, 3: 64}[info["layout"]]
        if layout:
            assert info["layout"] == layout
        elif info["layout"] == 3:  # chosen only where one block per row fills the chip
            assert D == 512 and heads > 32 and rows * -(-heads // 64) >= info["num_cus"]
        assert info["merges_chunks"] == (C > 1)
        units = rows * C
        # the rows_per_sequence x chunks units of a sequence (one row when
        # rows are not co-scheduled) are grouped whenever there is more than one
        G = info["rows_per_sequence"] * C
        if G > 1:
            assert info["workgroups"] == -(-(rows // info["rows_per_sequence"]) // 8) * 8 * G * HB
        else:
            assert info["workgroups"] == -(-units // 8) * 8 * HB
        assert info["workgroups"] >= units * HB
        need = 4 + 2 * rows * HB * 4                 # status word and counters
        if C > 1:
            slots = rows * HB * C * info["heads_per_block"]
            need += slots * D * 4 + slots * 2 * 4
        assert need <= p.workspace_bytes <= need + 8 * 256
        assert p.info()["counters_offset"] >= 4
        p.close()

    check()
