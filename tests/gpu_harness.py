"""Helpers shared by the GPU tests: move a workload to the device, run the
decode through the C ABI, run the oracle on chosen rows, compare."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import sparse_attention_decode_row_amd as dsa
import workloads as WL

TOL = 1e-2  # max normwise relative error per (row, head)


def dev():
    return torch.device("cuda", torch.cuda.current_device())


def q_tensor(q_bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(q_bits).view(np.int16)).to(dev()).view(torch.bfloat16)


def i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev())


class GpuRun:
    def __init__(self, out, ids, counts, offsets, info):
        self.out = out          # float64 [R, H, D]
        self.out_bits = None    # uint16 [R, H, D]
        self.ids = ids
        self.counts = counts
        self.offsets = offsets
        self.info = info


def plan_for(wl: WL.Workload, chunk_tokens: int = 0, max_seq_len=None,
             layout: int = 0, rows_per_sequence: int = 0,
             export_selection: bool = False, merge_in_kernel: bool = False) -> dsa.Plan:
    return dsa.Plan(num_rows=wl.rows, num_q_heads=wl.heads, kv_lora_rank=wl.D,
                    block_size=wl.block_size, index_kpool=wl.kpool,
                    sel_width=wl.width, block_table_stride=wl.bt_stride,
                    max_seq_len=max_seq_len or wl.max_seq_len,
                    sm_scale=wl.sm_scale,
                    cache_stride_bytes=wl.cache_stride_bytes,
                    chunk_tokens=chunk_tokens, layout=layout,
                    rows_per_sequence=rows_per_sequence,
                    export_selection=export_selection, merge_in_kernel=merge_in_kernel,
                    qk_rope_dim=wl.rope, device=torch.cuda.current_device())


def run_gpu(wl: WL.Workload, *, k_pool=None, v_pool=None, chunk_tokens: int = 0,
            q_bits=None, sel=None, seq_lens=None, with_selection: bool = True,
            max_seq_len=None, layout: int = 0, rows_per_sequence: int = 0,
            merge_in_kernel: bool = False) -> GpuRun:
    """Run the decode on the GPU. k_pool / v_pool: device uint8 tensors
    (default: the workload's host pool uploaded; v_pool defaults to k_pool)."""
    if k_pool is None:
        k_pool = u8(wl.pool)
    if v_pool is None:
        v_pool = k_pool
    q = q_tensor(wl.q_bits if q_bits is None else q_bits)
    bt = i32(wl.block_tables)
    sl = i32(wl.seq_lens if seq_lens is None else seq_lens)
    sl_ = wl.sel if sel is None else sel
    s = i32(sl_)
    out = torch.full((wl.rows, wl.heads, wl.D), float("nan"), dtype=torch.bfloat16,
                     device=dev())
    plan = plan_for(wl, chunk_tokens, max_seq_len=max_seq_len, layout=layout,
                    rows_per_sequence=rows_per_sequence, export_selection=with_selection,
                    merge_in_kernel=merge_in_kernel)
    ws = plan.new_workspace()
    plan.launch(q, k_pool, v_pool, bt, sl, s, wl.k_scale, wl.v_scale, out, ws)
    ids = counts = offs = None
    if with_selection:
        ids = torch.empty((wl.rows, wl.width), dtype=torch.int32, device=dev())
        counts = torch.empty(wl.rows, dtype=torch.int32, device=dev())
        offs = torch.empty((wl.rows, wl.width), dtype=torch.int64, device=dev())
        plan.read_selection(ws, ids=ids, counts=counts, offsets=offs)
    torch.cuda.synchronize()
    res = GpuRun(out.float().cpu().numpy().astype(np.float64),
                 None if ids is None else ids.cpu().numpy(),
                 None if counts is None else counts.cpu().numpy(),
                 None if offs is None else offs.cpu().numpy().view(np.uint64),
                 plan.info())
    res.out_bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
    plan.close()
    return res


def oracle_rows(wl: WL.Workload, rows, *, host_pool=None, host_v_pool=None,
                q_bits=None, sel=None, seq_lens=None) -> np.ndarray:
    """Oracle output for the given rows ([len(rows), H, D] float64)."""
    rows = list(rows)
    pool = wl.pool if host_pool is None else host_pool
    qb = (wl.q_bits if q_bits is None else q_bits)[rows]
    sl_all = wl.seq_lens if seq_lens is None else seq_lens
    sel_all = wl.sel if sel is None else sel
    if wl.bt_stride:
        bt = wl.block_tables[rows]
    else:
        bt = wl.block_tables[:1]
    return oracle.decode(qb, pool, host_v_pool, bt, sl_all[rows], sel_all[rows],
                         block_size=wl.block_size, bt_stride=wl.bt_stride,
                         cache_stride_bytes=wl.cache_stride_bytes,
                         sm_scale=wl.sm_scale, k_scale=wl.k_scale,
                         v_scale=wl.v_scale, v_dim=wl.D)


def normwise_err(got: np.ndarray, want: np.ndarray) -> np.ndarray:
    """Per (row, head): max_d |got - want| / max_d |want| (absolute error
    where the reference row is all zero)."""
    num = np.abs(got - want).max(axis=-1)
    den = np.abs(want).max(axis=-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def check_selection(wl: WL.Workload, run: GpuRun, rows=None, sel=None, seq_lens=None,
                    check_offsets: bool = True) -> None:
    """Bit-exact: the set of ids the GPU attended (and each one's byte
    offset) equals the oracle's."""
    sel_all = wl.sel if sel is None else sel
    sl_all = wl.seq_lens if seq_lens is None else seq_lens
    rows = range(wl.rows) if rows is None else rows
    for r in rows:
        want = oracle.select_row(sel_all[r], int(sl_all[r]))
        n = int(run.counts[r])
        assert n == want.size, f"row {r}: GPU attended {n} ids, oracle {want.size}"
        assert np.array_equal(run.ids[r, :n], want), f"row {r}: attended ids differ"
        if check_offsets:
            table = wl.block_tables[r if wl.bt_stride else 0]
            want_off = np.array([oracle.token_offset(table, int(t), wl.block_size,
                                                     wl.cache_stride_bytes, wl.token_bytes)
                                 for t in want], dtype=np.uint64)
            assert np.array_equal(run.offsets[r, :n], want_off), f"row {r}: offsets differ"


def sub_pool_for_rows(wl: WL.Workload, pool_dev: torch.Tensor, rows):
    """Copy the pages the rows' selections touch back to the host and build a
    compact pool plus a remapped table, so the oracle can run those rows of a
    pool too large for host memory. Returns (host_pool, workload view)."""
    import copy
    rows = list(rows)
    pages = WL.pages_of_rows(wl, rows)
    page_bytes = wl.cache_stride_bytes
    idx = torch.from_numpy(pages.astype(np.int64)).to(pool_dev.device)
    sub = pool_dev.view(-1, page_bytes).index_select(0, idx).cpu().numpy().ravel()
    remap = {int(p): i for i, p in enumerate(pages)}
    v = copy.copy(wl)
    bt = np.zeros_like(wl.block_tables)
    for r in rows:
        src = wl.block_tables[r if wl.bt_stride else 0]
        dst = bt[r if wl.bt_stride else 0]
        for j, p in enumerate(src):
            dst[j] = remap.get(int(p), 0)
    v.block_tables = bt
    v.pool = sub
    v.num_pages = len(pages)
    return sub, v
