"""MI355X (gfx950) selected-index NoPE MLA paged decode: Python binding.

A thin ctypes layer over ``libdsa_decode.so`` (C ABI in include/dsa_decode.h).
It only marshals arguments: torch tensors become device pointers, the current
torch stream becomes the launch stream, and the library's status codes become
exceptions. Every step of the decode runs in the library's HIP kernels; if
the library is not built, every call raises.

    plan = Plan(num_rows=R, num_q_heads=H, kv_lora_rank=512, block_size=64,
                index_kpool=4, sel_width=2048, block_table_stride=128,
                max_seq_len=8192, sm_scale=1/16, device=0)
    ws = plan.new_workspace()          # allocated and zeroed once
    plan.launch(q, cache, cache, block_tables, seq_lens, sel, k_scale, v_scale,
                out, ws)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))

DSA_DECODE_OK = 0
DSA_DECODE_ERR_INVALID = -1
DSA_DECODE_ERR_UNSUPPORTED = -2
DSA_DECODE_ERR_DEVICE = -3
DSA_DECODE_ERR_WORKSPACE = -4
DSA_DECODE_ERR_LAUNCH = -5

DSA_DECODE_FLAG_EXPORT_SELECTION = 1
DSA_DECODE_FLAG_MERGE_IN_KERNEL = 2

EXPORTED_SYMBOLS = (
    "dsa_decode_plan", "dsa_decode_plan_destroy", "dsa_decode_workspace_bytes",
    "dsa_decode_workspace_init", "dsa_decode_plan_get_info", "dsa_decode_launch", "dsa_decode_read_selection",
    "dsa_decode_timing_begin", "dsa_decode_timing_end", "dsa_decode_last_error",
    "dsa_decode_version", "dsa_decode_latent_write", "dsa_decode_masked_reference",
    "dsa_decode_launch_static",
)


def library_path() -> str:
    return os.path.join(_HERE, "libdsa_decode.so")


class DsaDecodeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[status {status}] {message}")
        self.status = status


class Params(ctypes.Structure):
    _fields_ = [
        ("num_rows", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("kv_lora_rank", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("index_kpool", ctypes.c_int32),
        ("sel_width", ctypes.c_int32),
        ("block_table_stride", ctypes.c_int32),
        ("cache_stride_bytes", ctypes.c_uint64),
        ("max_seq_len", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("chunk_tokens", ctypes.c_int32),
        ("layout", ctypes.c_int32),
        ("rows_per_sequence", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("qk_rope_dim", ctypes.c_int32),
        ("reserved", ctypes.c_int32 * 2),
    ]


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("device", ctypes.c_int32),
        ("chunk_tokens", ctypes.c_int32),
        ("chunks_per_row", ctypes.c_int32),
        ("head_blocks", ctypes.c_int32),
        ("workgroups", ctypes.c_int32),
        ("merges_chunks", ctypes.c_int32),
        ("num_cus", ctypes.c_int32),
        ("chunk_lead", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_uint64),
        ("layout", ctypes.c_int32),
        ("heads_per_block", ctypes.c_int32),
        ("rows_per_sequence", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("qk_rope_dim", ctypes.c_int32),
        ("status_offset", ctypes.c_uint64),
        ("counters_offset", ctypes.c_uint64),
    ]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_ if name != "reserved"}


_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library; raise if it has not been built."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: the HIP extension is not built "
                "(run __graft_entry__.build()); there is no other implementation")
        L = ctypes.CDLL(path)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.dsa_decode_plan.restype = ctypes.c_int
        L.dsa_decode_plan.argtypes = [ctypes.POINTER(Params), ctypes.c_int, ctypes.POINTER(vp)]
        L.dsa_decode_plan_destroy.restype = None
        L.dsa_decode_plan_destroy.argtypes = [vp]
        L.dsa_decode_workspace_bytes.restype = sz
        L.dsa_decode_workspace_bytes.argtypes = [vp]
        L.dsa_decode_workspace_init.restype = ctypes.c_int
        L.dsa_decode_workspace_init.argtypes = [vp, vp, sz, vp]
        L.dsa_decode_plan_get_info.restype = ctypes.c_int
        L.dsa_decode_plan_get_info.argtypes = [vp, ctypes.POINTER(PlanInfo)]
        L.dsa_decode_launch.restype = ctypes.c_int
        L.dsa_decode_launch.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_float,
                                        ctypes.c_float, vp, vp, sz, vp]
        L.dsa_decode_launch_static.restype = ctypes.c_int
        L.dsa_decode_launch_static.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_float,
                                               ctypes.c_float, vp, vp]
        L.dsa_decode_read_selection.restype = ctypes.c_int
        L.dsa_decode_read_selection.argtypes = [vp, vp, sz, vp, vp, vp, vp]
        L.dsa_decode_timing_begin.restype = ctypes.c_int
        L.dsa_decode_timing_begin.argtypes = [vp, i32]
        L.dsa_decode_timing_end.restype = ctypes.c_int
        L.dsa_decode_timing_end.argtypes = [vp, ctypes.POINTER(ctypes.c_float),
                                            ctypes.POINTER(i32)]
        L.dsa_decode_last_error.restype = ctypes.c_char_p
        L.dsa_decode_last_error.argtypes = []
        L.dsa_decode_version.restype = ctypes.c_int
        L.dsa_decode_version.argtypes = []
        L.dsa_decode_latent_write.restype = ctypes.c_int
        L.dsa_decode_latent_write.argtypes = [vp, vp, vp, i32, i32, i32, ctypes.c_uint64,
                                              ctypes.c_float, ctypes.c_float, vp, vp]
        L.dsa_decode_masked_reference.restype = ctypes.c_int
        L.dsa_decode_masked_reference.argtypes = [ctypes.POINTER(Params), vp, vp, vp, vp, vp, vp,
                                           ctypes.c_float, ctypes.c_float, vp, vp]
        _lib = L
    return _lib


def last_error() -> str:
    return lib().dsa_decode_last_error().decode()


def _check(status: int) -> None:
    if status != DSA_DECODE_OK:
        raise DsaDecodeError(status, last_error())


def _ptr(x) -> Optional[int]:
    """Device pointer of a torch tensor (or an int / None passed through)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


class Plan:
    """A validated decode geometry (dsa_decode_plan). device=-1 builds a
    host-only plan (validation and sizing, no launches). export_selection
    sets DSA_DECODE_FLAG_EXPORT_SELECTION (needed by read_selection),
    merge_in_kernel DSA_DECODE_FLAG_MERGE_IN_KERNEL."""

    def __init__(self, *, num_rows: int, num_q_heads: int, kv_lora_rank: int,
                 block_size: int, index_kpool: int, sel_width: int,
                 block_table_stride: int, max_seq_len: int, sm_scale: float,
                 num_kv_heads: int = 1, cache_stride_bytes: int = 0,
                 chunk_tokens: int = 0, layout: int = 0, rows_per_sequence: int = 0,
                 export_selection: bool = False, merge_in_kernel: bool = False,
                 flags: int = 0, qk_rope_dim: int = 0, device: Optional[int] = None):
        if device is None:
            import torch
            device = torch.cuda.current_device()
        self._lib = lib()
        if export_selection:
            flags |= DSA_DECODE_FLAG_EXPORT_SELECTION
        if merge_in_kernel:
            flags |= DSA_DECODE_FLAG_MERGE_IN_KERNEL
        self.params = Params(num_rows, num_q_heads, num_kv_heads, kv_lora_rank,
                             block_size, index_kpool, sel_width, block_table_stride,
                             cache_stride_bytes, max_seq_len, sm_scale, chunk_tokens,
                             layout, rows_per_sequence, flags, qk_rope_dim,
                             (ctypes.c_int32 * 2)(0, 0))
        h = ctypes.c_void_p()
        _check(self._lib.dsa_decode_plan(ctypes.byref(self.params), int(device),
                                         ctypes.byref(h)))
        self._h = h

    @property
    def handle(self) -> ctypes.c_void_p:
        if self._h is None:
            raise RuntimeError("plan has been destroyed")
        return self._h

    @property
    def workspace_bytes(self) -> int:
        return int(self._lib.dsa_decode_workspace_bytes(self.handle))

    def workspace_init(self, workspace, workspace_bytes=None, stream=None) -> None:
        """Zero `workspace` for this plan (once after allocation, and before
        reusing it with another plan)."""
        if workspace_bytes is None:
            workspace_bytes = workspace.numel() * workspace.element_size()
        _check(self._lib.dsa_decode_workspace_init(
            self.handle, _ptr(workspace), int(workspace_bytes), _stream(stream)))

    def new_workspace(self, device=None, stream=None):
        """A torch uint8 device tensor of workspace_bytes, zeroed for this plan."""
        import torch
        dev = torch.device("cuda", torch.cuda.current_device() if device is None else device)
        ws = torch.empty(max(self.workspace_bytes, 256), dtype=torch.uint8, device=dev)
        self.workspace_init(ws, stream=stream)
        return ws

    def info(self) -> dict:
        inf = PlanInfo()
        _check(self._lib.dsa_decode_plan_get_info(self.handle, ctypes.byref(inf)))
        return inf.as_dict()

    def launch(self, q, k_cache, v_cache, block_tables, seq_lens, sel_indices,
               k_scale: float, v_scale: float, out, workspace, workspace_bytes=None,
               stream=None) -> None:
        if workspace_bytes is None:
            workspace_bytes = (workspace.numel() * workspace.element_size()
                               if hasattr(workspace, "numel") else 0)
        _check(self._lib.dsa_decode_launch(
            self.handle, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
            _ptr(seq_lens), _ptr(sel_indices), float(k_scale), float(v_scale),
            _ptr(out), _ptr(workspace), int(workspace_bytes), _stream(stream)))

    def launch_static(self, q, k_cache, v_cache, block_tables, seq_lens, sel_indices,
                      k_scale: float, v_scale: float, out, stream=None) -> None:
        """dsa_decode_launch_static: the decode with the library's static
        scratch instead of a caller workspace (allocates nothing)."""
        _check(self._lib.dsa_decode_launch_static(
            self.handle, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
            _ptr(seq_lens), _ptr(sel_indices), float(k_scale), float(v_scale),
            _ptr(out), _stream(stream)))

    def read_selection(self, workspace, ids=None, counts=None, offsets=None,
                       workspace_bytes=None, stream=None) -> None:
        if workspace_bytes is None:
            workspace_bytes = workspace.numel() * workspace.element_size()
        _check(self._lib.dsa_decode_read_selection(
            self.handle, _ptr(workspace), int(workspace_bytes), _ptr(ids),
            _ptr(counts), _ptr(offsets), _stream(stream)))

    def timing_begin(self, max_launches: int) -> None:
        _check(self._lib.dsa_decode_timing_begin(self.handle, int(max_launches)))

    def timing_end(self) -> Tuple[float, int]:
        """(milliseconds in the decode kernel summed over the recorded
        launches, number of launches recorded)."""
        ms = ctypes.c_float()
        n = ctypes.c_int32()
        _check(self._lib.dsa_decode_timing_end(self.handle, ctypes.byref(ms),
                                               ctypes.byref(n)))
        return float(ms.value), int(n.value)

    def close(self) -> None:
        if getattr(self, "_h", None) is not None:
            self._lib.dsa_decode_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def decode(q, k_cache, v_cache, block_tables, seq_lens, sel_indices, *,
           k_scale: float, v_scale: float, block_size: int, index_kpool: int,
           block_table_stride: int, max_seq_len: int, sm_scale: float,
           cache_stride_bytes: int = 0, chunk_tokens: int = 0, out=None,
           workspace=None, stream=None):
    """One-shot helper: plan, allocate out/workspace with torch, launch.
    q: bf16 [R, H, D] on the GPU; returns out (bf16 [R, H, D]). A workspace
    passed in must have been zeroed for this geometry (Plan.workspace_init).
    Buffers it allocates come from the launch stream's pool and are marked as
    used by that stream, so torch does not hand them out again before the
    launch has finished with them."""
    import torch
    R, H, D = q.shape
    plan = Plan(num_rows=R, num_q_heads=H, kv_lora_rank=D, block_size=block_size,
                index_kpool=index_kpool, sel_width=sel_indices.shape[1],
                block_table_stride=block_table_stride, max_seq_len=max_seq_len,
                sm_scale=sm_scale, cache_stride_bytes=cache_stride_bytes,
                chunk_tokens=chunk_tokens, device=q.device.index)
    if stream is None or isinstance(stream, int):
        ts = torch.cuda.current_stream(q.device) if stream is None else \
            torch.cuda.ExternalStream(stream, device=q.device)
    else:
        ts = stream
    try:
        with torch.cuda.stream(ts):
            if out is None:
                out = torch.empty_like(q)
                out.record_stream(ts)
            if workspace is None:
                workspace = plan.new_workspace(q.device.index, stream=ts)
                workspace.record_stream(ts)
        plan.launch(q, k_cache, v_cache, block_tables, seq_lens, sel_indices,
                    k_scale, v_scale, out, workspace, stream=ts)
    finally:
        plan.close()
    return out


def latent_write(kv_a, weight, slots, k_pool, *, block_size: int, rms_eps: float,
                 inv_kv_scale: float, cache_stride_bytes: int = 0, stream=None) -> None:
    """The cache writer: kv_a bf16 [N, D], weight bf16 [D], slots int64 [N]
    (negative: skipped), k_pool the uint8 FP8 pool, all on the GPU. Writes
    the FP8 rows in place; asynchronous on `stream`."""
    n, d = kv_a.shape
    _check(lib().dsa_decode_latent_write(
        _ptr(kv_a), _ptr(weight), _ptr(slots), int(n), int(d), int(block_size),
        int(cache_stride_bytes), float(rms_eps), float(inv_kv_scale), _ptr(k_pool),
        _stream(stream)))


def masked_reference(q, k_cache, v_cache, block_tables, seq_lens, sel_indices, *,
                     k_scale: float, v_scale: float, block_size: int, index_kpool: int,
                     block_table_stride: int, max_seq_len: int, sm_scale: float,
                     cache_stride_bytes: int = 0, out=None, stream=None):
    """Dense masked-attention reference of the decode on the GPU
    (dsa_decode_masked_reference): plain fp32, one workgroup per (row, head). Same
    inputs as decode(); returns out, float32 [R, H, D]."""
    import torch
    R, H, D = q.shape
    params = Params(R, H, 1, D, block_size, index_kpool, sel_indices.shape[1],
                    block_table_stride, cache_stride_bytes, max_seq_len, sm_scale, 0, 0, 0,
                    0, 0, (ctypes.c_int32 * 2)(0, 0))
    if out is None:
        out = torch.empty((R, H, D), dtype=torch.float32, device=q.device)
    _check(lib().dsa_decode_masked_reference(
        ctypes.byref(params), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        _ptr(seq_lens), _ptr(sel_indices), float(k_scale), float(v_scale), _ptr(out),
        _stream(stream)))
    return out
