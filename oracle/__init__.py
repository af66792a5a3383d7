"""CPU oracle for the selected-index NoPE MLA paged decode (ctypes binding).

TEST INFRASTRUCTURE ONLY: imported by tests/, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py``. The product package never imports it,
and it imports nothing from the product package.

The arithmetic lives in ``dsa_oracle.c`` (plain C, double precision). This
module only moves numpy arrays across the C boundary.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa_oracle.so")
SRC_PATH = os.path.join(_HERE, "dsa_oracle.c")

_lib = None


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc (OpenMP for the (row, head) loop)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", LIB_PATH, SRC_PATH, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return LIB_PATH


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) or (
                os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH)):
            build()
        L = ctypes.CDLL(LIB_PATH)
        L.dsa_oracle_fp8_e4m3fn.restype = ctypes.c_double
        L.dsa_oracle_fp8_e4m3fn.argtypes = [ctypes.c_uint8]
        L.dsa_oracle_bf16.restype = ctypes.c_double
        L.dsa_oracle_bf16.argtypes = [ctypes.c_uint16]
        L.dsa_oracle_select_row.restype = ctypes.c_int32
        L.dsa_oracle_select_row.argtypes = [ctypes.c_void_p, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_void_p]
        L.dsa_oracle_token_offset.restype = ctypes.c_uint64
        L.dsa_oracle_token_offset.argtypes = [ctypes.c_void_p, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.c_uint64,
                                              ctypes.c_int32]
        L.dsa_oracle_decode.restype = ctypes.c_int
        L.dsa_oracle_decode.argtypes = (
            [ctypes.c_int32] * 6 + [ctypes.c_uint64] +
            [ctypes.c_double] * 3 + [ctypes.c_void_p] * 7 + [ctypes.c_int32])
        L.dsa_oracle_decode_qkv.restype = ctypes.c_int
        L.dsa_oracle_decode_qkv.argtypes = (
            [ctypes.c_int32] * 7 + [ctypes.c_uint64] +
            [ctypes.c_double] * 3 + [ctypes.c_void_p] * 7 + [ctypes.c_int32])
        L.dsa_oracle_max_threads.restype = ctypes.c_int32
        L.dsa_oracle_max_threads.argtypes = []
        L.dsa_oracle_fp8_e4m3fn_encode.restype = ctypes.c_uint8
        L.dsa_oracle_fp8_e4m3fn_encode.argtypes = [ctypes.c_double]
        L.dsa_oracle_latent_write.restype = ctypes.c_int
        L.dsa_oracle_latent_write.argtypes = (
            [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
             ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_double,
             ctypes.c_double, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p])
        _lib = L
    return _lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def fp8_e4m3fn(codes) -> np.ndarray:
    """Decode uint8 FP8 E4M3FN codes to float64, one call per code."""
    L = lib()
    flat = np.asarray(codes, dtype=np.uint8).ravel()
    out = np.array([L.dsa_oracle_fp8_e4m3fn(int(c)) for c in flat], dtype=np.float64)
    return out.reshape(np.shape(codes))


def bf16(bits) -> np.ndarray:
    L = lib()
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    out = np.array([L.dsa_oracle_bf16(int(b)) for b in flat], dtype=np.float64)
    return out.reshape(np.shape(bits))


def select_row(sel_row, seq_len: int) -> np.ndarray:
    """Sorted distinct valid ids of one selection row."""
    sel_row = _c(sel_row, np.int32)
    out = np.empty(max(1, sel_row.size), dtype=np.int32)
    n = lib().dsa_oracle_select_row(sel_row.ctypes.data, sel_row.size,
                                    int(seq_len), out.ctypes.data)
    return out[:n].copy()


def token_offset(bt_row, t: int, block_size: int, cache_stride_bytes: int,
                 kv_lora_rank: int) -> int:
    bt_row = _c(bt_row, np.int32)
    return int(lib().dsa_oracle_token_offset(bt_row.ctypes.data, int(t),
                                             int(block_size),
                                             int(cache_stride_bytes),
                                             int(kv_lora_rank)))


def fp8_e4m3fn_encode(values) -> np.ndarray:
    """Nearest FP8 E4M3FN codes (ties to even, saturating at +-448), one call
    per value."""
    L = lib()
    flat = np.asarray(values, dtype=np.float64).ravel()
    out = np.array([L.dsa_oracle_fp8_e4m3fn_encode(float(v)) for v in flat], dtype=np.uint8)
    return out.reshape(np.shape(values))


def latent_write(kv_a_bits, weight_bits, slots, pool, *, block_size: int,
                 cache_stride_bytes: int, eps: float, inv_kv_scale: float):
    """The cache writer: writes the FP8 rows into `pool` (uint8, modified in
    place) and returns the pre-quantisation values [rows, D] (float64)."""
    kv_a_bits = _c(kv_a_bits, np.uint16)
    R, D = kv_a_bits.shape
    w = _c(weight_bits, np.uint16).ravel()
    sl = _c(slots, np.int64).ravel()
    assert w.size == D and sl.size == R
    assert pool.dtype == np.uint8 and pool.flags["C_CONTIGUOUS"]
    values = np.zeros((R, D), dtype=np.float64)
    rc = lib().dsa_oracle_latent_write(R, D, kv_a_bits.ctypes.data, w.ctypes.data,
                                       sl.ctypes.data, int(block_size),
                                       int(cache_stride_bytes), float(eps),
                                       float(inv_kv_scale), pool.ctypes.data,
                                       pool.size, values.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle latent_write rejected its arguments (rc={rc})")
    return values


def max_threads() -> int:
    return int(lib().dsa_oracle_max_threads())


def decode(q_bits, k_cache, v_cache, block_tables, seq_lens, sel, *,
           block_size: int, bt_stride: int, cache_stride_bytes: int,
           sm_scale: float, k_scale: float, v_scale: float,
           num_threads: int = 0, v_dim: int = 0) -> np.ndarray:
    """Full decode. q_bits: [R, H, Dqk] uint16 (bf16 bits); caches: uint8
    pools of Dqk-byte tokens; block_tables: int32 (row stride bt_stride, 0 =
    shared); seq_lens [R]; sel [R, W]. v_dim (default Dqk): the values and the
    output are the first v_dim bytes of each token (a token with a tail after
    its latent). Returns float64 [R, H, v_dim]."""
    q_bits = _c(q_bits, np.uint16)
    R, H, D = q_bits.shape
    Dv = v_dim or D
    sel = _c(sel, np.int32)
    W = sel.shape[1] if sel.ndim == 2 else 0
    k_cache = _c(k_cache, np.uint8).ravel()
    v_cache = k_cache if v_cache is None else _c(v_cache, np.uint8).ravel()
    bt = _c(block_tables, np.int32).ravel()
    sl = _c(seq_lens, np.int32).ravel()
    out = np.zeros((R, H, Dv), dtype=np.float64)
    if Dv == D:
        rc = lib().dsa_oracle_decode(R, H, D, W, int(block_size), int(bt_stride),
                                     int(cache_stride_bytes), float(sm_scale),
                                     float(k_scale), float(v_scale),
                                     q_bits.ctypes.data, k_cache.ctypes.data,
                                     v_cache.ctypes.data, bt.ctypes.data,
                                     sl.ctypes.data, sel.ctypes.data,
                                     out.ctypes.data, int(num_threads))
    else:
        rc = lib().dsa_oracle_decode_qkv(R, H, D, Dv, W, int(block_size), int(bt_stride),
                                         int(cache_stride_bytes), float(sm_scale),
                                         float(k_scale), float(v_scale),
                                         q_bits.ctypes.data, k_cache.ctypes.data,
                                         v_cache.ctypes.data, bt.ctypes.data,
                                         sl.ctypes.data, sel.ctypes.data,
                                         out.ctypes.data, int(num_threads))
    if rc != 0:
        raise ValueError(f"oracle decode rejected its arguments (rc={rc})")
    return out
