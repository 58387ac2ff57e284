"""fp64 CPU oracle for attention over a paged KV cache -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package.  It is independent of the HIP library: it neither imports nor
links anything from ``paged_kv_cache_98_amd`` and shares no helper with it.

Contents
  * ``kv_append`` / ``paged_attention``: ctypes wrappers over the plain C
    fp64 reference in ``pkv_oracle.c`` (gather into contiguous K/V, then
    three-pass softmax attention).
  * ``online``: fp64 replicas of the single-pass online-softmax recurrence and
    of the log-sum-exp merge of partition summaries.
  * ``sizing``: the pages' KV-cache and block-memory formulas.
  * ``blocks``: the pages' block pool (allocate / free / fork / append with
    copy-on-write, reference counts) and the whole-block copy of
    copy-on-write.
  * ``fp8``: the E4M3 format, the quantised append and the fp64 decode and
    chunked prefill over an FP8 cache with per-cache scales.
  * ``tree``: fp64 attention of token-tree verification chunks (each node
    sees the context and its own path).

Every function names the passage it follows.  Functions without an
independent pin say "parity unpinned" in their docstring (none at present).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_kv_append.restype = ctypes.c_int
    lib.oracle_kv_append.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
        ctypes.c_int, ctypes.c_int]
    lib.oracle_paged_attention.restype = ctypes.c_int
    lib.oracle_paged_attention.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_int, ctypes.c_int]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    _lib = lib
    return lib


class OracleError(RuntimeError):
    pass


def _u16(a):
    """A C-contiguous uint16 view of bf16 data (numpy uint16/int16 or torch bf16)."""
    if hasattr(a, "detach"):  # torch tensor
        import torch
        if a.dtype != torch.bfloat16:
            raise TypeError("expected a bfloat16 tensor")
        a = a.detach().cpu().contiguous().view(torch.int16).numpy()
    a = np.ascontiguousarray(a)
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError("expected bf16 bit patterns as uint16")
    return a


def _i(a, dtype):
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def max_threads() -> int:
    return _load().oracle_max_threads()


def kv_append(k_new, v_new, slot_mapping, k_cache, v_cache):
    """kv_append reference (byte copy into slot // bs, slot % bs; slot < 0 skipped).

    k_new, v_new: [T, Hkv, D] bf16 bits; k_cache, v_cache: [NB, bs, Hkv, D]
    bf16 bits, returned as new uint16 arrays (inputs are not modified).
    Follows "LLM 推理优化技术全景", section "KV Cache" (append and reuse) and
    "让 Agent 跑得快：LLM 推理服务", section 五 (a block per 16 tokens; only the
    current token writes).
    """
    kn, vn = _u16(k_new), _u16(v_new)
    kc, vc = _u16(k_cache).copy(), _u16(v_cache).copy()
    sm = _i(slot_mapping, np.int64)
    nb, bs, hkv, d = kc.shape
    if kn.shape != (sm.shape[0], hkv, d) or vn.shape != kn.shape or vc.shape != kc.shape:
        raise ValueError("shape mismatch")
    st = _load().oracle_kv_append(_ptr(kn), _ptr(vn), _ptr(sm), sm.shape[0],
                                  _ptr(kc), _ptr(vc), nb, bs, hkv, d)
    if st != 0:
        raise OracleError(f"oracle_kv_append status {st}")
    return kc, vc


def paged_attention(q, k_cache, v_cache, block_table, context_lens, scale,
                    cu_q_lens=None, causal=True, num_threads=0):
    """fp64 attention over the paged cache: gather, then three-pass softmax.

    q: [sum Lq, Hq, D] bf16 (decode: [B, Hq, D] with cu_q_lens None).
    Returns an fp64 numpy array shaped like q.  Follows "LLM 推理优化技术全景",
    "Flash Attention 深度剖析 > 标准注意力的问题" and "在线 Softmax" (the
    three-sweep stable softmax), with the gather of "LLM 推理引擎深度解析 ...",
    section 2.1.
    """
    qa = _u16(q)
    kc, vc = _u16(k_cache), _u16(v_cache)
    bt = _i(block_table, np.int32)
    cl = _i(context_lens, np.int32)
    nb, bs, hkv, d = kc.shape
    nseq = cl.shape[0]
    if bt.ndim != 2 or bt.shape[0] != nseq:
        raise ValueError("block_table must be [num_seqs, max_blocks]")
    hq = qa.shape[1]
    if cu_q_lens is not None:
        cu = _i(cu_q_lens, np.int32)
        if cu.shape != (nseq + 1,) or qa.shape[0] != int(cu[-1]):
            raise ValueError("cu_q_lens does not match q")
        cu_p = _ptr(cu)
    else:
        cu = None
        cu_p = None
        if qa.shape[0] != nseq:
            raise ValueError("decode q must be [num_seqs, Hq, D]")
    out = np.zeros(qa.shape, dtype=np.float64)
    st = _load().oracle_paged_attention(
        _ptr(out), _ptr(qa), cu_p, _ptr(kc), _ptr(vc), nb, _ptr(bt), bt.shape[1],
        _ptr(cl), nseq, hq, hkv, d, bs, float(scale), 1 if causal else 0,
        int(num_threads))
    if st != 0:
        raise OracleError(f"oracle_paged_attention status {st}")
    return out
