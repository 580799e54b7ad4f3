"""Python binding of the LRKV decode library (liblrkv.so, C ABI in include/lrkv.h).

Argument marshalling only: every step of the decode runs in the HIP kernels
behind the C ABI.  Tensors are passed as torch tensors on the GPU (their
data pointers are handed over) or as raw integer device addresses; `stream`
is a torch.cuda.Stream, a raw hipStream_t integer, or None for torch's
current stream.  There is no CPU fallback: if the library is not built the
first call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
# LRKV_LIBRARY selects another build of the same library (tuning experiments); default: in-tree
LIB_PATH = os.environ.get("LRKV_LIBRARY") or os.path.join(_HERE, "liblrkv.so")

LRKV_OK = 0
LRKV_ERR_INVALID_ARG = 1
LRKV_ERR_UNSUPPORTED = 2
LRKV_ERR_WORKSPACE = 3
LRKV_ERR_HIP = 4
LRKV_F32 = 0
LRKV_BF16 = 1

EXPORTED = ("lrkv_absorb_query", "lrkv_cache_append", "lrkv_append_absorb", "lrkv_decode_workspace_bytes", "lrkv_decode_num_splits",
            "lrkv_decode_split_plan",
            "lrkv_decode", "lrkv_decode_partial", "lrkv_decode_merge", "lrkv_decode_step_workspace_bytes",
            "lrkv_decode_step_sync_offset", "lrkv_decode_step_fused", "lrkv_decode_step", "lrkv_decode_noalloc_max_bytes",
            "lrkv_decode_noalloc", "lrkv_latents_to_token_major", "lrkv_decode_multi_workspace_bytes",
            "lrkv_decode_multi", "lrkv_paged_append", "lrkv_decode_paged", "lrkv_rope_table",
            "lrkv_decode_rope_workspace_bytes", "lrkv_decode_rope", "lrkv_key_scales", "lrkv_norm_query",
            "lrkv_decode_normed", "lrkv_materialize", "lrkv_project_append", "lrkv_output_project", "lrkv_read_probe",
            "lrkv_cache_bytes", "lrkv_status_str", "lrkv_last_error")


class LrkvError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        super().__init__(f"{func}: {status_name(status)}: {detail}")
        self.status = status


class Dims(ctypes.Structure):
    """lrkv_dims: batch, H, d_h, r, L_cap, dtype."""
    _fields_ = [("batch", ctypes.c_int32), ("H", ctypes.c_int32), ("d_h", ctypes.c_int32), ("r", ctypes.c_int32),
                ("L_cap", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class Cache(ctypes.Structure):
    """lrkv_cache: device pointers k_shared, v_shared, z_k, z_v, seq_lens."""
    _fields_ = [("k_shared", ctypes.c_void_p), ("v_shared", ctypes.c_void_p), ("z_k", ctypes.c_void_p),
                ("z_v", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p)]


class PagedCache(ctypes.Structure):
    """lrkv_paged_cache: page pools k/v/zk/zv, block_table, seq_lens (device pointers), page_rows, max_pages,
    n_pages."""
    _fields_ = [("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p), ("zk_pages", ctypes.c_void_p),
                ("zv_pages", ctypes.c_void_p), ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("page_rows", ctypes.c_int32), ("max_pages", ctypes.c_int32), ("n_pages", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the in-tree liblrkv.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (python rank_shared_kv_amd/_build.py)")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
        D, C = ctypes.POINTER(Dims), ctypes.POINTER(Cache)
        PC = ctypes.POINTER(PagedCache)
        sig = {
            "lrkv_absorb_query": ([D, vp, vp, vp, vp], ctypes.c_int),
            "lrkv_cache_append": ([D, C, vp, vp, vp, vp, vp], ctypes.c_int),
            "lrkv_append_absorb": ([D, C, vp, vp, vp, vp, vp, vp, vp, vp], ctypes.c_int),
            "lrkv_decode_workspace_bytes": ([D, i32], sz),
            "lrkv_decode_num_splits": ([D, i32, ctypes.POINTER(i32)], i32),
            "lrkv_decode_split_plan": ([D, i32, vp, i32, vp, vp, vp], ctypes.c_int),
            "lrkv_decode": ([D, C, i32, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
            "lrkv_decode_partial": ([D, C, i32, vp, vp, vp, sz, vp], ctypes.c_int),
            "lrkv_decode_merge": ([D, vp, i32, vp, vp, vp, sz, vp], ctypes.c_int),
            "lrkv_decode_step_workspace_bytes": ([D, i32], sz),
            "lrkv_decode_step_sync_offset": ([D, i32], sz),
            "lrkv_decode_step_fused": ([D, i32], i32),
            "lrkv_decode_step": ([D, C, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
            "lrkv_decode_noalloc_max_bytes": ([], sz),
            "lrkv_latents_to_token_major": ([D, vp, vp, vp], ctypes.c_int),
            "lrkv_decode_noalloc": ([D, C, i32, vp, vp, vp, vp, vp], ctypes.c_int),
            "lrkv_decode_multi_workspace_bytes": ([D, i32, i32], sz),
            "lrkv_decode_multi": ([D, i32, C, i32, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
            "lrkv_paged_append": ([D, PC, vp, vp, vp, vp, vp], ctypes.c_int),
            "lrkv_decode_paged": ([D, PC, i32, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
            "lrkv_rope_table": ([i32, i32, ctypes.c_float, vp, vp], ctypes.c_int),
            "lrkv_read_probe": ([vp, sz, vp, vp], ctypes.c_int),
            "lrkv_decode_rope_workspace_bytes": ([D, i32], sz),
            "lrkv_decode_rope": ([D, C, i32, vp, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
            "lrkv_key_scales": ([D, C, i32, i32, vp, ctypes.c_float, vp, vp], ctypes.c_int),
            "lrkv_norm_query": ([D, vp, vp, vp, ctypes.c_float, vp, vp], ctypes.c_int),
            "lrkv_decode_normed": ([D, C, vp, i32, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
            "lrkv_materialize": ([D, C, i32, vp, vp, vp, vp, vp], ctypes.c_int),
            "lrkv_project_append": ([D, i32, C, vp, vp, vp, vp], ctypes.c_int),
            "lrkv_output_project": ([D, i32, vp, vp, vp, vp], ctypes.c_int),
            "lrkv_cache_bytes": ([D, vp], ctypes.c_uint64),
            "lrkv_status_str": ([ctypes.c_int], ctypes.c_char_p),
            "lrkv_last_error": ([], ctypes.c_char_p),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def status_name(status: int) -> str:
    return lib().lrkv_status_str(status).decode()


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        if not getattr(x, "is_cuda", False):
            raise ValueError("tensor arguments must live on the GPU")
        return x.data_ptr()
    if hasattr(x, "ctypes"):  # numpy array (host arrays only where the C ABI says host)
        return x.ctypes.data
    raise TypeError(f"cannot pass {type(x)} as a pointer")


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, func: str):
    if status != LRKV_OK:
        raise LrkvError(status, func, lib().lrkv_last_error().decode())


def make_dims(batch: int, H: int, d_h: int, r: int, L_cap: int, dtype: int) -> Dims:
    return Dims(batch, H, d_h, r, L_cap, dtype)


def make_cache(k_shared, v_shared, z_k, z_v, seq_lens) -> Cache:
    c = Cache(_ptr(k_shared), _ptr(v_shared), _ptr(z_k), _ptr(z_v), _ptr(seq_lens))
    c._tensors = (k_shared, v_shared, z_k, z_v, seq_lens)  # keep the pointed-to tensors alive with the structure
    return c


def lrkv_absorb_query(dims: Dims, q, B_k, p, stream=None) -> None:
    _check(lib().lrkv_absorb_query(ctypes.byref(dims), _ptr(q), _ptr(B_k), _ptr(p), _stream(stream)),
           "lrkv_absorb_query")


def lrkv_cache_append(dims: Dims, cache: Cache, k_new, v_new, zk_new, zv_new, stream=None) -> None:
    _check(lib().lrkv_cache_append(ctypes.byref(dims), ctypes.byref(cache), _ptr(k_new), _ptr(v_new), _ptr(zk_new),
                                   _ptr(zv_new), _stream(stream)), "lrkv_cache_append")


def lrkv_append_absorb(dims: Dims, cache: Cache, k_new, v_new, zk_new, zv_new, q, B_k, p, stream=None) -> None:
    _check(lib().lrkv_append_absorb(ctypes.byref(dims), ctypes.byref(cache), _ptr(k_new), _ptr(v_new), _ptr(zk_new),
                                    _ptr(zv_new), _ptr(q), _ptr(B_k), _ptr(p), _stream(stream)), "lrkv_append_absorb")


def lrkv_decode_workspace_bytes(dims: Dims, max_len: int) -> int:
    return int(lib().lrkv_decode_workspace_bytes(ctypes.byref(dims), max_len))


def lrkv_decode_num_splits(dims: Dims, max_len: int) -> Tuple[int, int]:
    chunk = ctypes.c_int32(0)
    s = lib().lrkv_decode_num_splits(ctypes.byref(dims), max_len, ctypes.byref(chunk))
    return int(s), int(chunk.value)


def lrkv_decode_split_plan(dims: Dims, max_len: int, seq_lens, append: int, first_wg, splits, stream=None) -> None:
    _check(lib().lrkv_decode_split_plan(ctypes.byref(dims), max_len, _ptr(seq_lens), append, _ptr(first_wg),
                                        _ptr(splits), _stream(stream)), "lrkv_decode_split_plan")


def lrkv_decode(dims: Dims, cache: Cache, max_len: int, q, p, B_v, out, workspace, workspace_bytes: int,
                stream=None) -> None:
    _check(lib().lrkv_decode(ctypes.byref(dims), ctypes.byref(cache), max_len, _ptr(q), _ptr(p), _ptr(B_v), _ptr(out),
                             _ptr(workspace), workspace_bytes, _stream(stream)), "lrkv_decode")


def lrkv_decode_step_workspace_bytes(dims: Dims, max_len: int) -> int:
    return int(lib().lrkv_decode_step_workspace_bytes(ctypes.byref(dims), max_len))


def lrkv_decode_step_sync_offset(dims: Dims, max_len: int) -> int:
    return int(lib().lrkv_decode_step_sync_offset(ctypes.byref(dims), max_len))


def lrkv_decode_step_fused(dims: Dims, max_len: int) -> bool:
    return bool(lib().lrkv_decode_step_fused(ctypes.byref(dims), max_len))


def lrkv_decode_step(dims: Dims, cache: Cache, max_len: int, k_new, v_new, zk_new, zv_new, q, B_k, B_v, p, out,
                     workspace, workspace_bytes: int, stream=None) -> None:
    _check(lib().lrkv_decode_step(ctypes.byref(dims), ctypes.byref(cache), max_len, _ptr(k_new), _ptr(v_new),
                                  _ptr(zk_new), _ptr(zv_new), _ptr(q), _ptr(B_k), _ptr(B_v), _ptr(p), _ptr(out),
                                  _ptr(workspace), workspace_bytes, _stream(stream)), "lrkv_decode_step")


def lrkv_latents_to_token_major(dims: Dims, src, dst, stream=None) -> None:
    _check(lib().lrkv_latents_to_token_major(ctypes.byref(dims), _ptr(src), _ptr(dst), _stream(stream)),
           "lrkv_latents_to_token_major")


def lrkv_decode_noalloc_max_bytes() -> int:
    return int(lib().lrkv_decode_noalloc_max_bytes())


def lrkv_decode_noalloc(dims: Dims, cache: Cache, max_len: int, q, p, B_v, out, stream=None) -> None:
    _check(lib().lrkv_decode_noalloc(ctypes.byref(dims), ctypes.byref(cache), max_len, _ptr(q), _ptr(p), _ptr(B_v),
                                     _ptr(out), _stream(stream)), "lrkv_decode_noalloc")


def lrkv_decode_partial(dims: Dims, cache: Cache, max_len: int, q, p, workspace, workspace_bytes: int,
                        stream=None) -> None:
    _check(lib().lrkv_decode_partial(ctypes.byref(dims), ctypes.byref(cache), max_len, _ptr(q), _ptr(p),
                                     _ptr(workspace), workspace_bytes, _stream(stream)), "lrkv_decode_partial")


def lrkv_decode_merge(dims: Dims, seq_lens, max_len: int, B_v, out, workspace, workspace_bytes: int,
                      stream=None) -> None:
    _check(lib().lrkv_decode_merge(ctypes.byref(dims), _ptr(seq_lens), max_len, _ptr(B_v), _ptr(out),
                                   _ptr(workspace), workspace_bytes, _stream(stream)), "lrkv_decode_merge")


def lrkv_decode_multi_workspace_bytes(dims: Dims, n_queries: int, max_len: int) -> int:
    return int(lib().lrkv_decode_multi_workspace_bytes(ctypes.byref(dims), n_queries, max_len))


def lrkv_decode_multi(dims: Dims, n_queries: int, cache: Cache, max_len: int, q, p, B_v, out, workspace,
                      workspace_bytes: int, stream=None) -> None:
    _check(lib().lrkv_decode_multi(ctypes.byref(dims), n_queries, ctypes.byref(cache), max_len, _ptr(q), _ptr(p),
                                   _ptr(B_v), _ptr(out), _ptr(workspace), workspace_bytes, _stream(stream)),
           "lrkv_decode_multi")


def make_paged_cache(k_pages, v_pages, zk_pages, zv_pages, block_table, seq_lens, page_rows: int, max_pages: int,
                     n_pages: int) -> PagedCache:
    pc = PagedCache(_ptr(k_pages), _ptr(v_pages), _ptr(zk_pages), _ptr(zv_pages), _ptr(block_table),
                    _ptr(seq_lens), page_rows, max_pages, n_pages)
    # the structure holds raw device pointers: keep the tensors alive as long as it is
    pc._tensors = (k_pages, v_pages, zk_pages, zv_pages, block_table, seq_lens)
    return pc


def lrkv_paged_append(dims: Dims, cache: PagedCache, k_new, v_new, zk_new, zv_new, stream=None) -> None:
    _check(lib().lrkv_paged_append(ctypes.byref(dims), ctypes.byref(cache), _ptr(k_new), _ptr(v_new), _ptr(zk_new),
                                   _ptr(zv_new), _stream(stream)), "lrkv_paged_append")


def lrkv_decode_paged(dims: Dims, cache: PagedCache, max_len: int, q, p, B_v, out, workspace, workspace_bytes: int,
                      stream=None) -> None:
    _check(lib().lrkv_decode_paged(ctypes.byref(dims), ctypes.byref(cache), max_len, _ptr(q), _ptr(p), _ptr(B_v),
                                   _ptr(out), _ptr(workspace), workspace_bytes, _stream(stream)), "lrkv_decode_paged")


READ_PROBE_SINK_WORDS = 1024


def lrkv_read_probe(src, nbytes: int, sink, stream=None) -> None:
    _check(lib().lrkv_read_probe(_ptr(src), nbytes, _ptr(sink), _stream(stream)), "lrkv_read_probe")


def lrkv_rope_table(d_h: int, n_pos: int, base: float, table, stream=None) -> None:
    _check(lib().lrkv_rope_table(d_h, n_pos, float(base), _ptr(table), _stream(stream)), "lrkv_rope_table")


def lrkv_decode_rope_workspace_bytes(dims: Dims, max_len: int) -> int:
    return int(lib().lrkv_decode_rope_workspace_bytes(ctypes.byref(dims), max_len))


def lrkv_decode_rope(dims: Dims, cache: Cache, max_len: int, q, B_k, table, B_v, out, workspace, workspace_bytes: int,
                     stream=None) -> None:
    _check(lib().lrkv_decode_rope(ctypes.byref(dims), ctypes.byref(cache), max_len, _ptr(q), _ptr(B_k), _ptr(table),
                                  _ptr(B_v), _ptr(out), _ptr(workspace), workspace_bytes, _stream(stream)),
           "lrkv_decode_rope")


def lrkv_key_scales(dims: Dims, cache: Cache, max_len: int, n_last: int, B_k, eps: float, rho, stream=None) -> None:
    _check(lib().lrkv_key_scales(ctypes.byref(dims), ctypes.byref(cache), max_len, n_last, _ptr(B_k), float(eps),
                                 _ptr(rho), _stream(stream)), "lrkv_key_scales")


def lrkv_norm_query(dims: Dims, q, g_q, g_k, eps: float, q_eff, stream=None) -> None:
    _check(lib().lrkv_norm_query(ctypes.byref(dims), _ptr(q), _ptr(g_q), _ptr(g_k), float(eps), _ptr(q_eff),
                                 _stream(stream)), "lrkv_norm_query")


def lrkv_decode_normed(dims: Dims, cache: Cache, rho, max_len: int, q_eff, p, B_v, out, workspace,
                       workspace_bytes: int, stream=None) -> None:
    _check(lib().lrkv_decode_normed(ctypes.byref(dims), ctypes.byref(cache), _ptr(rho), max_len, _ptr(q_eff),
                                    _ptr(p), _ptr(B_v), _ptr(out), _ptr(workspace), workspace_bytes,
                                    _stream(stream)), "lrkv_decode_normed")


def lrkv_materialize(dims: Dims, cache: Cache, max_len: int, B_k, B_v, K_out, V_out, stream=None) -> None:
    _check(lib().lrkv_materialize(ctypes.byref(dims), ctypes.byref(cache), max_len, _ptr(B_k), _ptr(B_v), _ptr(K_out),
                                  _ptr(V_out), _stream(stream)), "lrkv_materialize")


def lrkv_project_append(dims: Dims, d_model: int, cache: Cache, x, W_in, q_out, stream=None) -> None:
    _check(lib().lrkv_project_append(ctypes.byref(dims), d_model, ctypes.byref(cache), _ptr(x), _ptr(W_in),
                                     _ptr(q_out), _stream(stream)), "lrkv_project_append")


def lrkv_output_project(dims: Dims, d_model: int, o, W_o, y, stream=None) -> None:
    _check(lib().lrkv_output_project(ctypes.byref(dims), d_model, _ptr(o), _ptr(W_o), _ptr(y), _stream(stream)),
           "lrkv_output_project")


def lrkv_cache_bytes(dims: Dims, host_seq_lens: Optional[Sequence[int]] = None) -> int:
    if host_seq_lens is None:
        return int(lib().lrkv_cache_bytes(ctypes.byref(dims), None))
    arr = (ctypes.c_int32 * len(host_seq_lens))(*[int(x) for x in host_seq_lens])
    return int(lib().lrkv_cache_bytes(ctypes.byref(dims), ctypes.cast(arr, ctypes.c_void_p)))
