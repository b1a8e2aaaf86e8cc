"""ctypes binding of libcsa2.so: the C ABI declared in include/csa2.h.

Argument marshalling only.  Each function has the name of the C entry point
it calls; tensors (torch) are passed as their device pointers, ``None`` as
NULL, and the stream defaults to torch's current HIP stream.  Every step of
the computation runs in the library's HIP kernels; there is no fallback, and
a missing library is an error.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_int, c_int32, c_int64, c_size_t, c_uint32, c_void_p

import torch  # loads the process's HIP runtime before the library binds to it

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("CSA2_LIB", os.path.join(_HERE, "libcsa2.so"))

CSA2_OK, CSA2_ERR_NULL, CSA2_ERR_SHAPE, CSA2_ERR_ALIGN = 0, 1, 2, 3
CSA2_ERR_SCHEDULE, CSA2_ERR_WORKSPACE, CSA2_ERR_HIP, CSA2_ERR_SCRATCH = 4, 5, 6, 7
CSA2_NOALLOC_SCRATCH_BYTES = 64 << 20
CSA2_FULL, CSA2_REINDEX, CSA2_REUSE = 0, 1, 2
CSA2_OP_TOPK, CSA2_OP_SPARSE_ATTN, CSA2_OP_SWA_MERGE, CSA2_OP_DECODE_LAYERS = 0, 1, 2, 3
CSA2_OP_PREFILL_LAYERS, CSA2_OP_SCORE_TOPK = 4, 5

EXPORTS = ("csa2_index_score", "csa2_topk", "csa2_score_topk", "csa2_sparse_attn",
           "csa2_swa_merge",
           "csa2_pool_append", "csa2_swa_append", "csa2_pool_restore", "csa2_pool_offload",
           "csa2_swa_restore", "csa2_swa_offload",
           "csa2_decode_layers", "csa2_decode_layer", "csa2_decode_layers_noalloc",
           "csa2_prefill_layers", "csa2_workspace_bytes",
           "csa2_status_string",
           "csa2_version")


class csa2_pool(ctypes.Structure):
    _fields_ = [("latent", c_void_p), ("scale", c_void_p), ("idx_key", c_void_p),
                ("B", c_int32), ("M", c_int32), ("D", c_int32), ("HI", c_int32),
                ("DI", c_int32), ("len", c_void_p), ("pages", c_void_p),
                ("page_log2", c_int32)]


class csa2_layer(ctypes.Structure):
    _fields_ = [("mode", c_int32), ("q_idx", c_void_p), ("w_idx", c_void_p),
                ("q", c_void_p), ("swa", c_void_p), ("o", c_void_p), ("lse", c_void_p),
                ("idx_out", c_void_p)]


class Csa2Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (fn, csa2_status_string(status), status))


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("CSA2 HIP library not found at %s; build it with "
                               "`python -m fp4_kv_cache_score_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        L.csa2_index_score.argtypes = [POINTER(csa2_pool), c_void_p, c_void_p, c_int32, c_int64,
                                       c_int32, c_void_p, c_int32, c_void_p, c_void_p, c_void_p]
        L.csa2_topk.argtypes = [c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_int32,
                                c_void_p, c_void_p, c_size_t, c_void_p]
        L.csa2_sparse_attn.argtypes = [POINTER(csa2_pool), c_void_p, c_int32, c_int32, c_void_p,
                                       c_int32, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
        L.csa2_swa_merge.argtypes = [c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p,
                                     c_int32, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
        L.csa2_score_topk.argtypes = [POINTER(csa2_pool), c_void_p, c_void_p, c_int32, c_void_p,
                                      c_void_p, c_size_t, c_void_p]
        L.csa2_decode_layers.argtypes = [POINTER(csa2_pool), POINTER(csa2_layer), c_int32,
                                         c_int32, c_int32, c_int32, c_int32, POINTER(c_int32),
                                         c_void_p, c_size_t, c_void_p]
        L.csa2_decode_layer.argtypes = [POINTER(csa2_pool), POINTER(csa2_layer), c_int32, c_int32,
                                        c_int32, c_int32, c_int32, c_int32, POINTER(c_int32),
                                        c_void_p, c_size_t, c_void_p]
        L.csa2_decode_layers_noalloc.argtypes = [POINTER(csa2_pool), POINTER(csa2_layer),
                                                 c_int32, c_int32, c_int32, c_int32, c_int32,
                                                 POINTER(c_int32), c_void_p]
        L.csa2_prefill_layers.argtypes = [POINTER(csa2_pool), POINTER(csa2_layer), c_int32,
                                          c_int32, c_int64, c_int32, c_int32, c_int32, c_int32,
                                          POINTER(c_int32), c_void_p, c_size_t, c_void_p]
        L.csa2_pool_append.argtypes = [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_void_p,
                                       c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_void_p]
        L.csa2_swa_append.argtypes = [c_void_p, c_int32, c_int32, c_void_p, c_int64, c_int32,
                                      c_void_p]
        for fn in ("csa2_pool_restore", "csa2_pool_offload"):
            getattr(L, fn).argtypes = [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                       c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]
        for fn in ("csa2_swa_restore", "csa2_swa_offload"):
            getattr(L, fn).argtypes = [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p]
        L.csa2_workspace_bytes.argtypes = [c_int, c_int32, c_int32, c_int32, c_int32, c_int32,
                                           c_int32, c_int32]
        L.csa2_workspace_bytes.restype = c_size_t
        L.csa2_status_string.argtypes = [c_int]
        L.csa2_status_string.restype = c_char_p
        L.csa2_version.argtypes = []
        L.csa2_version.restype = c_char_p
        for fn in ("csa2_index_score", "csa2_topk", "csa2_score_topk", "csa2_sparse_attn",
                   "csa2_swa_merge",
                   "csa2_decode_layers", "csa2_decode_layer", "csa2_decode_layers_noalloc",
                   "csa2_prefill_layers", "csa2_pool_append",
                   "csa2_swa_append", "csa2_pool_restore", "csa2_pool_offload",
                   "csa2_swa_restore", "csa2_swa_offload"):
            getattr(L, fn).restype = c_int
        _lib = L
    return _lib


def _p(x):
    """Tensor / int / None -> pointer value for a c_void_p argument."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _s(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    if torch.cuda.is_available():
        return torch.cuda.current_stream().cuda_stream
    return None


def _check(fn, st, raise_on_error):
    if st != CSA2_OK and raise_on_error:
        raise Csa2Error(fn, st)
    return st


def make_pool(latent, scale, idx_key, B: int, M: int, D: int = 512, HI: int = 8,
              DI: int = 64, len=None, pages=None, page_log2: int = 0) -> csa2_pool:
    """len: None, or a device int32 tensor [B] of per-sequence entry counts;
    pages: None (contiguous), or a device int32 page table [B][M >> page_log2]."""
    return csa2_pool(_p(latent), _p(scale), _p(idx_key), B, M, D, HI, DI, _p(len), _p(pages),
                     page_log2 if pages is not None else 0)


def csa2_status_string(status: int) -> str:
    return lib().csa2_status_string(status).decode()


def csa2_version() -> str:
    return lib().csa2_version().decode()


def csa2_workspace_bytes(op: int, B: int, Q: int, M: int, K: int, P: int, W: int,
                         H: int) -> int:
    return int(lib().csa2_workspace_bytes(op, B, Q, M, K, P, W, H))


def csa2_index_score(pool: csa2_pool, q_idx, w_idx, Q: int, pos0: int, ratio: int, cand,
                     P: int, scores, hist=None, stream=None, raise_on_error=True) -> int:
    st = lib().csa2_index_score(ctypes.byref(pool), _p(q_idx), _p(w_idx), Q, pos0, ratio,
                                _p(cand), P, _p(scores), _p(hist), _s(stream))
    return _check("csa2_index_score", st, raise_on_error)


def csa2_topk(scores, R: int, N: int, n_valid, cand, K: int, idx, ws, ws_bytes: int,
              stream=None, raise_on_error=True) -> int:
    st = lib().csa2_topk(_p(scores), R, N, _p(n_valid), _p(cand), K, _p(idx), _p(ws),
                         ws_bytes, _s(stream))
    return _check("csa2_topk", st, raise_on_error)


def csa2_sparse_attn(pool: csa2_pool, q, Q: int, H: int, idx, K: int, o, lse, ws,
                     ws_bytes: int, stream=None, raise_on_error=True) -> int:
    st = lib().csa2_sparse_attn(ctypes.byref(pool), _p(q), Q, H, _p(idx), K, _p(o), _p(lse),
                                _p(ws), ws_bytes, _s(stream))
    return _check("csa2_sparse_attn", st, raise_on_error)


def csa2_pool_append(latent, scale, idx_key, B: int, M: int, x_latent, x_key, slot, T: int,
                     stream=None, raise_on_error=True, pages=None, page_log2: int = 0) -> int:
    st = lib().csa2_pool_append(_p(latent), _p(scale), _p(idx_key), B, M, _p(x_latent),
                                _p(x_key), _p(slot), T, _p(pages),
                                page_log2 if pages is not None else 0, _s(stream))
    return _check("csa2_pool_append", st, raise_on_error)


def csa2_swa_append(swa, B: int, W: int, x, pos0: int, T: int, stream=None,
                    raise_on_error=True) -> int:
    st = lib().csa2_swa_append(_p(swa), B, W, _p(x), pos0, T, _s(stream))
    return _check("csa2_swa_append", st, raise_on_error)


def csa2_swa_merge(q, B: int, Q: int, H: int, D: int, swa, W: int, o, lse, ws,
                   ws_bytes: int, stream=None, raise_on_error=True) -> int:
    st = lib().csa2_swa_merge(_p(q), B, Q, H, D, _p(swa), W, _p(o), _p(lse), _p(ws),
                              ws_bytes, _s(stream))
    return _check("csa2_swa_merge", st, raise_on_error)


def csa2_score_topk(pool: csa2_pool, q_idx, w_idx, K: int, idx, ws, ws_bytes: int, stream=None,
                    raise_on_error=True) -> int:
    st = lib().csa2_score_topk(ctypes.byref(pool), _p(q_idx), _p(w_idx), K, _p(idx), _p(ws),
                               ws_bytes, _s(stream))
    return _check("csa2_score_topk", st, raise_on_error)


def csa2_decode_layers(pool: csa2_pool, layers, H: int, K: int, P: int, W: int, ws,
                       ws_bytes: int, stream=None, raise_on_error=True):
    """layers: sequence of csa2_layer.  Returns (status, src_layer list)."""
    L = len(layers)
    arr = (csa2_layer * L)(*layers)
    src = (c_int32 * L)()
    st = lib().csa2_decode_layers(ctypes.byref(pool), arr, L, H, K, P, W, src, _p(ws),
                                  ws_bytes, _s(stream))
    _check("csa2_decode_layers", st, raise_on_error)
    return st, list(src)


def csa2_decode_layers_noalloc(pool: csa2_pool, layers, H: int, K: int, P: int, W: int,
                               stream=None, raise_on_error=True):
    """csa2_decode_layers in the library's static scratch (no workspace
    argument, no device allocation).  Returns (status, src_layer list)."""
    L = len(layers)
    arr = (csa2_layer * L)(*layers)
    src = (c_int32 * L)()
    st = lib().csa2_decode_layers_noalloc(ctypes.byref(pool), arr, L, H, K, P, W, src,
                                          _s(stream))
    _check("csa2_decode_layers_noalloc", st, raise_on_error)
    return st, list(src)


def csa2_decode_layer(pool: csa2_pool, layers, l: int, H: int, K: int, P: int, W: int, ws,
                      ws_bytes: int, stream=None, raise_on_error=True):
    """Layer l of the schedule `layers` (a sequence of csa2_layer, or a ctypes
    array of them).  Returns (status, source layer of l)."""
    if not isinstance(layers, ctypes.Array):
        layers = (csa2_layer * len(layers))(*layers)
    src = c_int32(-1)
    st = lib().csa2_decode_layer(ctypes.byref(pool), layers, len(layers), l, H, K, P, W,
                                 ctypes.byref(src), _p(ws), ws_bytes, _s(stream))
    _check("csa2_decode_layer", st, raise_on_error)
    return st, src.value


def csa2_prefill_layers(pool: csa2_pool, layers, Q: int, pos0: int, ratio: int, H: int, K: int,
                        W: int, ws, ws_bytes: int, stream=None, raise_on_error=True):
    """layers: sequence of csa2_layer (per-chunk shapes).  Returns (status, src_layer list)."""
    L = len(layers)
    arr = (csa2_layer * L)(*layers)
    src = (c_int32 * L)()
    st = lib().csa2_prefill_layers(ctypes.byref(pool), arr, L, Q, pos0, ratio, H, K, W, src,
                                   _p(ws), ws_bytes, _s(stream))
    _check("csa2_prefill_layers", st, raise_on_error)
    return st, list(src)


def csa2_pool_restore(latent, scale, idx_key, B: int, M: int, seq: int, entry0: int, n: int,
                      h_latent, h_scale, h_key, stream=None, raise_on_error=True) -> int:
    st = lib().csa2_pool_restore(_p(latent), _p(scale), _p(idx_key), B, M, seq, entry0, n,
                                 _p(h_latent), _p(h_scale), _p(h_key), _s(stream))
    return _check("csa2_pool_restore", st, raise_on_error)


def csa2_pool_offload(latent, scale, idx_key, B: int, M: int, seq: int, entry0: int, n: int,
                      h_latent, h_scale, h_key, stream=None, raise_on_error=True) -> int:
    st = lib().csa2_pool_offload(_p(latent), _p(scale), _p(idx_key), B, M, seq, entry0, n,
                                 _p(h_latent), _p(h_scale), _p(h_key), _s(stream))
    return _check("csa2_pool_offload", st, raise_on_error)


def csa2_swa_restore(swa, B: int, W: int, seq: int, h_swa, stream=None, raise_on_error=True) -> int:
    st = lib().csa2_swa_restore(_p(swa), B, W, seq, _p(h_swa), _s(stream))
    return _check("csa2_swa_restore", st, raise_on_error)


def csa2_swa_offload(swa, B: int, W: int, seq: int, h_swa, stream=None, raise_on_error=True) -> int:
    st = lib().csa2_swa_offload(_p(swa), B, W, seq, _p(h_swa), _s(stream))
    return _check("csa2_swa_offload", st, raise_on_error)
