"""Thin ctypes binding of libbinv.so (argument marshalling only).

Every function takes torch tensors for device memory, passes their data
pointers, sizes and the current HIP stream to the C entry point of the same
name in include/binv.h, and raises BinvError on a non-zero status.  No
computation happens here.  If libbinv.so is missing the first call raises:
there is no fallback path.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbinv.so")

BINV_F32 = 0
BINV_BF16 = 1
CHUNK = 256
MAX_KV_LEN = 256 * 512
PAGE_SIZE = 16

_lib = None


class BinvError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status})")


def _declare(lib):
    vp, i64, i32, f32, sz, ci = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                 ctypes.c_float, ctypes.c_size_t, ctypes.c_int)
    sig = {
        "binv_status_str": (ctypes.c_char_p, [ci]),
        "binv_version": (ctypes.c_char_p, []),
        "binv_rmsnorm": (ci, [vp, ci, i64, vp, ci, vp, ci, i64, i64, i64, f32, vp]),
        "binv_rmsnorm_tuned": (ci, [vp, ci, i64, vp, ci, vp, ci, i64, i64, i64, f32, vp]),
        "binv_gemm_bf16": (ci, [vp, i64, vp, i64, vp, ci, i64, i64, i64, i64, vp]),
        "binv_gemm_bf16_tuned_workspace_bytes": (sz, [i64, i64, i64]),
        "binv_gemm_bf16_tuned": (ci, [vp, i64, vp, i64, vp, ci, i64, i64, i64, i64, vp, sz, vp]),
        "binv_attn_workspace_bytes": (sz, [i64, ci, ci, i64]),
        "binv_attn_decode_paged": (ci, [vp, vp, vp, vp, i64, vp, vp, i64, i64, ci, ci, ci, ci,
                                        f32, vp, sz, vp]),
        "binv_attn_prefill_paged": (ci, [vp, vp, vp, vp, vp, i64, vp, vp, i64, i64, i64, i64,
                                         ci, ci, ci, ci, f32, vp, sz, vp]),
        "binv_attn_decode_tuned_workspace_bytes": (sz, [i64, ci, ci, i64]),
        "binv_attn_decode_paged_tuned": (ci, [vp, vp, vp, vp, i64, vp, vp, i64, i64, ci, ci, ci,
                                              ci, f32, vp, sz, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def lib():
    """The loaded libbinv.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(there is no fallback implementation)")
        _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def status_str(status):
    return lib().binv_status_str(int(status)).decode()


def version():
    return lib().binv_version().decode()


def _check(status, where):
    if status != 0:
        raise BinvError(status, where)


def _dt(t):
    if t.dtype == torch.bfloat16:
        return BINV_BF16
    if t.dtype == torch.float32:
        return BINV_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _rows(t):
    """(rows, leading dimension) of a 2-D tensor whose rows are contiguous."""
    assert t.dim() == 2 and t.stride(1) == 1, "expected a 2-D tensor with contiguous rows"
    return t.shape[0], t.stride(0)


def _dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libbinv takes device (cuda/hip) tensors")


def _workspace(nbytes, device, workspace):
    if workspace is not None:
        return workspace, workspace.numel() * workspace.element_size()
    ws = torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)
    return ws, ws.numel()


# ---------------------------------------------------------------- RMSNorm
def rmsnorm(x, gamma, eps=1e-6, out=None, out_dtype=torch.bfloat16, tuned=False):
    _dev(x, gamma, out)
    M, ldx = _rows(x)
    d = x.shape[1]
    if out is None:
        out = torch.empty((M, d), dtype=out_dtype, device=x.device)
    _, ldy = _rows(out)
    fn = lib().binv_rmsnorm_tuned if tuned else lib().binv_rmsnorm
    _check(fn(_ptr(x), _dt(x), ldx, _ptr(gamma), _dt(gamma), _ptr(out), _dt(out), ldy, M, d,
              float(eps), _stream(x)), fn.__name__)
    return out


# ---------------------------------------------------------------- GEMM
def gemm(a, w, out=None, out_dtype=torch.bfloat16, tuned=False, workspace=None):
    _dev(a, w, out)
    M, lda = _rows(a)
    K, ldw = _rows(w)
    N = w.shape[1]
    assert a.shape[1] == K and a.dtype == torch.bfloat16 and w.dtype == torch.bfloat16
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    _, ldc = _rows(out)
    if tuned:
        need = lib().binv_gemm_bf16_tuned_workspace_bytes(M, N, K)
        ws, nbytes = _workspace(need, a.device, workspace)
        st = lib().binv_gemm_bf16_tuned(_ptr(a), lda, _ptr(w), ldw, _ptr(out), _dt(out), ldc, M,
                                        N, K, _ptr(ws), nbytes, _stream(a))
        _check(st, "binv_gemm_bf16_tuned")
    else:
        _check(lib().binv_gemm_bf16(_ptr(a), lda, _ptr(w), ldw, _ptr(out), _dt(out), ldc, M, N,
                                    K, _stream(a)), "binv_gemm_bf16")
    return out


# ---------------------------------------------------------------- attention
def attn_workspace_bytes(n_query_tokens, Hq, D, max_kv_len):
    return lib().binv_attn_workspace_bytes(n_query_tokens, Hq, D, max_kv_len)


def attn_decode(q, k_cache, v_cache, page_table, kv_lens, max_kv_len, scale, out=None,
                workspace=None, tuned=False):
    """q [B, Hq, D] bf16; caches as laid out in include/binv.h."""
    _dev(q, k_cache, v_cache, page_table, kv_lens, out)
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    page = k_cache.shape[2]
    assert q.is_contiguous() and k_cache.is_contiguous() and v_cache.is_contiguous()
    assert page_table.dtype == torch.int32 and kv_lens.dtype == torch.int32
    assert page_table.dim() == 2 and page_table.stride(1) == 1
    if out is None:
        out = torch.empty_like(q)
    if tuned:
        need = lib().binv_attn_decode_tuned_workspace_bytes(B, Hq, D, max_kv_len)
        fn = lib().binv_attn_decode_paged_tuned
    else:
        need = lib().binv_attn_workspace_bytes(B, Hq, D, max_kv_len)
        fn = lib().binv_attn_decode_paged
    ws, nbytes = _workspace(need, q.device, workspace)
    st = fn(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table), page_table.stride(0),
            _ptr(kv_lens), _ptr(out), B, int(max_kv_len), Hq, Hkv, D, page, float(scale),
            _ptr(ws), nbytes, _stream(q))
    _check(st, fn.__name__)
    return out


def attn_prefill(q, cu_q, k_cache, v_cache, page_table, kv_lens, max_q_len, max_kv_len, scale,
                 out=None, workspace=None):
    """q [T, Hq, D] bf16 (new tokens of all sequences); cu_q int32 [B+1]."""
    _dev(q, cu_q, k_cache, v_cache, page_table, kv_lens, out)
    T, Hq, D = q.shape
    B = cu_q.shape[0] - 1
    Hkv = k_cache.shape[1]
    page = k_cache.shape[2]
    assert q.is_contiguous() and cu_q.dtype == torch.int32
    if out is None:
        out = torch.empty_like(q)
    need = lib().binv_attn_workspace_bytes(T, Hq, D, max_kv_len)
    ws, nbytes = _workspace(need, q.device, workspace)
    st = lib().binv_attn_prefill_paged(_ptr(q), _ptr(cu_q), _ptr(k_cache), _ptr(v_cache),
                                       _ptr(page_table), page_table.stride(0), _ptr(kv_lens),
                                       _ptr(out), B, T, int(max_q_len), int(max_kv_len), Hq, Hkv,
                                       D, page, float(scale), _ptr(ws), nbytes, _stream(q))
    _check(st, "binv_attn_prefill_paged")
    return out
