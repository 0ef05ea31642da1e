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
        "binv_add_rmsnorm": (ci, [vp, i64, vp, i64, vp, ci, vp, ci, i64, i64, i64, f32, vp]),
        "binv_gemm_bf16": (ci, [vp, i64, vp, i64, vp, ci, i64, i64, i64, i64, vp]),
        "binv_gemm_bf16_tuned_workspace_bytes": (sz, [i64, i64, i64]),
        "binv_gemm_bf16_packed_bytes": (sz, [i64, i64]),
        "binv_gemm_bf16_pack": (ci, [vp, i64, i64, i64, vp, vp]),
        "binv_gemm_bf16_packed": (ci, [vp, i64, vp, vp, ci, i64, i64, i64, i64, vp]),
        "binv_gemm_bf16_tuned": (ci, [vp, i64, vp, i64, vp, ci, i64, i64, i64, i64, vp, sz, vp]),
        "binv_attn_workspace_bytes": (sz, [i64, ci, ci, i64]),
        "binv_attn_prefill_workspace_bytes": (sz, [i64, i64, i64, i64, ci, ci, ci]),
        "binv_attn_decode_paged": (ci, [vp, vp, vp, vp, i64, vp, vp, i64, i64, ci, ci, ci, ci,
                                        f32, vp, sz, vp]),
        "binv_attn_prefill_paged": (ci, [vp, vp, vp, vp, vp, i64, vp, vp, i64, i64, i64, i64,
                                         ci, ci, ci, ci, f32, vp, sz, vp]),
        "binv_attn_decode_paged_noalloc": (ci, [vp, vp, vp, vp, i64, vp, vp, i64, i64, ci, ci,
                                                ci, ci, f32, vp]),
        "binv_attn_decode_tuned_workspace_bytes": (sz, [i64, ci, ci, i64]),
        "binv_attn_decode_paged_tuned": (ci, [vp, vp, vp, vp, i64, vp, vp, i64, i64, ci, ci, ci,
                                              ci, f32, vp, sz, vp]),
        "binv_embed": (ci, [vp, i64, vp, i64, i64, vp, vp]),
        "binv_rope_kv_write": (ci, [vp, i64, vp, vp, i64, ci, ci, ci, ctypes.c_double, vp, vp, vp,
                                    vp, i64, ci, vp]),
        "binv_swiglu": (ci, [vp, i64, i64, i64, vp, i64, vp]),
        "binv_residual_add": (ci, [vp, i64, vp, i64, i64, i64, vp]),
        "binv_gather_rows": (ci, [vp, ci, i64, vp, i64, vp, i64, i64, vp]),
        "binv_topk": (ci, [vp, i64, i64, i64, ci, vp, vp, vp]),
        "binv_split_bf16x3": (ci, [vp, i64, i64, i64, vp, i64, vp]),
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


def add_rmsnorm(h, a, gamma, eps=1e-6, out=None, out_dtype=torch.bfloat16):
    """h += a (h fp32 [M, d] in place, a bf16), then rmsnorm of the updated h:
    the bits of residual_add(h, a) followed by rmsnorm(h, ...)."""
    _dev(h, a, gamma, out)
    M, ldh = _rows(h)
    _, lda = _rows(a)
    d = h.shape[1]
    assert h.dtype == torch.float32 and a.dtype == torch.bfloat16 and tuple(a.shape) == (M, d)
    if out is None:
        out = torch.empty((M, d), dtype=out_dtype, device=h.device)
    _, ldy = _rows(out)
    _check(lib().binv_add_rmsnorm(_ptr(h), ldh, _ptr(a), lda, _ptr(gamma), _dt(gamma), _ptr(out),
                                  _dt(out), ldy, M, d, float(eps), _stream(h)), "binv_add_rmsnorm")
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


class PackedWeight:
    """W [K, N] bf16 re-laid out per 16-column strip (binv_gemm_bf16_pack),
    for gemm_packed; data is a flat device tensor of
    binv_gemm_bf16_packed_bytes(N, K) bytes."""

    def __init__(self, data, K, N):
        self.data, self.K, self.N = data, K, N


def gemm_pack(w):
    _dev(w)
    K, ldw = _rows(w)
    N = w.shape[1]
    assert w.dtype == torch.bfloat16
    data = torch.empty(lib().binv_gemm_bf16_packed_bytes(N, K), dtype=torch.uint8,
                       device=w.device)
    _check(lib().binv_gemm_bf16_pack(_ptr(w), ldw, K, N, _ptr(data), _stream(w)),
           "binv_gemm_bf16_pack")
    return PackedWeight(data, K, N)


def gemm_packed(a, wp, out=None, out_dtype=torch.bfloat16):
    """a [M <= 64, K] bf16 times the packed weight wp: the bits of gemm(a, w)."""
    _dev(a, wp.data, out)
    M, lda = _rows(a)
    assert a.shape[1] == wp.K and a.dtype == torch.bfloat16
    if out is None:
        out = torch.empty((M, wp.N), dtype=out_dtype, device=a.device)
    _, ldc = _rows(out)
    _check(lib().binv_gemm_bf16_packed(_ptr(a), lda, _ptr(wp.data), _ptr(out), _dt(out), ldc, M,
                                       wp.N, wp.K, _stream(a)), "binv_gemm_bf16_packed")
    return out


# ---------------------------------------------------------------- attention
def attn_workspace_bytes(n_query_tokens, Hq, D, max_kv_len):
    return lib().binv_attn_workspace_bytes(n_query_tokens, Hq, D, max_kv_len)


def attn_prefill_workspace_bytes(B, T, max_q_len, max_kv_len, Hq, Hkv, D):
    return lib().binv_attn_prefill_workspace_bytes(B, T, max_q_len, max_kv_len, Hq, Hkv, D)


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


def attn_decode_noalloc(q, k_cache, v_cache, page_table, kv_lens, max_kv_len, scale, out):
    """binv_attn_decode_paged_noalloc: decode with the library's fixed partials
    buffer instead of a workspace; `out` [B, Hq, D] bf16 must be given (nothing
    is allocated on this path)."""
    _dev(q, k_cache, v_cache, page_table, kv_lens, out)
    B, Hq, D = q.shape
    assert q.is_contiguous() and k_cache.is_contiguous() and v_cache.is_contiguous()
    assert page_table.dtype == torch.int32 and kv_lens.dtype == torch.int32
    assert page_table.dim() == 2 and page_table.stride(1) == 1 and out.is_contiguous()
    st = lib().binv_attn_decode_paged_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table), page_table.stride(0),
        _ptr(kv_lens), _ptr(out), B, int(max_kv_len), Hq, k_cache.shape[1], D,
        k_cache.shape[2], float(scale), _stream(q))
    _check(st, "binv_attn_decode_paged_noalloc")
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
    need = lib().binv_attn_prefill_workspace_bytes(B, T, int(max_q_len), int(max_kv_len), Hq, Hkv,
                                                   D)
    ws, nbytes = _workspace(need, q.device, workspace)
    st = lib().binv_attn_prefill_paged(_ptr(q), _ptr(cu_q), _ptr(k_cache), _ptr(v_cache),
                                       _ptr(page_table), page_table.stride(0), _ptr(kv_lens),
                                       _ptr(out), B, T, int(max_q_len), int(max_kv_len), Hq, Hkv,
                                       D, page, float(scale), _ptr(ws), nbytes, _stream(q))
    _check(st, "binv_attn_prefill_paged")
    return out


# ---------------------------------------------------------------- decoder glue
def embed(ids, table, out=None):
    """out fp32 [T, H] = table[ids] (bf16 table [V, H])."""
    _dev(ids, table, out)
    T = ids.shape[0]
    V, H = table.shape
    assert ids.dtype == torch.int32 and table.dtype == torch.bfloat16 and table.is_contiguous()
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=table.device)
    assert out.is_contiguous()
    _check(lib().binv_embed(_ptr(ids), T, _ptr(table), V, H, _ptr(out), _stream(table)),
           "binv_embed")
    return out


def rope_kv_write(qkv, tok_seq, tok_pos, Hq, Hkv, D, theta, k_cache, v_cache, page_table,
                  q_out=None):
    """RoPE on the q/k heads of qkv [T, >= (Hq + 2 Hkv) D], rotated q -> q_out [T, Hq, D],
    k and v -> the paged caches at (tok_seq, tok_pos)."""
    _dev(qkv, tok_seq, tok_pos, k_cache, v_cache, page_table, q_out)
    T, ld = _rows(qkv)
    if q_out is None:
        q_out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=qkv.device)
    st = lib().binv_rope_kv_write(_ptr(qkv), ld, _ptr(tok_seq), _ptr(tok_pos), T, Hq, Hkv, D,
                                  float(theta), _ptr(q_out), _ptr(k_cache), _ptr(v_cache),
                                  _ptr(page_table), page_table.stride(0), k_cache.shape[2],
                                  _stream(qkv))
    _check(st, "binv_rope_kv_write")
    return q_out


def swiglu(gate_up, out=None):
    """out [T, F] = silu(gate_up[:, :F]) * gate_up[:, F:]."""
    _dev(gate_up, out)
    T, ld = _rows(gate_up)
    F = gate_up.shape[1] // 2
    if out is None:
        out = torch.empty((T, F), dtype=torch.bfloat16, device=gate_up.device)
    _, ldo = _rows(out)
    _check(lib().binv_swiglu(_ptr(gate_up), ld, T, F, _ptr(out), ldo, _stream(gate_up)),
           "binv_swiglu")
    return out


def residual_add(h, x):
    """h (fp32) += x (bf16), in place."""
    _dev(h, x)
    T, ldh = _rows(h)
    _, ldx = _rows(x)
    _check(lib().binv_residual_add(_ptr(h), ldh, _ptr(x), ldx, T, h.shape[1], _stream(h)),
           "binv_residual_add")
    return h


def gather_rows(src, idx, out=None):
    """out[r] = src[idx[r]] (bit copy)."""
    _dev(src, idx, out)
    _, lds = _rows(src)
    R = idx.shape[0]
    if out is None:
        out = torch.empty((R, src.shape[1]), dtype=src.dtype, device=src.device)
    _, ldd = _rows(out)
    _check(lib().binv_gather_rows(_ptr(src), _dt(src), lds, _ptr(idx), R, _ptr(out), ldd,
                                  src.shape[1], _stream(src)), "binv_gather_rows")
    return out


def split_bf16x3(x, out=None):
    """fp32 [M, K] -> bf16 [M, 3K] = [hi | mid | lo] with hi + mid + lo == x."""
    _dev(x, out)
    assert x.dtype == torch.float32
    M, ldx = _rows(x)
    K = x.shape[1]
    if out is None:
        out = torch.empty((M, 3 * K), dtype=torch.bfloat16, device=x.device)
    _, ldo = _rows(out)
    _check(lib().binv_split_bf16x3(_ptr(x), ldx, M, K, _ptr(out), ldo, _stream(x)),
           "binv_split_bf16x3")
    return out


def topk(x, K=20):
    """Exact top-K per fp32 row: (ids int32 [R, K], vals fp32 [R, K])."""
    _dev(x)
    R, ldx = _rows(x)
    ids = torch.empty((R, K), dtype=torch.int32, device=x.device)
    vals = torch.empty((R, K), dtype=torch.float32, device=x.device)
    _check(lib().binv_topk(_ptr(x), ldx, R, x.shape[1], K, _ptr(ids), _ptr(vals), _stream(x)),
           "binv_topk")
    return ids, vals
