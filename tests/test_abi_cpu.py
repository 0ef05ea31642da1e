"""Host-side checks of libbinv that need no GPU: the library loads, exports
every entry point the header declares, and rejects bad arguments with the
documented status codes before launching anything."""
import ctypes
import os
import re

import pytest

import invariant_deterministic_fixed_amd as binv
from invariant_deterministic_fixed_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "binv.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, SCRATCH = 0, 1, 2, 3, 5


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(binv_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ["binv_gemm_bf16", "binv_rmsnorm", "binv_attn_decode_paged", "binv_attn_prefill_paged"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(binding.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings_and_version():
    assert binv.status_str(0) == "BINV_OK"
    assert "WORKSPACE" in binv.status_str(3)
    assert "unknown" in binv.status_str(99)
    assert "gfx950" in binv.version()


L = None  # null pointer
FAKE = 1 << 20   # a 16-byte aligned non-null address; never dereferenced by these calls


def _lib():
    return binding.lib()


def test_rmsnorm_validation():
    f = _lib().binv_rmsnorm
    assert f(L, 1, 8, L, 1, L, 1, 8, 0, 8, 1e-6, L) == OK                 # M = 0: no-op
    assert f(L, 1, 8, L, 1, L, 1, 8, 4, 8, 1e-6, L) == INVALID            # null pointers
    assert f(FAKE, 1, 8, FAKE, 1, FAKE, 1, 8, -1, 8, 1e-6, L) == INVALID  # negative M
    assert f(FAKE, 1, 12, FAKE, 1, FAKE, 1, 8, 4, 8, 1e-6, L) == INVALID  # ldx not 16B multiple
    assert f(FAKE + 2, 1, 8, FAKE, 1, FAKE, 1, 8, 4, 8, 1e-6, L) == INVALID  # misaligned x
    assert f(FAKE, 1, 16, FAKE, 1, FAKE, 1, 16, 4, 12, 1e-6, L) == UNSUPPORTED  # d % 8
    assert f(FAKE, 1, 32768, FAKE, 1, FAKE, 1, 32768, 4, 32768, 1e-6, L) == UNSUPPORTED
    assert f(FAKE, 7, 8, FAKE, 1, FAKE, 1, 8, 4, 8, 1e-6, L) == INVALID   # bad dtype
    assert f(FAKE, 1, 8, FAKE, 1, FAKE, 1, 8, 4, 8, -1.0, L) == INVALID   # negative eps


def test_gemm_validation():
    f = _lib().binv_gemm_bf16
    assert f(L, 8, L, 8, L, 1, 8, 0, 8, 8, L) == OK                      # M = 0
    assert f(L, 8, L, 8, L, 1, 8, 8, 0, 8, L) == OK                      # N = 0
    assert f(L, 8, L, 8, L, 1, 8, 8, 8, 8, L) == INVALID                 # nulls
    assert f(FAKE, 8, FAKE, 8, FAKE, 1, 8, 8, 8, -8, L) == INVALID       # negative K
    assert f(FAKE, 8, FAKE, 8, FAKE, 1, 8, 8, 8, 12, L) == INVALID       # lda < K
    assert f(FAKE, 16, FAKE, 16, FAKE, 1, 16, 8, 12, 16, L) == UNSUPPORTED  # N % 8
    assert f(FAKE, 16, FAKE, 16, FAKE, 1, 16, 8, 16, 12, L) == UNSUPPORTED  # K % 8
    assert f(FAKE, 9, FAKE, 8, FAKE, 1, 8, 8, 8, 8, L) == INVALID        # lda not 16B multiple
    g = _lib().binv_gemm_bf16_tuned
    need = _lib().binv_gemm_bf16_tuned_workspace_bytes(1, 4096, 4096)
    assert need > 0
    assert g(FAKE, 4096, FAKE, 4096, FAKE, 1, 4096, 1, 4096, 4096, L, 0, L) == WORKSPACE


def test_gemm_packed_validation_and_size():
    size = _lib().binv_gemm_bf16_packed_bytes
    # ceil(N / 16) strips x 2 ceil(K / 64) k-blocks x 1 KB
    assert size(4096, 4096) == 256 * 128 * 1024
    assert size(200, 72) == 13 * 4 * 1024
    assert size(8, 0) == 0 and size(-1, 8) == 0
    pack = _lib().binv_gemm_bf16_pack
    assert pack(L, 8, 0, 8, L, L) == OK                                   # K = 0
    assert pack(L, 8, 8, 8, L, L) == INVALID                              # nulls
    assert pack(FAKE, 8, 8, 16, FAKE, L) == INVALID                       # ldw < N
    assert pack(FAKE, 16, 12, 16, FAKE, L) == UNSUPPORTED                 # K % 8
    assert pack(FAKE + 2, 8, 8, 8, FAKE, L) == INVALID                    # misaligned W
    f = _lib().binv_gemm_bf16_packed
    assert f(L, 8, L, L, 1, 8, 0, 8, 8, L) == OK                          # M = 0
    assert f(L, 8, L, L, 1, 8, 4, 8, 8, L) == INVALID                     # nulls
    assert f(FAKE, 4096, FAKE, FAKE, 1, 4096, 65, 4096, 4096, L) == UNSUPPORTED   # M > 64
    assert f(FAKE, 16, FAKE, FAKE, 1, 16, 4, 12, 16, L) == UNSUPPORTED    # N % 8
    assert f(FAKE, 8, FAKE, FAKE, 1, 8, 4, 8, 12, L) == INVALID           # lda < K
    assert f(FAKE, 8, FAKE + 8, FAKE, 1, 8, 4, 8, 8, L) == INVALID        # misaligned Wp


def _dec(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, pt=FAKE, pts=4, kl=FAKE, out=FAKE, B=2, maxl=64, Hq=8,
             Hkv=2, D=128, page=16, scale=0.1, ws=FAKE, wsb=1 << 30, s=L)
    a.update(over)
    return _lib().binv_attn_decode_paged(a["q"], a["k"], a["v"], a["pt"], a["pts"], a["kl"],
                                         a["out"], a["B"], a["maxl"], a["Hq"], a["Hkv"], a["D"],
                                         a["page"], a["scale"], a["ws"], a["wsb"], a["s"])


def test_attention_decode_validation():
    assert _dec(B=0) == OK
    assert _dec(q=L) == INVALID
    assert _dec(Hq=6, Hkv=4) == INVALID
    assert _dec(Hq=6, Hkv=2) == UNSUPPORTED            # group of 3
    assert _dec(D=96) == UNSUPPORTED
    assert _dec(page=32) == UNSUPPORTED
    assert _dec(maxl=0) == INVALID
    assert _dec(maxl=256 * 512 + 1) == UNSUPPORTED
    assert _dec(wsb=16) == WORKSPACE
    assert _dec(ws=L) == WORKSPACE
    assert _dec(scale=float("nan")) == INVALID
    assert _dec(B=70000) == UNSUPPORTED


def _dec_noalloc(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, pt=FAKE, pts=4, kl=FAKE, out=FAKE, B=2, maxl=64, Hq=8,
             Hkv=2, D=128, page=16, scale=0.1, s=L)
    a.update(over)
    return _lib().binv_attn_decode_paged_noalloc(a["q"], a["k"], a["v"], a["pt"], a["pts"],
                                                 a["kl"], a["out"], a["B"], a["maxl"], a["Hq"],
                                                 a["Hkv"], a["D"], a["page"], a["scale"], a["s"])


def test_attention_decode_noalloc_validation():
    # argument checks and the scratch limit are decided on the host, before the
    # entry point looks up its device array or launches anything
    assert _dec_noalloc(B=0) == OK
    assert _dec_noalloc(q=L) == INVALID
    assert _dec_noalloc(out=FAKE + 8) == INVALID
    assert _dec_noalloc(Hq=6, Hkv=2) == UNSUPPORTED
    assert _dec_noalloc(maxl=256 * 512 + 1) == UNSUPPORTED
    assert "SCRATCH" in binv.status_str(SCRATCH)
    limit = 128 << 20                                   # BINV_NOALLOC_SCRATCH_BYTES
    per_b_chunk = 32 * (128 + 2) * 4                    # Hq = 32, D = 128
    fits = limit // per_b_chunk                         # 8065 (sequence, chunk) slots
    assert binv.attn_workspace_bytes(fits, 32, 128, 256) <= limit
    assert binv.attn_workspace_bytes(fits + 1, 32, 128, 256) > limit
    assert _dec_noalloc(B=fits + 1, maxl=256, Hq=32, Hkv=8) == SCRATCH
    assert _dec_noalloc(B=64, maxl=32768, Hq=32, Hkv=8) == SCRATCH
    assert _dec_noalloc(B=32, maxl=65536, Hq=32, Hkv=8) == SCRATCH


def test_attention_prefill_validation():
    f = _lib().binv_attn_prefill_paged
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, FAKE, 1, 10, 10, 64, 8, 2, 128, 16, 0.1,
            FAKE, 1 << 30, L]
    assert f(*args[:8], 0, *args[9:]) == OK                       # B = 0
    assert f(*args[:9], 0, *args[10:]) == OK                      # T = 0
    bad = list(args); bad[1] = L
    assert f(*bad) == INVALID                                     # null cu_q
    bad = list(args); bad[10] = 100
    assert f(*bad) == INVALID                                     # max_q_len > max_kv_len
    bad = list(args); bad[18] = 8
    assert f(*bad) == WORKSPACE


def test_workspace_sizes():
    ws = binv.attn_workspace_bytes(256, 32, 128, 32768)
    assert ws == 256 * 32 * 128 * (128 + 2) * 4
    assert binv.attn_workspace_bytes(0, 32, 128, 100) == 0


def test_prefill_workspace_sizes():
    f = binv.attn_prefill_workspace_bytes
    node = 32 * (128 + 2) * 4                      # one partial of every head of a token
    # one long sequence: the pending subtrees above the two the kernel keeps in
    # registers only, max(1, floor(log2(chunks)) - 1) per row
    assert f(1, 4096, 4096, 4096, 32, 8, 128) == 4096 * 3 * node
    assert f(1, 4096, 4096, 32768, 32, 8, 128) == 4096 * 6 * node
    assert f(1, 64, 64, 256, 32, 8, 128) == 64 * 1 * node
    assert f(1, 2048, 2048, 4096, 32, 8, 128) == 2048 * 3 * node
    # one sequence whose 128-row blocks (x KV heads) number fewer than the 256
    # CUs, over at most 64 chunks: a node per aligned pair of chunks and token
    assert f(1, 64, 64, 1024, 32, 8, 128) == 64 * 2 * node
    assert f(1, 512, 512, 4096, 32, 8, 128) == 512 * 8 * node
    assert f(1, 256, 256, 16384, 32, 8, 128) == 256 * 32 * node
    # ... and over more than 64 chunks the looping kernel's stacks again
    assert f(1, 512, 512, 32768, 32, 8, 128) == 512 * 6 * node
    # four long sequences: stacks per token plus leaves for at most 15 short
    # tokens per sequence (the block kernel takes runs of 16 or more at G = 4)
    assert f(4, 4096, 1024, 4096, 32, 8, 128) == (4096 * 3 + 4 * 15 * 16) * node
    # one prompt chunk among decode rows: leaves per token are smaller
    T = 512 + 63
    assert f(64, T, 512, 1024, 32, 8, 128) == binv.attn_workspace_bytes(T, 32, 128, 1024)
    # short runs only, and D = 64: one leaf per row and chunk
    assert f(8, 8, 1, 4096, 32, 8, 128) == binv.attn_workspace_bytes(8, 32, 128, 4096)
    assert f(1, 4096, 4096, 4096, 8, 8, 64) == binv.attn_workspace_bytes(4096, 8, 64, 4096)
    # never more than one partial per row and chunk
    for B in (1, 2, 7, 64):
        for T in (B, 3 * B, 100, 4096):
            if T < B:
                continue
            for mq in sorted({1, 15, 16, 64, T - B + 1}):
                for kv in (256, 1000, 4096, 131072):
                    if mq > kv:
                        continue
                    for (hq, hkv) in ((32, 8), (32, 32), (16, 1)):
                        assert 0 < f(B, T, mq, kv, hq, hkv, 128) <= \
                            binv.attn_workspace_bytes(T, hq, 128, kv)
    # rejected arguments
    assert f(0, 16, 16, 256, 32, 8, 128) == 0
    assert f(1, 16, 16, 256, 32, 7, 128) == 0


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", "/nonexistent/libbinv.so")
    with pytest.raises(RuntimeError, match="no fallback"):
        binding.lib()


def test_embed_validation():
    f = _lib().binv_embed
    assert f(L, 0, L, 10, 8, L, L) == OK                                    # T = 0: no-op
    assert f(FAKE, -1, FAKE, 10, 8, FAKE, L) == INVALID                     # negative T
    assert f(FAKE, 4, FAKE, 0, 8, FAKE, L) == INVALID                       # empty table
    assert f(L, 4, FAKE, 10, 8, FAKE, L) == INVALID                         # null ids
    assert f(FAKE, 4, FAKE + 8, 10, 8, FAKE, L) == INVALID                  # misaligned table
    assert f(FAKE, 4, FAKE, 10, 12, FAKE, L) == UNSUPPORTED                 # H % 8


def test_rope_kv_write_validation():
    f = _lib().binv_rope_kv_write
    args = lambda **k: [k.get("qkv", FAKE), k.get("ld", 48 * 128), FAKE, FAKE, k.get("T", 4),
                        k.get("Hq", 32), k.get("Hkv", 8), k.get("D", 128), k.get("theta", 5e5),
                        FAKE, FAKE, FAKE, FAKE, k.get("pts", 64), k.get("page", 16), L]
    assert f(*args(T=0)) == OK
    assert f(*args(T=-1)) == INVALID
    assert f(*args(qkv=L)) == INVALID
    assert f(*args(Hkv=0)) == INVALID
    assert f(*args(theta=1.0)) == INVALID                                   # theta must exceed 1
    assert f(*args(theta=float("inf"))) == INVALID
    assert f(*args(pts=0)) == INVALID
    assert f(*args(D=96)) == UNSUPPORTED
    assert f(*args(page=32)) == UNSUPPORTED
    assert f(*args(ld=48 * 128 - 8)) == INVALID                             # row shorter than q|k|v


def test_swiglu_validation():
    f = _lib().binv_swiglu
    assert f(L, 16, 0, 8, L, 8, L) == OK                                    # T = 0
    assert f(FAKE, 16, 4, 0, FAKE, 8, L) == OK                              # F = 0
    assert f(FAKE, 16, -1, 8, FAKE, 8, L) == INVALID
    assert f(FAKE, 8, 4, 8, FAKE, 8, L) == INVALID                          # ld_gu < 2F
    assert f(FAKE, 16, 4, 8, FAKE, 4, L) == INVALID                         # ld_out < F
    assert f(FAKE + 8, 16, 4, 8, FAKE, 8, L) == INVALID                     # misaligned
    assert f(FAKE, 24, 4, 12, FAKE, 16, L) == UNSUPPORTED                   # F % 8
    assert f(FAKE, 16, 70000, 8, FAKE, 8, L) == UNSUPPORTED                 # T > 65535


def test_residual_add_validation():
    f = _lib().binv_residual_add
    assert f(L, 8, L, 8, 0, 8, L) == OK
    assert f(FAKE, 8, FAKE, 8, -2, 8, L) == INVALID
    assert f(FAKE, 4, FAKE, 8, 2, 8, L) == INVALID                          # ldh < H
    assert f(FAKE + 4, 8, FAKE, 8, 2, 8, L) == INVALID                      # h not 16B aligned
    assert f(FAKE, 8, FAKE + 2, 8, 2, 8, L) == INVALID                      # x not 8B aligned
    assert f(FAKE, 8, FAKE, 8, 2, 6, L) == UNSUPPORTED                      # H % 4


def test_add_rmsnorm_validation():
    f = _lib().binv_add_rmsnorm
    assert f(L, 8, L, 8, L, 1, L, 1, 8, 0, 8, 1e-6, L) == OK                # M = 0: no-op
    assert f(FAKE, 8, L, 8, FAKE, 1, FAKE, 1, 8, 2, 8, 1e-6, L) == INVALID  # null a
    assert f(FAKE, 8, FAKE + 2, 8, FAKE, 1, FAKE, 1, 8, 2, 8, 1e-6, L) == INVALID  # a not 8B aligned
    assert f(FAKE, 8, FAKE, 6, FAKE, 1, FAKE, 1, 8, 2, 8, 1e-6, L) == INVALID  # lda % 4
    assert f(FAKE, 8, FAKE, 4, FAKE, 1, FAKE, 1, 8, 2, 8, 1e-6, L) == INVALID  # lda < d
    assert f(FAKE + 4, 8, FAKE, 8, FAKE, 1, FAKE, 1, 8, 2, 8, 1e-6, L) == INVALID  # h misaligned
    assert f(FAKE, 8, FAKE, 8, FAKE, 1, FAKE, 1, 8, 2, 8, -1.0, L) == INVALID  # negative eps
    assert f(FAKE, 8, FAKE, 8, FAKE, 7, FAKE, 1, 8, 2, 8, 1e-6, L) == INVALID  # bad dtype
    assert f(FAKE, 8, FAKE, 8, FAKE, 1, FAKE, 1, 8, 2, 6, 1e-6, L) == UNSUPPORTED  # d % 4
    assert f(FAKE, 16384, FAKE, 16384, FAKE, 1, FAKE, 1, 16384, 2, 16384, 1e-6,
             L) == UNSUPPORTED                                              # fp32 rows <= 8192


def test_gather_rows_validation():
    f = _lib().binv_gather_rows
    assert f(L, 1, 8, L, 0, L, 8, 8, L) == OK                               # R = 0
    assert f(FAKE, 7, 8, FAKE, 2, FAKE, 8, 8, L) == INVALID                 # unknown dtype
    assert f(FAKE, 1, 8, L, 2, FAKE, 8, 8, L) == INVALID                    # null idx
    assert f(FAKE, 1, 4, FAKE, 2, FAKE, 8, 8, L) == INVALID                 # lds < cols
    assert f(FAKE, 1, 8, FAKE, 2, FAKE, 8, 3, L) == INVALID                 # 6-byte rows


def test_topk_validation():
    f = _lib().binv_topk
    assert f(L, 16, 0, 16, 20, L, L, L) == OK                               # R = 0
    assert f(FAKE, 16, 2, 16, 0, FAKE, FAKE, L) == INVALID                  # K < 1
    assert f(FAKE, 16, 2, 16, 33, FAKE, FAKE, L) == UNSUPPORTED             # K > 32
    assert f(FAKE, 8, 2, 16, 4, FAKE, FAKE, L) == INVALID                   # ldx < n
    assert f(FAKE, 16, 2, 16, 4, L, FAKE, L) == INVALID                     # null ids
    assert f(FAKE, 16, -1, 16, 4, FAKE, FAKE, L) == INVALID


def test_split_bf16x3_validation():
    f = _lib().binv_split_bf16x3
    assert f(L, 8, 0, 8, L, 24, L) == OK                                    # M = 0
    assert f(L, 8, 2, 8, FAKE, 24, L) == INVALID                            # null x
    assert f(FAKE, 8, 2, 8, FAKE, 16, L) == INVALID                         # ld_out < 3K
    assert f(FAKE + 4, 8, 2, 8, FAKE, 24, L) == INVALID                     # misaligned x
    assert f(FAKE, 8, 2, 6, FAKE, 24, L) == UNSUPPORTED                     # K % 4
    assert f(FAKE, 8, -1, 8, FAKE, 24, L) == INVALID
