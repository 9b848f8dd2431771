"""Host-side checks of the C ABI (no GPU needed).

The library loads on a machine without a GPU (only the HIP runtime library
is needed), exports every function the ``include/*.h`` headers declare, and rejects
invalid arguments with the documented status codes before touching HIP.
Every call here fails validation (or is an empty no-op), so no fake pointer
ever reaches a launch.
"""
import ctypes
import glob
import os
import re

import pytest

import long_context_attention_tiled_amd as lcat
from long_context_attention_tiled_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

OK, NULL, SHAPE, DTYPE, ALIGN, UNSUP, WS, HIP = range(8)
P = ctypes.c_void_p
A16 = P(0x10000)      # aligned, never dereferenced (every call below fails first)
MIS = P(0x10001)      # misaligned
NUL = P(0)
S0 = P(0)             # stream


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"^\s*(?:[a-z_0-9]+\s+)+\*?\s*([a-z_0-9]+)\s*\(", text, re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libattn.so not built")
    return lcat.load_library()


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["attn_prefill", "attn_chunked_prefill", "attn_decode", "attn_decode_workspace_bytes",
              "attn_kv_append", "rope_apply", "rope_apply_qk", "seq_to_head_permute",
              "seq_to_head_permute_qkv", "head_to_seq_permute", "seq_to_head_permute_qkv_rope", "cp_shard_tokens",
              "cp_shard", "cp_unshard", "attn_key_limits", "attn_prefill_limited", "attn_merge",
              "attn_decode_fp8", "attn_kv_quantize_fp8", "attn_kv_append_fp8",
              "attn_status_string", "attn_build_id", "attn_decode_noalloc", "attn_quantize_fp8_blocks",
              "attn_prefill_fp8", "attn_quantize_fp8_v", "attn_prefill_fp8_pv",
              "attn_measure_mfma_rate"]:
        assert n in names
    assert set(names) == set(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in range(8):
        s = lcat.attn_status_string(code)
        assert s and s != "unknown status"
    assert lcat.attn_status_string(99) == "unknown status"


def test_prefill_validation(lib):
    f = lib.attn_prefill
    # shape: Hq not a multiple of Hkv
    assert f(A16, A16, A16, A16, NUL, 1, 64, 3, 2, 128, 1, 1, 0.1, S0) == SHAPE
    assert f(A16, A16, A16, A16, NUL, -1, 64, 2, 2, 128, 1, 1, 0.1, S0) == SHAPE
    # dtype
    assert f(A16, A16, A16, A16, NUL, 1, 64, 2, 2, 128, 7, 1, 0.1, S0) == DTYPE
    # empty input is a no-op
    assert f(NUL, NUL, NUL, NUL, NUL, 1, 0, 2, 2, 128, 1, 1, 0.1, S0) == OK
    assert f(NUL, NUL, NUL, NUL, NUL, 0, 10, 2, 2, 128, 1, 1, 0.1, S0) == OK
    # nulls
    assert f(NUL, A16, A16, A16, NUL, 1, 64, 2, 2, 128, 1, 1, 0.1, S0) == NULL
    assert f(A16, A16, A16, NUL, NUL, 1, 64, 2, 2, 128, 1, 1, 0.1, S0) == NULL
    # unsupported head dim / group
    assert f(A16, A16, A16, A16, NUL, 1, 64, 2, 2, 64, 1, 1, 0.1, S0) == UNSUP
    assert f(A16, A16, A16, A16, NUL, 1, 64, 12, 1, 128, 1, 1, 0.1, S0) == UNSUP
    assert f(A16, A16, A16, A16, NUL, 1, 64, 2, 2, 96, 0, 1, 0.1, S0) == UNSUP
    # alignment
    assert f(MIS, A16, A16, A16, NUL, 1, 64, 2, 2, 128, 1, 1, 0.1, S0) == ALIGN
    assert f(A16, A16, A16, MIS, NUL, 1, 64, 2, 2, 64, 0, 1, 0.1, S0) == ALIGN


def test_chunked_and_append_validation(lib):
    f = lib.attn_chunked_prefill
    args = dict(q=A16, kn=A16, vn=A16, kp=A16, vp=A16, nb=10, bh=A16, bt=A16, mb=4, cb=A16, C=64,
                o=A16, lse=NUL, B=1, Hq=16, Hkv=2, D=128, base=0, scale=0.1, st=NUL, s=S0)

    def call(**kw):
        a = dict(args, **kw)
        return f(*a.values())

    assert call(Hq=15) == SHAPE
    assert call(mb=0) == SHAPE
    assert call(D=64) == UNSUP
    assert call(C=0, q=NUL) == OK
    assert call(bt=NUL) == NULL
    assert call(cb=NUL) == NULL
    assert call(vp=MIS) == ALIGN
    g = lib.attn_kv_append
    assert g(A16, A16, A16, A16, 10, A16, A16, 4, A16, 8, 1, 2, 64, 0, NUL, S0) == UNSUP
    assert g(A16, A16, A16, A16, 10, A16, A16, 0, A16, 8, 1, 2, 128, 0, NUL, S0) == SHAPE
    assert g(A16, A16, A16, A16, 10, NUL, A16, 4, A16, 8, 1, 2, 128, 0, NUL, S0) == NULL
    assert g(NUL, NUL, NUL, NUL, 10, NUL, NUL, 4, NUL, 0, 1, 2, 128, 0, NUL, S0) == OK


def test_decode_validation(lib):
    f = lib.attn_decode
    need = lib.attn_decode_workspace_bytes(32, 16, 128, 2048, 1024)
    assert need == 32 * 16 * 128 * 132 * 4
    # 0 = automatic: records of at most 768 waves + one per (request, KV head)
    # piece boundary, each holding 132 floats per query head
    assert lib.attn_decode_workspace_bytes(32, 16, 128, 2048, 0) == (768 + 32) * 16 * 132 * 4
    assert lib.attn_decode_workspace_bytes(32, 16, 128, 2048, 100) == 0    # not a multiple of 64
    assert lib.attn_decode_workspace_bytes(32, 16, 64, 2048, 0) == 0

    def call(ws=A16, wsb=need, split=1024, Hq=16, Hkv=2, D=128, q=A16):
        return f(q, A16, A16, 100, A16, A16, 2048, A16, A16, NUL, 32, Hq, Hkv, D, 0, 0.1, split,
                 ws, wsb, NUL, S0)

    assert call(split=100) == SHAPE
    assert call(Hq=15) == SHAPE
    assert call(Hq=64, Hkv=2) == UNSUP      # group of 32 > 16
    assert call(D=64) == UNSUP
    assert call(q=NUL) == NULL
    assert call(ws=NUL) == WS
    assert call(wsb=need - 1) == WS
    assert call(ws=MIS) == ALIGN


def test_decode_noalloc_validation(lib):
    """The entry point without a workspace checks its arguments like
    attn_decode, and rejects a call whose split records exceed the fixed
    device array (ATTN_ERR_SCRATCH) before any HIP call."""
    f = lib.attn_decode_noalloc
    SCRATCH = 8

    def call(B=32, Hq=16, Hkv=2, D=128, split=0, max_blocks=2048, q=A16):
        return f(q, A16, A16, 100, A16, A16, max_blocks, A16, A16, NUL, B, Hq, Hkv, D, 0, 0.1,
                 split, NUL, S0)

    assert call(split=100) == SHAPE
    assert call(Hq=15) == SHAPE
    assert call(D=64) == UNSUP
    assert call(q=NUL) == NULL
    assert _lib.ATTN_NOALLOC_SCRATCH_BYTES == 16 << 20
    # automatic splits: (768 + B) * Hq * 528 bytes; 16 heads fit up to B = 1217
    assert lib.attn_decode_workspace_bytes(1218, 16, 128, 2048, 0) > 16 << 20
    assert call(B=1218) == SCRATCH
    # fixed splits of 64 keys over 2048 blocks: 32 * 16 * 2048 records, far too many
    assert call(split=64) == SCRATCH
    assert lcat.attn_status_string(SCRATCH).startswith("call needs more decode scratch")


def test_fp8_prefill_validation(lib):
    qz, pf = lib.attn_quantize_fp8_blocks, lib.attn_prefill_fp8
    codes, sc = P(0x200000), P(0x300000)
    assert qz(A16, codes, sc, -1, 128, NUL, S0) == SHAPE
    assert qz(A16, codes, sc, 4, 48, NUL, S0) == UNSUP          # D % 32 != 0
    assert qz(A16, codes, sc, 0, 128, NUL, S0) == OK
    assert qz(NUL, codes, sc, 4, 128, NUL, S0) == NULL
    assert qz(MIS, codes, sc, 4, 128, NUL, S0) == ALIGN
    assert qz(A16, P(0x10000 + 512), sc, 4, 128, NUL, S0) == SHAPE   # codes overlap x
    # rotation signs: a host array of 128 values, each +1 or -1, and D = 128
    good = (ctypes.c_int8 * 128)(*([1, -1] * 64))
    bad = (ctypes.c_int8 * 128)(*([1] * 127 + [0]))
    sp = lambda a: ctypes.cast(a, ctypes.c_void_p)
    assert qz(A16, codes, sc, 0, 128, sp(good), S0) == OK
    assert qz(A16, codes, sc, 0, 128, sp(bad), S0) == SHAPE
    assert qz(A16, codes, sc, 4, 64, sp(good), S0) == UNSUP       # rotation needs D = 128
    args = lambda **kw: [kw.get(n, d) for n, d in (("q", A16), ("k8", A16), ("ks", A16), ("v", A16), ("o", A16))]
    def call(B=1, S=64, Hq=16, Hkv=2, D=128, signs=NUL, **kw):
        return pf(*args(**kw), NUL, B, S, Hq, Hkv, D, 1, 0.1, signs, S0)
    assert call(Hq=15) == SHAPE
    assert call(D=64) == UNSUP
    assert call(Hq=6, Hkv=2) == UNSUP                        # group 3
    assert call(S=0) == OK
    assert call(S=0, signs=sp(good)) == OK
    assert call(S=0, signs=sp(bad)) == SHAPE
    assert call(k8=NUL) == NULL
    assert call(ks=P(0x10002)) == ALIGN                     # scales 4-byte aligned
    assert call(v=MIS) == ALIGN


def test_fp8_pv_prefill_validation(lib):
    qv, pf = lib.attn_quantize_fp8_v, lib.attn_prefill_fp8_pv
    v8, vs = P(0x200000), P(0x300000)
    assert qv(A16, v8, vs, 1, -1, 2, 128, S0) == SHAPE
    assert qv(A16, v8, vs, 1, 64, 0, 128, S0) == SHAPE
    assert qv(A16, v8, vs, 1, 64, 2, 64, S0) == UNSUP          # D != 128
    assert qv(A16, v8, vs, 0, 64, 2, 128, S0) == OK
    assert qv(NUL, v8, vs, 1, 64, 2, 128, S0) == NULL
    assert qv(A16, MIS, vs, 1, 64, 2, 128, S0) == ALIGN
    assert qv(A16, P(0x10000 + 4096), vs, 1, 64, 2, 128, S0) == SHAPE   # codes overlap v
    assert qv(A16, v8, vs, 1, 1 << 24, 2, 128, S0) == SHAPE      # 128 * S64 >= 2^31
    names = ("q", "k8", "ks", "v8", "vs", "o")
    def call(B=1, S=64, Hq=16, Hkv=2, D=128, signs=NUL, **kw):
        ptrs = [kw.get(n, A16) for n in names]
        return pf(*ptrs, NUL, B, S, Hq, Hkv, D, 1, 0.1, signs, S0)
    bad = (ctypes.c_int8 * 128)(*([-1] * 64 + [2] * 64))
    assert call(S=0, signs=ctypes.cast(bad, ctypes.c_void_p)) == SHAPE
    assert call(Hq=15) == SHAPE
    assert call(D=64) == UNSUP
    assert call(Hq=6, Hkv=2) == UNSUP                          # group 3
    assert call(S=0) == OK
    assert call(S=1 << 24) == SHAPE
    assert call(v8=NUL) == NULL
    assert call(vs=NUL) == NULL
    assert call(vs=P(0x10002)) == ALIGN                        # scales 4-byte aligned
    assert call(v8=MIS) == ALIGN


def test_rope_and_permute_validation(lib):
    r = lib.rope_apply
    assert r(A16, A16, 10, 2, 100, 10000.0, S0) == UNSUP
    assert r(A16, A16, 10, 2, 128, -1.0, S0) == SHAPE
    assert r(NUL, NUL, 0, 2, 128, 10000.0, S0) == OK
    assert r(NUL, A16, 10, 2, 128, 10000.0, S0) == NULL
    assert r(MIS, A16, 10, 2, 128, 10000.0, S0) == ALIGN
    r2 = lib.rope_apply_qk
    K = P(0x40000000)
    assert r2(A16, K, A16, 10, 16, 2, 100, 10000.0, S0) == UNSUP
    assert r2(A16, K, A16, 10, 16, 0, 128, 10000.0, S0) == SHAPE
    assert r2(A16, K, A16, 10, 16, 2, 128, 0.0, S0) == SHAPE
    assert r2(NUL, NUL, NUL, 0, 16, 2, 128, 10000.0, S0) == OK
    assert r2(A16, NUL, A16, 10, 16, 2, 128, 10000.0, S0) == NULL
    assert r2(A16, MIS, A16, 10, 16, 2, 128, 10000.0, S0) == ALIGN
    assert r2(A16, P(0x10000 + 1024), A16, 10, 16, 2, 128, 10000.0, S0) == SHAPE   # k inside q
    p = lib.seq_to_head_permute
    assert p(A16, P(0x90000000), 4, 16, 6, 128, 0, 2, S0) == SHAPE     # 6 % 4
    assert p(A16, P(0x90000000), 4, 16, 8, 128, 4, 2, S0) == SHAPE     # rank out of range
    assert p(A16, P(0x90000000), 4, 16, 8, 128, 0, 3, S0) == DTYPE
    assert p(A16, NUL, 4, 16, 8, 128, 0, 2, S0) == NULL
    assert p(NUL, NUL, 4, 0, 8, 128, 0, 2, S0) == OK
    assert p(A16, P(0x10000 + 64), 4, 16, 8, 128, 0, 2, S0) == SHAPE   # overlapping buffers

    u = lib.head_to_seq_permute
    assert u(A16, P(0x90000000), 4, 16, 6, 128, 0, 2, S0) == SHAPE     # 6 % 4
    assert u(A16, P(0x90000000), 4, 16, 8, 128, -1, 2, S0) == SHAPE    # rank out of range
    assert u(A16, P(0x90000000), 4, 16, 8, 128, 0, 5, S0) == DTYPE
    assert u(NUL, P(0x90000000), 4, 16, 8, 128, 0, 2, S0) == NULL
    assert u(NUL, NUL, 4, 0, 8, 128, 0, 2, S0) == OK
    assert u(P(0x10000 + 64), A16, 4, 16, 8, 128, 0, 2, S0) == SHAPE   # overlapping buffers

    f = lib.seq_to_head_permute_qkv
    q, k, v = P(0x10000), P(0x20000000), P(0x40000000)
    qo, ko, vo = P(0x60000000), P(0x80000000), P(0xA0000000)
    assert f(q, k, v, qo, ko, vo, 4, 16, 6, 8, 128, 0, 2, S0) == SHAPE      # 6 % 4
    assert f(q, k, v, qo, ko, vo, 4, 16, 8, 6, 128, 0, 2, S0) == SHAPE      # 6 % 4
    assert f(q, k, v, qo, ko, vo, 4, 16, 8, 8, 128, 4, 2, S0) == SHAPE      # rank out of range
    assert f(q, k, v, qo, ko, vo, 4, 16, 8, 8, 128, 0, 3, S0) == DTYPE
    assert f(q, k, NUL, qo, ko, vo, 4, 16, 8, 8, 128, 0, 2, S0) == NULL
    assert f(NUL, NUL, NUL, NUL, NUL, NUL, 4, 0, 8, 8, 128, 0, 2, S0) == OK
    assert f(q, k, v, qo, P(0x60000000 + 64), vo, 4, 16, 8, 8, 128, 0, 2, S0) == SHAPE  # outputs overlap
    assert f(q, k, v, qo, ko, P(0x40000000 + 64), 4, 16, 8, 8, 128, 0, 2, S0) == SHAPE  # output on an input

    g = lib.seq_to_head_permute_qkv_rope
    pos = P(0xC0000000)
    assert g(q, k, v, qo, ko, vo, pos, 4, 16, 6, 8, 128, 0, 1e4, S0) == SHAPE      # 6 % 4
    assert g(q, k, v, qo, ko, vo, pos, 4, 16, 8, 8, 128, 4, 1e4, S0) == SHAPE      # rank out of range
    assert g(q, k, v, qo, ko, vo, pos, 4, 16, 8, 8, 120, 0, 1e4, S0) == UNSUP      # D % 16
    assert g(q, k, v, qo, ko, vo, pos, 4, 16, 8, 8, 272, 0, 1e4, S0) == UNSUP      # D > 256
    assert g(q, k, v, qo, ko, vo, pos, 4, 16, 8, 8, 128, 0, 0.0, S0) == SHAPE      # base
    assert g(q, k, v, qo, ko, vo, NUL, 4, 16, 8, 8, 128, 0, 1e4, S0) == NULL
    assert g(q, NUL, v, qo, ko, vo, pos, 4, 16, 8, 8, 128, 0, 1e4, S0) == NULL
    assert g(q, k, v, qo, P(0x80000000 + 8), vo, pos, 4, 16, 8, 8, 128, 0, 1e4, S0) == ALIGN
    assert g(q, k, v, qo, P(0x60000000 + 64), vo, pos, 4, 16, 8, 8, 128, 0, 1e4, S0) == SHAPE
    assert g(NUL, NUL, NUL, NUL, NUL, NUL, NUL, 4, 0, 8, 8, 128, 0, 1e4, S0) == OK


def test_cp_shard_tokens_match_the_oracle_split(lib):
    import oracle
    for mode, code in (("contiguous", 0), ("striped", 1), ("zigzag", 2)):
        for S, N in ((16, 4), (50, 4), (48, 4), (7, 3), (131072, 4)):
            for r in range(N):
                try:
                    want = len(oracle.cp_tokens(S, N, mode, r))
                except ValueError:
                    want = -SHAPE
                assert lib.cp_shard_tokens(S, N, r, code) == want, (mode, S, N, r)
    assert lib.cp_shard_tokens(16, 4, 0, 3) == -UNSUP
    assert lib.cp_shard_tokens(16, 4, 4, 0) == -SHAPE
    assert lib.cp_shard_tokens(16, 0, 0, 0) == -SHAPE


def test_cp_and_merge_validation(lib):
    sh = lib.cp_shard
    pos = P(0xC0000000)
    assert sh(A16, P(0x90000000), pos, 16, 8, 128, 2, 4, 0, 5, S0) == UNSUP     # mode
    assert sh(A16, P(0x90000000), pos, 18, 8, 128, 2, 4, 0, 1, S0) == SHAPE     # striped S % N
    assert sh(A16, P(0x90000000), pos, 7, 8, 128, 2, 4, 0, 2, S0) == SHAPE      # zigzag S < 2N
    assert sh(A16, P(0x90000000), pos, 16, 8, 128, 3, 4, 0, 0, S0) == DTYPE
    assert sh(NUL, P(0x90000000), pos, 16, 8, 128, 2, 4, 0, 0, S0) == NULL
    assert sh(A16, P(0x10000 + 64), pos, 16, 8, 128, 2, 4, 0, 0, S0) == SHAPE   # overlap
    assert sh(NUL, NUL, NUL, 0, 8, 128, 2, 4, 0, 2, S0) == SHAPE                # 0 < 2N
    assert sh(NUL, NUL, NUL, 0, 8, 128, 2, 1, 0, 1, S0) == OK
    un = lib.cp_unshard
    assert un(A16, P(0x90000000), 16, 8, 128, 2, 4, 4, 0, S0) == SHAPE         # rank
    assert un(P(0x10000 + 64), A16, 16, 8, 128, 2, 4, 0, 0, S0) == SHAPE       # overlap
    kl = lib.attn_key_limits
    assert kl(A16, NUL, P(0x90000000), 1, 10, 10, S0) == NULL
    assert kl(A16, A16, P(0x90000000), 1, -1, 10, S0) == SHAPE
    assert kl(NUL, NUL, NUL, 1, 0, 10, S0) == OK
    pl = lib.attn_prefill_limited
    q, k, v, o = P(0x10000), P(0x20000000), P(0x40000000), P(0x60000000)
    assert pl(q, k, v, pos, o, NUL, 1, 64, 64, 16, 2, 64, 0.1, 0, S0) == UNSUP   # D
    assert pl(q, k, v, pos, o, NUL, 1, 64, 64, 16, 3, 128, 0.1, 0, S0) == SHAPE  # Hq % Hkv
    assert pl(q, k, v, pos, o, NUL, 1, 64, 0, 16, 2, 128, 0.1, 0, S0) == SHAPE   # Sk = 0
    assert pl(q, k, v, NUL, o, NUL, 1, 64, 64, 16, 2, 128, 0.1, 0, S0) == NULL
    assert pl(q, k, v, pos, o, NUL, 1, 64, 64, 16, 2, 128, 0.1, 1, S0) == NULL   # accumulate, no lse
    assert pl(q, k, v, pos, P(0x60000000 + 8), NUL, 1, 64, 64, 16, 2, 128, 0.1, 0, S0) == ALIGN
    assert pl(NUL, NUL, NUL, NUL, NUL, NUL, 1, 0, 64, 16, 2, 128, 0.1, 0, S0) == OK
    mg = lib.attn_merge
    la, lb = P(0xA0000000), P(0xB0000000)
    assert mg(q, la, k, lb, o, NUL, 1, 64, 16, 100, S0) == UNSUP               # D % 8
    assert mg(q, la, k, lb, o, NUL, 1, 64, 16, 24, S0) == UNSUP                # 64 % (D/8)
    assert mg(q, NUL, k, lb, o, NUL, 1, 64, 16, 128, S0) == NULL
    assert mg(q, la, k, lb, P(0x10000 + 256), NUL, 1, 64, 16, 128, S0) == SHAPE   # partial overlap
    assert mg(q, la, k, lb, o, P(0xA0000000 + 4), 1, 64, 16, 128, S0) == SHAPE   # lse overlap


def test_fp8_validation(lib):
    qz = lib.attn_kv_quantize_fp8
    k, v, k8, v8, ks, vs = (P(0x10000 * (i + 1)) for i in range(6))
    assert qz(k, v, k8, v8, ks, vs, 4, 64, S0) == UNSUP
    assert qz(k, v, k8, v8, ks, vs, -1, 128, S0) == SHAPE
    assert qz(k, v, k8, NUL, ks, vs, 4, 128, S0) == NULL
    assert qz(k, v, k8, v8, P(0x30000 + 4), vs, 4, 128, S0) == ALIGN
    assert qz(NUL, NUL, NUL, NUL, NUL, NUL, 0, 128, S0) == OK
    ap = lib.attn_kv_append_fp8
    kn, vn, bh, bt, sp = (P(0x1000000 * (i + 1)) for i in range(5))
    assert ap(kn, vn, k8, v8, ks, vs, 8, bh, bt, 4, sp, 10, 2, 2, 64, 0, NUL, S0) == UNSUP
    assert ap(kn, vn, k8, v8, ks, vs, 0, bh, bt, 4, sp, 10, 2, 2, 128, 0, NUL, S0) == SHAPE
    assert ap(kn, vn, k8, v8, NUL, vs, 8, bh, bt, 4, sp, 10, 2, 2, 128, 0, NUL, S0) == NULL
    assert ap(MIS, vn, k8, v8, ks, vs, 8, bh, bt, 4, sp, 10, 2, 2, 128, 0, NUL, S0) == ALIGN
    assert ap(NUL, NUL, NUL, NUL, NUL, NUL, 8, NUL, NUL, 4, NUL, 0, 2, 2, 128, 0, NUL, S0) == OK
    d = lib.attn_decode_fp8
    q, bh, bt, cl, o, ws = (P(0x100000 * (i + 1)) for i in range(6))
    args = lambda **kw: [kw.get("q", q), k8, v8, kw.get("ks", ks), vs, 8, bh, bt, 4, cl, o, NUL,
                         2, 16, 2, kw.get("D", 128), 0, 0.1, kw.get("split", 0), ws,
                         kw.get("wsb", 1 << 30), NUL, S0]
    assert d(*args(D=64)) == UNSUP
    assert d(*args(split=100)) == SHAPE
    assert d(*args(ks=NUL)) == NULL
    assert d(*args(ks=P(0x30000 + 8))) == ALIGN
    assert d(*args(wsb=16)) == WS


def test_measure_validation(lib):
    m = lib.attn_measure_mfma_rate
    out = P(0x10000)
    assert m(NUL, 256, 64, 1, 0, S0) == NULL
    assert m(out, 0, 64, 1, 0, S0) == SHAPE
    assert m(out, 65537, 64, 1, 1, S0) == SHAPE
    assert m(out, 256, 6, 1, 0, S0) == SHAPE     # not a multiple of 4
    assert m(out, 256, 0, 1, 1, S0) == SHAPE
    assert m(out, 256, (1 << 24) + 4, 1, 0, S0) == SHAPE
    assert m(out, 256, 64, 1, 2, S0) == SHAPE    # a_from_lds is 0 or 1
    with pytest.raises(ValueError):
        lcat.measure_mfma_rate(n_wg=16, iters=10)
    rd, rb, cp = lib.attn_measure_hbm_read, lib.attn_measure_hbm_read_bytes, lib.attn_measure_hbm_copy
    buf, o2 = P(0x100000), P(0x200000)
    assert rd(NUL, 1 << 20, out, 64, S0) == NULL
    assert rd(buf, 1 << 20, NUL, 64, S0) == NULL
    assert rd(buf, 1 << 20, out, 0, S0) == SHAPE
    assert rd(buf, 16 * 63, out, 64, S0) == SHAPE        # fewer units than waves
    assert rd(P(0x100004), 1 << 20, out, 64, S0) == ALIGN
    assert rb(1000 * 16 + 5, 64) == (1000 // 64) * 64 * 16
    assert rb(8, 64) == 0 and rb(1 << 20, 0) == 0
    assert cp(NUL, o2, 1024, S0) == NULL
    assert cp(buf, o2, 1000, S0) == SHAPE                # not a multiple of 16
    assert cp(buf, o2, 0, S0) == SHAPE
    assert cp(buf, P(0x100000 + 512), 1024, S0) == SHAPE # overlap
    assert cp(P(0x100008), o2, 1024, S0) == ALIGN


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load()


def test_library_matches_its_sources(lib):
    """The loader only accepts a library built from the sources next to it."""
    from long_context_attention_tiled_amd import _build
    assert lib.attn_build_id().decode() == _build.source_hash()
