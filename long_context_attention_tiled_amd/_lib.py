"""ctypes loader for ``libattn.so`` with the C signatures of ``include/attn.h`` and
``include/attn_measure.h``."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libattn.so")

# enum attn_status / attn_dtype / attn_dev_status
ATTN_OK = 0
ATTN_ERR_SCRATCH = 8
ATTN_NOALLOC_SCRATCH_BYTES = 16 << 20
ATTN_DTYPE_F32 = 0
ATTN_DTYPE_BF16 = 1
ATTN_DEV_OK = 0
ATTN_DEV_BAD_TAG = 1
ATTN_DEV_BAD_BLOCK = 2
ATTN_CP_CONTIGUOUS = 0
ATTN_CP_STRIPED = 1
ATTN_CP_ZIGZAG = 2

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t
_ll = ctypes.c_longlong

SIGNATURES = {
    "attn_prefill": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp]),
    "attn_kv_append": (_i, [_vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _vp, _i, _i, _i, _i, _i, _vp,
                            _vp]),
    "attn_chunked_prefill": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _vp, _i, _vp, _vp,
                                  _i, _i, _i, _i, _i, _f, _vp, _vp]),
    "attn_decode": (_i, [_vp, _vp, _vp, _i, _vp, _vp, _i, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f,
                         _i, _vp, _sz, _vp, _vp]),
    "attn_decode_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "attn_decode_noalloc": (_i, [_vp, _vp, _vp, _i, _vp, _vp, _i, _vp, _vp, _vp, _i, _i, _i, _i,
                                 _i, _f, _i, _vp, _vp]),
    "attn_decode_fp8": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _vp, _vp, _vp, _i, _i, _i,
                             _i, _i, _f, _i, _vp, _sz, _vp, _vp]),
    "attn_kv_quantize_fp8": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _vp]),
    "attn_kv_append_fp8": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _vp, _i, _i, _i,
                                _i, _i, _vp, _vp]),
    "attn_quantize_fp8_blocks": (_i, [_vp, _vp, _vp, _ll, _i, _vp, _vp]),
    "attn_prefill_fp8": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _vp,
                              _vp]),
    "attn_quantize_fp8_v": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _vp]),
    "attn_prefill_fp8_pv": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f,
                                 _vp, _vp]),
    "rope_apply": (_i, [_vp, _vp, _i, _i, _i, _f, _vp]),
    "rope_apply_qk": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _f, _vp]),
    "seq_to_head_permute": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, _vp]),
    "head_to_seq_permute": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, _vp]),
    "seq_to_head_permute_qkv_rope": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i,
                                          _i, _f, _vp]),
    "seq_to_head_permute_qkv": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i,
                                     _vp]),
    "cp_shard_tokens": (_ll, [_ll, _i, _i, _i]),
    "cp_shard": (_i, [_vp, _vp, _vp, _ll, _i, _i, _i, _i, _i, _i, _vp]),
    "cp_unshard": (_i, [_vp, _vp, _ll, _i, _i, _i, _i, _i, _i, _vp]),
    "attn_key_limits": (_i, [_vp, _vp, _vp, _i, _i, _i, _vp]),
    "attn_prefill_limited": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i,
                                  _vp]),
    "attn_merge": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp]),
    "attn_status_string": (ctypes.c_char_p, [_i]),
    "attn_build_id": (ctypes.c_char_p, []),
    # include/attn_measure.h
    "attn_measure_mfma_rate": (_i, [_vp, _i, _i, ctypes.c_uint32, _i, _vp]),
    "attn_measure_hbm_read": (_i, [_vp, _ll, _vp, _i, _vp]),
    "attn_measure_hbm_read_bytes": (_ll, [_ll, _i]),
    "attn_measure_hbm_copy": (_i, [_vp, _vp, _ll, _vp]),
}


class AttnError(RuntimeError):
    """A libattn call returned a non-zero status."""

    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


_lib = None


BUILD_HINT = "(python -c 'import __graft_entry__ as g; g.build()')"


def load() -> ctypes.CDLL:
    """Load the HIP library; fails loudly when it has not been built, or when
    it was built from sources other than the ones next to it."""
    global _lib
    if _lib is None:
        from . import _build
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build the HIP extension first {BUILD_HINT}")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        built, want = lib.attn_build_id().decode(), _build.source_hash()
        if built != want:
            raise RuntimeError(f"{LIB_PATH} was built from sources {built}, but the sources here "
                               f"hash to {want}: rebuild it {BUILD_HINT}")
        _lib = lib
    return _lib


def check(fn: str, status: int) -> None:
    if status != ATTN_OK:
        text = load().attn_status_string(status).decode()
        raise AttnError(fn, status, text)
