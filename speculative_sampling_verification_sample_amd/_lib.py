"""ctypes view of libspecverify.so (the C ABI declared in include/specverify.h).

The product path runs only through this library: if it is missing the import
fails with an explicit error; there is no fallback implementation.
"""

import ctypes
import os

# SPECVERIFY_LIB names another build of the same library (the host-sanitized
# one, for the ABI checks under AddressSanitizer).
LIB_PATH = os.environ.get("SPECVERIFY_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                            "libspecverify.so")

SV_OK = 0
SV_F32 = 0
SV_BF16 = 1

# Every function the header declares, with its ctypes signature.
_c_int32 = ctypes.c_int32
_ptr = ctypes.c_void_p
_size = ctypes.c_size_t


class SamplingParamsC(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("top_k", ctypes.c_int32), ("top_p", ctypes.c_float)]


SIGNATURES = {
    "spec_verify_workspace_size": (_size, [_c_int32, _c_int32, _c_int32, ctypes.c_int, SamplingParamsC]),
    "spec_verify_sample": (
        ctypes.c_int,
        [_ptr, ctypes.c_int, _ptr, _ptr, _ptr, _ptr, _c_int32, _c_int32, _c_int32, SamplingParamsC,
         _ptr, _ptr, _ptr, _ptr, _size, _ptr],
    ),
    "spec_verify_sample_noalloc": (
        ctypes.c_int,
        [_ptr, ctypes.c_int, _ptr, _ptr, _ptr, _ptr, _c_int32, _c_int32, _c_int32, SamplingParamsC,
         _ptr, _ptr, _ptr, _ptr],
    ),
    "spec_verify_greedy": (
        ctypes.c_int,
        [_ptr, ctypes.c_int, _ptr, _c_int32, _c_int32, _c_int32, _ptr, _ptr, _ptr, _ptr, _size, _ptr],
    ),
    "spec_accept_stats": (
        ctypes.c_int,
        [_ptr, ctypes.c_int, _ptr, _ptr, _c_int32, _c_int32, _c_int32, SamplingParamsC,
         _ptr, _ptr, _ptr, _ptr, _ptr, _size, _ptr],
    ),
    "spec_verify_draft_logits_workspace_size": (
        _size, [_c_int32, _c_int32, _c_int32, ctypes.c_int, ctypes.c_int, SamplingParamsC]),
    "spec_verify_sample_draft_logits": (
        ctypes.c_int,
        [_ptr, ctypes.c_int, _ptr, ctypes.c_int, _ptr, _ptr, _ptr, _c_int32, _c_int32, _c_int32,
         SamplingParamsC, _ptr, _ptr, _ptr, _ptr, _size, _ptr],
    ),
    "spec_accept_stats_draft_logits": (
        ctypes.c_int,
        [_ptr, ctypes.c_int, _ptr, ctypes.c_int, _ptr, _c_int32, _c_int32, _c_int32, SamplingParamsC,
         _ptr, _ptr, _ptr, _ptr, _ptr, _size, _ptr],
    ),
    "spec_verify_sample_stats": (
        ctypes.c_int,
        [_ptr, ctypes.c_int, _ptr, _ptr, _ptr, _ptr, _c_int32, _c_int32, _c_int32, SamplingParamsC,
         _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _size, _ptr],
    ),
    "spec_verify_sample_stats_draft_logits": (
        ctypes.c_int,
        [_ptr, ctypes.c_int, _ptr, ctypes.c_int, _ptr, _ptr, _ptr, _c_int32, _c_int32, _c_int32, SamplingParamsC,
         _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _size, _ptr],
    ),
    "spec_verify_sample_lenient": (
        ctypes.c_int,
        [_ptr, ctypes.c_int, _ptr, _ptr, _ptr, _ptr, _c_int32, _c_int32, _c_int32, SamplingParamsC,
         ctypes.c_float, _ptr, _ptr, _ptr, _ptr, _size, _ptr],
    ),
    "spec_verify_sample_ragged": (
        ctypes.c_int,
        [_ptr, ctypes.c_int, _ptr, _ptr, _ptr, _c_int32, _ptr, _ptr, _c_int32, _c_int32, _c_int32,
         SamplingParamsC, _c_int32, _ptr, _ptr, _ptr, _ptr, _size, _ptr],
    ),
    "spec_verify_sample_ragged_draft_logits": (
        ctypes.c_int,
        [_ptr, ctypes.c_int, _ptr, ctypes.c_int, _ptr, _ptr, _c_int32, _ptr, _ptr, _c_int32, _c_int32, _c_int32,
         SamplingParamsC, _c_int32, _ptr, _ptr, _ptr, _ptr, _size, _ptr],
    ),
    "spec_verify_greedy_ragged": (
        ctypes.c_int,
        [_ptr, ctypes.c_int, _ptr, _ptr, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _ptr, _ptr, _ptr,
         _ptr, _size, _ptr],
    ),
    "spec_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "spec_set_rowpass_timer": (ctypes.c_int, [_ptr, _ptr]),
    "spec_set_stage_timer": (ctypes.c_int, [_c_int32, _ptr, _ptr]),
}

_LIB = None


def load_library(path: str = LIB_PATH):
    """Load libspecverify.so once; raise if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()')"
        )
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def status_string(code: int) -> str:
    return load_library().spec_status_string(int(code)).decode()
