"""libkvc: decode attention over a compressed KV cache on AMD MI355X.

The compute runs in libkvc.so (hand-written HIP for gfx950); this package
holds the library sources (csrc/), its build script and the ctypes binding.
Importing the package loads the library and fails if it is not built.
"""
from ._lib import (  # noqa: F401
    Cache, KvcError, EXPORTS, HEAD_DIM, T_ALIGN, KVC_F32, KVC_BF16, KVC_OK, KVC_EINVAL,
    KVC_EDTYPE, KVC_EALIGN, KVC_EWORKSPACE, KVC_EALIAS, KVC_EHIP, KVC_ESCRATCH, KVC_V_TILES,
    KVC_V_ROWS,
    NOALLOC_SCRATCH_BYTES, lib, strerror,
    kvc_version, kvc_strerror, kvc_share_map, kvc_append, kvc_decode_attn_ws_bytes,
    kvc_decode_attn, kvc_decode_attn_noalloc, kvc_value_range, kvc_score_ws_bytes, kvc_score,
    kvc_score_seq,
    kvc_select_ws_bytes,
    kvc_select, kvc_select_seq, kvc_compact, kvc_philox_words, kvc_dkv_ws_bytes, kvc_dkv_score,
    kvc_gaussian_bf16, QCache, kvc_q8_quantize, kvc_q8_append, kvc_q8_decode_attn_ws_bytes,
    kvc_q8_decode_attn, XkvStore, kvc_xkv_factor_ws_bytes, kvc_xkv_factor, kvc_xkv_decode_ws_bytes,
    kvc_xkv_decode_attn, kvc_read_probe, PROBE_BLOCKS, ATTN_COUNTERS,
)

lib()
