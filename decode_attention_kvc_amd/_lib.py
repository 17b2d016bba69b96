"""ctypes binding of libkvc.so.

Argument marshalling only: every function here has the name of the C export
it calls, converts torch tensors to device pointers (and the current HIP
stream), and raises KvcError on a non-zero status.  All computation runs in
the library's HIP kernels; there is no fallback path.
"""
import ctypes
import dataclasses
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvc.so")

KVC_OK, KVC_EINVAL, KVC_EDTYPE, KVC_EALIGN, KVC_EWORKSPACE, KVC_EALIAS, KVC_EHIP = 0, -1, -2, -3, -4, -5, -6
KVC_ESCRATCH = -7
NOALLOC_SCRATCH_BYTES = 32 << 20
KVC_F32, KVC_BF16 = 0, 1
KVC_V_TILES, KVC_V_ROWS = 0, 1
HEAD_DIM = 128
T_ALIGN = 64
V_TILE = 32

EXPORTS = (
    "kvc_version", "kvc_strerror", "kvc_share_map", "kvc_append",
    "kvc_decode_attn_ws_bytes", "kvc_decode_attn", "kvc_decode_attn_noalloc", "kvc_value_range",
    "kvc_score_ws_bytes", "kvc_score", "kvc_score_seq", "kvc_select_ws_bytes", "kvc_select",
    "kvc_select_seq",
    "kvc_compact", "kvc_philox_words", "kvc_dkv_ws_bytes", "kvc_dkv_score",
    "kvc_gaussian_bf16", "kvc_q8_quantize", "kvc_q8_append", "kvc_q8_decode_attn_ws_bytes",
    "kvc_q8_decode_attn", "kvc_xkv_factor_ws_bytes", "kvc_xkv_factor", "kvc_xkv_decode_ws_bytes",
    "kvc_xkv_decode_attn", "kvc_read_probe",
)


class KvcError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: status {status} ({strerror(status)})")


class kvc_cache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("n_slots", ctypes.c_int32), ("nb", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("t_len", ctypes.c_int32), ("t_cap", ctypes.c_int32),
                ("nb_cap", ctypes.c_int32), ("batch_idx", ctypes.c_void_p),
                ("seq_len", ctypes.c_void_p), ("v_layout", ctypes.c_int32)]


class kvc_qcache(ctypes.Structure):
    _fields_ = [("kq", ctypes.c_void_p), ("vq", ctypes.c_void_p), ("sk", ctypes.c_void_p),
                ("sv", ctypes.c_void_p), ("kp", ctypes.c_void_p), ("vp", ctypes.c_void_p),
                ("n_slots", ctypes.c_int32), ("nb", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("t_len", ctypes.c_int32), ("t_cap", ctypes.c_int32),
                ("p_len", ctypes.c_int32), ("p_cap", ctypes.c_int32)]


class kvc_xkv(ctypes.Structure):
    _fields_ = [("ak", ctypes.c_void_p), ("av", ctypes.c_void_p), ("lk", ctypes.c_void_p),
                ("bk", ctypes.c_void_p), ("bv", ctypes.c_void_p), ("nb", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("window", ctypes.c_int32), ("rank", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("t_len", ctypes.c_int32), ("t_cap", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m decode_attention_kvc_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz, f32 = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                 ctypes.c_size_t, ctypes.c_float)
        cp = ctypes.POINTER(kvc_cache)
        qp = ctypes.POINTER(kvc_qcache)
        xp = ctypes.POINTER(kvc_xkv)
        ip = ctypes.POINTER(ctypes.c_int32)
        szp = ctypes.POINTER(ctypes.c_size_t)
        sig = {
            "kvc_version": ([], i32),
            "kvc_strerror": ([i32], ctypes.c_char_p),
            "kvc_share_map": ([i32, ip, i32, ip, ip], i32),
            "kvc_append": ([cp, i32, vp, vp, vp], i32),
            "kvc_decode_attn_ws_bytes": ([cp, i32, i32, szp], i32),
            "kvc_decode_attn": ([cp, vp, i64, i32, ip, i32, f32, vp, vp, i32, vp, i64, vp, i64,
                                 vp, sz, vp], i32),
            "kvc_decode_attn_noalloc": ([cp, vp, i64, i32, ip, i32, f32, vp, vp, i32, vp, i64,
                                         vp, i64, vp], i32),
            "kvc_value_range": ([cp, i32, vp, vp], i32),
            "kvc_score_ws_bytes": ([cp, i32, i32, szp], i32),
            "kvc_score": ([cp, i32, vp, i32, i32, f32, vp, vp, vp, vp, sz, vp], i32),
            "kvc_score_seq": ([cp, i32, vp, i32, vp, i32, i32, f32, vp, vp, vp, vp, sz, vp], i32),
            "kvc_select_ws_bytes": ([i32, i32, i32, szp], i32),
            "kvc_select": ([vp, vp, i32, i32, i32, i32, i32, i32, ctypes.c_uint64, i32, vp, vp,
                            sz, vp], i32),
            "kvc_select_seq": ([vp, vp, i32, i32, i32, vp, vp, i32, i32, i32, ctypes.c_uint64,
                                i32, vp, vp, sz, vp], i32),
            "kvc_compact": ([cp, i32, vp, i32, cp, vp], i32),
            "kvc_philox_words": ([i64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                  ctypes.c_uint64, vp, vp], i32),
            "kvc_read_probe": ([vp, sz, vp, vp], i32),
            "kvc_dkv_ws_bytes": ([cp, i32, szp], i32),
            "kvc_dkv_score": ([cp, i32, vp, i32, vp, vp, vp, sz, vp], i32),
            "kvc_gaussian_bf16": ([i64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, vp,
                                   vp], i32),
            "kvc_q8_quantize": ([cp, i32, vp, i32, qp, vp], i32),
            "kvc_q8_append": ([qp, i32, vp, vp, vp], i32),
            "kvc_q8_decode_attn_ws_bytes": ([qp, i32, i32, szp], i32),
            "kvc_q8_decode_attn": ([qp, vp, i64, i32, ip, i32, f32, vp, i64, vp, i64, vp, sz,
                                    vp], i32),
            "kvc_xkv_factor_ws_bytes": ([xp, szp], i32),
            "kvc_xkv_factor": ([cp, i32, i32, ctypes.c_uint64, xp, vp, sz, vp], i32),
            "kvc_xkv_decode_ws_bytes": ([xp, i32, i32, szp], i32),
            "kvc_xkv_decode_attn": ([xp, i32, vp, i32, f32, i32, vp, vp, vp, vp, vp, vp, sz, vp],
                                    i32),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def strerror(status):
    return lib().kvc_strerror(int(status)).decode()


def _check(status, where):
    if status != KVC_OK:
        raise KvcError(status, where)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _arg(t, name, dtype, elems, n=1, stride=0):
    """Check a device-memory argument before its pointer crosses the ABI (the
    C side sees only the pointer): element type, an extent of `elems`
    elements (packed, stride 0: t contiguous with at least that many), or
    `n` blocks of `elems` elements `stride` elements apart inside t's
    storage, and a device tensor.  Returns the pointer (None for None)."""
    if t is None:
        return None
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if stride == 0:
        if not t.is_contiguous():
            raise ValueError(f"{name}: must be contiguous")
        if t.numel() < n * elems:
            raise ValueError(f"{name}: {t.numel()} elements, the call uses {n * elems}")
    else:
        span = (n - 1) * stride + elems
        if (t.storage_offset() + span) * t.element_size() > t.untyped_storage().nbytes():
            raise ValueError(f"{name}: {n} blocks of {elems} elements {stride} apart leave "
                             f"the tensor's storage")
    return t.data_ptr()


def _on_device(**tensors):
    """The device arguments of a call, checked after their types and extents."""
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name}: must be a device tensor")


_HAS_GPU = None


def _stream(stream):
    """The caller's stream, else torch's current stream (None without a GPU)."""
    global _HAS_GPU
    if stream is not None:
        return stream
    if _HAS_GPU is None:
        _HAS_GPU = torch.cuda.is_available()
    return torch.cuda.current_stream().cuda_stream if _HAS_GPU else None


def _dtype_code(dt):
    if dt == torch.float32:
        return KVC_F32
    if dt == torch.bfloat16:
        return KVC_BF16
    raise ValueError(f"unsupported dtype {dt}")


@dataclass
class Cache:
    """A leader-slot KV cache in libkvc's layout (see include/kvc.h).

    k: [n_slots][nb_cap][n_kv_heads][t_cap][128] rows;
    v: [n_slots][nb_cap][n_kv_heads][t_cap/32][128][32], tiles of 32 tokens,
    each tile channel-major (v_layout "tiles", the decode layout), or
    [n_slots][nb_cap][n_kv_heads][t_cap][128] rows like k (v_layout "rows",
    a prefill's layout: an input of the prompt compression).
    Ragged batches: batch_idx (device int32 [n]: the entry of each sequence)
    and seq_len (device int32 [n]: its rows) make the object address n
    sequences; t_len is then the bound on their lengths.  seqs() makes such a
    view of the same buffers."""
    k: torch.Tensor
    v: torch.Tensor
    t_len: int
    batch_idx: Optional[torch.Tensor] = None
    seq_len: Optional[torch.Tensor] = None
    v_layout: str = "tiles"

    def seqs(self, batch_idx=None, seq_len=None, t_len=None):
        """The same buffers addressing the sequences of batch_idx / seq_len."""
        for a in (batch_idx, seq_len):
            if a is not None and (a.dtype != torch.int32 or not a.is_contiguous()):
                raise ValueError("batch_idx / seq_len must be contiguous int32 tensors")
        if batch_idx is not None and seq_len is not None and batch_idx.numel() != seq_len.numel():
            raise ValueError("batch_idx and seq_len differ in length")
        return dataclasses.replace(self, batch_idx=batch_idx, seq_len=seq_len,
                                   t_len=self.t_len if t_len is None else t_len)

    @staticmethod
    def empty(n_slots, nb, n_kv_heads, t_cap, dtype=torch.bfloat16, device="cuda", t_len=0,
              v_layout="tiles"):
        t_cap = int(math.ceil(t_cap / T_ALIGN) * T_ALIGN)
        k = torch.empty((n_slots, nb, n_kv_heads, t_cap, HEAD_DIM), dtype=dtype, device=device)
        if v_layout == "rows":
            v = torch.empty_like(k)
        elif v_layout == "tiles":
            v = torch.empty((n_slots, nb, n_kv_heads, t_cap // V_TILE, HEAD_DIM, V_TILE),
                            dtype=dtype, device=device)
        else:
            raise ValueError(f"unknown value layout {v_layout!r}")
        return Cache(k, v, t_len, v_layout=v_layout)

    @property
    def n_slots(self):
        return self.k.shape[0]

    @property
    def nb_cap(self):
        return self.k.shape[1]

    @property
    def nb(self):
        """Sequences the object addresses."""
        for a in (self.batch_idx, self.seq_len):
            if a is not None:
                return a.numel()
        return self.nb_cap

    @property
    def n_kv_heads(self):
        return self.k.shape[2]

    @property
    def t_cap(self):
        return self.k.shape[3]

    @property
    def dtype(self):
        return self.k.dtype

    def desc(self):
        """The kvc_cache descriptor (built once per object; t_len refreshed)."""
        d = self.__dict__.get("_desc")
        key = (self.k.data_ptr(), self.v.data_ptr(), _ptr(self.batch_idx), _ptr(self.seq_len))
        if d is None or self.__dict__.get("_desc_key") != key:
            if self.v_layout not in ("tiles", "rows"):
                raise ValueError(f"unknown value layout {self.v_layout!r}")
            d = kvc_cache(key[0], key[1], _dtype_code(self.k.dtype), self.n_slots, self.nb,
                          self.n_kv_heads, HEAD_DIM, 0, self.t_cap, self.nb_cap, key[2], key[3],
                          KVC_V_ROWS if self.v_layout == "rows" else KVC_V_TILES)
            self.__dict__["_desc"], self.__dict__["_desc_key"] = d, key
        d.t_len = int(self.t_len)
        return d

    # views in logical [..][t][d] form (plumbing for tests and data setup)
    def k_rows(self, slot):
        return self.k[slot, :, :, : self.t_len, :]

    def v_rows(self, slot):
        """Logical value rows [nb][hkv][t_len][128] (a copy for tiles, a view
        for rows)."""
        if self.v_layout == "rows":
            return self.v[slot, :, :, : self.t_len, :]
        v = self.v[slot].transpose(-1, -2).reshape(self.nb_cap, self.n_kv_heads, self.t_cap,
                                                    HEAD_DIM)
        return v[:, :, : self.t_len]

    def v_row(self, slot, t):
        """Value row t of every (b, kv head): [nb][hkv][128] (a view)."""
        if self.v_layout == "rows":
            return self.v[slot, :, :, t, :]
        return self.v[slot, :, :, t // V_TILE, :, t % V_TILE]

    def fill(self, slot, k_rows, v_rows):
        """Write logical rows [nb][hkv][T][d] into a slot and set t_len = T;
        rows past T keep their old contents."""
        T = k_rows.shape[2]
        self.k[slot, :, :, :T, :].copy_(k_rows)
        if self.v_layout == "rows":
            self.v[slot, :, :, :T, :].copy_(v_rows)
            self.t_len = T
            return
        nfull, rem = divmod(T, V_TILE)
        nb, h = self.nb_cap, self.n_kv_heads
        if nfull:
            self.v[slot, :, :, :nfull].copy_(
                v_rows[:, :, : nfull * V_TILE].reshape(nb, h, nfull, V_TILE, HEAD_DIM)
                .transpose(-1, -2))
        if rem:
            self.v[slot, :, :, nfull, :, :rem].copy_(v_rows[:, :, nfull * V_TILE:].transpose(-1, -2))
        self.t_len = T


@dataclass
class QCache:
    """A range-protected int8 cache in libkvc's layout (see include/kvc.h).

    kq: uint8 [n_slots][nb][hkv][t_cap][128] key codes + 128;
    vq: uint8 [n_slots][nb][hkv][t_cap/32][128][32] value codes + 128;
    sk, sv: float32 [n_slots][nb][hkv][t_cap] row scales (sk < 0: protected);
    kp, vp: bf16 protected rows, [n_slots][nb][hkv][p_cap][128] and tiled."""
    kq: torch.Tensor
    vq: torch.Tensor
    sk: torch.Tensor
    sv: torch.Tensor
    kp: torch.Tensor
    vp: torch.Tensor
    t_len: int
    p_len: int

    @staticmethod
    def empty(n_slots, nb, n_kv_heads, t_cap, p_cap, device="cuda"):
        t_cap = int(math.ceil(t_cap / T_ALIGN) * T_ALIGN)
        p_cap = int(math.ceil(max(p_cap, 1) / T_ALIGN) * T_ALIGN)
        u8 = dict(dtype=torch.uint8, device=device)
        kq = torch.empty((n_slots, nb, n_kv_heads, t_cap, HEAD_DIM), **u8)
        vq = torch.empty((n_slots, nb, n_kv_heads, t_cap // V_TILE, HEAD_DIM, V_TILE), **u8)
        sk = torch.empty((n_slots, nb, n_kv_heads, t_cap), dtype=torch.float32, device=device)
        sv = torch.empty_like(sk)
        kp = Cache.empty(n_slots, nb, n_kv_heads, p_cap, device=device)
        return QCache(kq, vq, sk, sv, kp.k, kp.v, 0, 0)

    @property
    def n_slots(self):
        return self.kq.shape[0]

    @property
    def nb(self):
        return self.kq.shape[1]

    @property
    def n_kv_heads(self):
        return self.kq.shape[2]

    @property
    def t_cap(self):
        return self.kq.shape[3]

    @property
    def p_cap(self):
        return self.kp.shape[3]

    def desc(self):
        """The kvc_qcache descriptor (built once per object; lengths refreshed)."""
        d = self.__dict__.get("_desc")
        key = tuple(t.data_ptr() for t in (self.kq, self.vq, self.sk, self.sv, self.kp, self.vp))
        if d is None or self.__dict__.get("_desc_key") != key:
            d = kvc_qcache(*key, self.n_slots, self.nb, self.n_kv_heads, HEAD_DIM, 0, self.t_cap,
                           0, self.p_cap)
            self.__dict__["_desc"], self.__dict__["_desc_key"] = d, key
        d.t_len = int(self.t_len)
        d.p_len = int(self.p_len)
        return d

    def nbytes_per_row(self):
        """HBM bytes decode attention reads per quantized row (codes + scales)."""
        return 2 * HEAD_DIM + 2 * 4


@dataclass
class XkvStore:
    """One window's cross-layer factorisation in libkvc's layout (see
    include/kvc.h): the key basis ak (bf16 [nb][hkv][t_cap][rank]), the value
    basis av chunk-transposed (bf16 [nb][hkv][t_cap/8][rank][8]: the 8 rows
    of a chunk side by side for each rank; av_rows / set_av_rows convert),
    key landmarks lk (bf16 [nb][hkv][t_cap/8][rank]) and the per-layer
    matrices, stored transposed in bk, bv (float32 [nb][hkv][window*128][rank])."""
    ak: torch.Tensor
    av: torch.Tensor
    lk: torch.Tensor
    bk: torch.Tensor
    bv: torch.Tensor
    window: int
    t_len: int

    CHUNK = 8

    @staticmethod
    def empty(nb, n_kv_heads, window, rank, t_cap, device="cuda", t_len=0):
        t_cap = int(math.ceil(max(t_cap, 1) / T_ALIGN) * T_ALIGN)
        bf = dict(dtype=torch.bfloat16, device=device)
        ak = torch.empty((nb, n_kv_heads, t_cap, rank), **bf)
        av = torch.empty((nb, n_kv_heads, t_cap // XkvStore.CHUNK, rank, XkvStore.CHUNK), **bf)
        lk = torch.empty((nb, n_kv_heads, t_cap // XkvStore.CHUNK, rank), **bf)
        bk = torch.empty((nb, n_kv_heads, window * HEAD_DIM, rank), dtype=torch.float32,
                         device=device)
        bv = torch.empty_like(bk)
        return XkvStore(ak, av, lk, bk, bv, window, t_len)

    @property
    def nb(self):
        return self.ak.shape[0]

    @property
    def n_kv_heads(self):
        return self.ak.shape[1]

    @property
    def t_cap(self):
        return self.ak.shape[2]

    @property
    def rank(self):
        return self.ak.shape[3]

    def av_rows(self, b=None, j=None):
        """The value basis as rows (a copy): bf16 [nb][hkv][t_cap][rank], or
        [t_cap][rank] for one (b, j)."""
        if b is not None:
            return self.av[b, j].transpose(-1, -2).reshape(self.t_cap, self.rank)
        return self.av.transpose(-1, -2).reshape(self.nb, self.n_kv_heads, self.t_cap, self.rank)

    def set_av_rows(self, b, j, rows):
        """Rows [0, len(rows)) of the value basis of (b, j) from [n][rank]."""
        n = rows.shape[0]
        full = self.av[b, j].transpose(-1, -2).reshape(self.t_cap, self.rank).clone()
        full[:n] = rows.to(full.dtype)
        self.av[b, j].copy_(full.reshape(self.t_cap // self.CHUNK, self.CHUNK,
                                         self.rank).transpose(-1, -2))

    def desc(self):
        return kvc_xkv(self.ak.data_ptr(), self.av.data_ptr(), self.lk.data_ptr(),
                       self.bk.data_ptr(), self.bv.data_ptr(), self.nb, self.n_kv_heads,
                       HEAD_DIM, self.window, self.rank, self.CHUNK, int(self.t_len), self.t_cap)

    def nbytes(self):
        """Bytes the window's factorisation occupies (bases, matrices, landmarks)."""
        return sum(t.numel() * t.element_size() for t in (self.ak, self.av, self.lk, self.bk,
                                                           self.bv))


# ---------------------------------------------------------------------------
# exports
# ---------------------------------------------------------------------------
def kvc_version():
    return lib().kvc_version()


def kvc_strerror(status):
    return strerror(status)


def kvc_share_map(n_layers, leaders):
    """Returns (src_layer, src_slot) as lists."""
    arr = (ctypes.c_int32 * max(1, len(leaders)))(*leaders)
    src = (ctypes.c_int32 * n_layers)()
    slot = (ctypes.c_int32 * n_layers)()
    _check(lib().kvc_share_map(n_layers, arr, len(leaders), src, slot), "kvc_share_map")
    return list(src), list(slot)


def kvc_append(cache, slot, k_new, v_new, stream=None):
    c = cache.desc()
    row = cache.nb * cache.n_kv_heads * HEAD_DIM
    pk, pv = _arg(k_new, "k_new", cache.dtype, row), _arg(v_new, "v_new", cache.dtype, row)
    _on_device(k_new=k_new, v_new=v_new)
    _check(lib().kvc_append(ctypes.byref(c), slot, pk, pv, _stream(stream)), "kvc_append")


def _attn_args(cache, q, out, lse, k_new, v_new, append_slot, nq, hq, qs, os_, ls):
    """Pointers of a decode-attention call's device arguments, checked."""
    per = cache.nb * hq * HEAD_DIM
    row = cache.nb * cache.n_kv_heads * HEAD_DIM
    app = append_slot >= 0
    ptrs = (_arg(q, "q", cache.dtype, per, nq, qs), _arg(out, "out", torch.float32, per, nq, os_),
            _arg(lse, "lse", torch.float32, cache.nb * hq, nq, ls),
            _arg(k_new if app else None, "k_new", cache.dtype, row),
            _arg(v_new if app else None, "v_new", cache.dtype, row))
    _on_device(q=q, out=out, lse=lse, k_new=k_new if app else None, v_new=v_new if app else None)
    return ptrs


def kvc_decode_attn_ws_bytes(cache, n_q_layers, n_q_heads):
    c = cache.desc()
    out = ctypes.c_size_t()
    _check(lib().kvc_decode_attn_ws_bytes(ctypes.byref(c), n_q_layers, n_q_heads,
                                          ctypes.byref(out)), "kvc_decode_attn_ws_bytes")
    return out.value


def kvc_decode_attn(cache, q, q_slot, out, lse=None, ws=None, scale=0.0, k_new=None,
                    v_new=None, append_slot=-1, q_layer_stride=0, out_layer_stride=0,
                    lse_layer_stride=0, n_q_layers=None, n_q_heads=None, stream=None):
    """q: [nq][nb][Hq][d] (or strided views given explicit strides); ws:
    kvc_decode_attn_ws_bytes bytes of device memory, allocated zeroed (its
    head of arrival counters starts at zero; every call leaves it zero)."""
    c = cache.desc()
    nq = len(q_slot) if n_q_layers is None else n_q_layers
    hq = q.shape[-2] if n_q_heads is None else n_q_heads
    slots = (ctypes.c_int32 * max(1, nq))(*[int(s) for s in q_slot])
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    pq, po, pl, pk, pv = _attn_args(cache, q, out, lse, k_new, v_new, append_slot, nq, hq,
                                    q_layer_stride, out_layer_stride, lse_layer_stride)
    _on_device(ws=ws)
    _check(lib().kvc_decode_attn(ctypes.byref(c), pq, q_layer_stride, nq, slots, hq,
                                 float(scale), pk, pv, append_slot, po, out_layer_stride, pl,
                                 lse_layer_stride, _arg(ws, "ws", None, 0), ws_bytes,
                                 _stream(stream)), "kvc_decode_attn")


def kvc_decode_attn_noalloc(cache, q, q_slot, out, lse=None, scale=0.0, k_new=None,
                            v_new=None, append_slot=-1, q_layer_stride=0, out_layer_stride=0,
                            lse_layer_stride=0, n_q_layers=None, n_q_heads=None, stream=None):
    """kvc_decode_attn with its partials in the library's own device array
    (no workspace argument, nothing allocated)."""
    c = cache.desc()
    nq = len(q_slot) if n_q_layers is None else n_q_layers
    hq = q.shape[-2] if n_q_heads is None else n_q_heads
    slots = (ctypes.c_int32 * max(1, nq))(*[int(s) for s in q_slot])
    pq, po, pl, pk, pv = _attn_args(cache, q, out, lse, k_new, v_new, append_slot, nq, hq,
                                    q_layer_stride, out_layer_stride, lse_layer_stride)
    _check(lib().kvc_decode_attn_noalloc(ctypes.byref(c), pq, q_layer_stride, nq, slots, hq,
                                         float(scale), pk, pv, append_slot, po,
                                         out_layer_stride, pl, lse_layer_stride,
                                         _stream(stream)),
           "kvc_decode_attn_noalloc")


def kvc_value_range(cache, slot, rng, stream=None):
    c = cache.desc()
    per_row = cache.nb * cache.n_kv_heads * int(cache.t_len)
    pr = _arg(rng, "range", torch.float32, per_row)
    _on_device(range=rng)
    _check(lib().kvc_value_range(ctypes.byref(c), slot, pr, _stream(stream)), "kvc_value_range")


def kvc_score_ws_bytes(cache, n_q_heads, w):
    c = cache.desc()
    out = ctypes.c_size_t()
    _check(lib().kvc_score_ws_bytes(ctypes.byref(c), n_q_heads, w, ctypes.byref(out)),
           "kvc_score_ws_bytes")
    return out.value


def kvc_score(cache, slot, q_obs, score, rng=None, lse_obs=None, ws=None, scale=0.0,
              stream=None):
    """q_obs: [w][nb][Hq][d]."""
    c = cache.desc()
    w, hq = q_obs.shape[0], q_obs.shape[2]
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    nb = cache.nb
    per_row = nb * cache.n_kv_heads * int(cache.t_len)
    if q_obs.dim() != 4 or q_obs.shape[1] != nb or q_obs.shape[3] != HEAD_DIM:
        raise ValueError(f"q_obs: shape {tuple(q_obs.shape)}, expected [w][{nb}][Hq][128]")
    pq = _arg(q_obs, "q_obs", cache.dtype, w * nb * hq * HEAD_DIM)
    pl = _arg(lse_obs, "lse_obs", torch.float32, w * nb * hq)
    ps = _arg(score, "score", torch.float32, per_row)
    pr = _arg(rng, "range", torch.float32, per_row)
    _on_device(q_obs=q_obs, lse_obs=lse_obs, score=score, range=rng, ws=ws)
    _check(lib().kvc_score(ctypes.byref(c), slot, pq, hq, w, float(scale), pl, ps, pr,
                           _arg(ws, "ws", None, 0), ws_bytes, _stream(stream)), "kvc_score")


def kvc_score_seq(cache, slot, q_obs, q_idx, score, rng=None, lse_obs=None, ws=None, scale=0.0,
                  stream=None):
    """q_obs: [w][q_nb][Hq][d] (the whole batch's window queries); q_idx:
    device int32 [cache.nb], the q_obs row of each sequence the cache view
    addresses, or None (row b)."""
    c = cache.desc()
    if q_obs.dim() != 4 or q_obs.shape[3] != HEAD_DIM:
        raise ValueError(f"q_obs: shape {tuple(q_obs.shape)}, expected [w][q_nb][Hq][128]")
    w, q_nb, hq = q_obs.shape[0], q_obs.shape[1], q_obs.shape[2]
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    per_row = cache.nb * cache.n_kv_heads * int(cache.t_len)
    pq = _arg(q_obs, "q_obs", cache.dtype, w * q_nb * hq * HEAD_DIM)
    pi = _arg(q_idx, "q_idx", torch.int32, cache.nb)
    pl = _arg(lse_obs, "lse_obs", torch.float32, w * q_nb * hq)
    ps = _arg(score, "score", torch.float32, per_row)
    pr = _arg(rng, "range", torch.float32, per_row)
    _on_device(q_obs=q_obs, q_idx=q_idx, lse_obs=lse_obs, score=score, range=rng, ws=ws)
    _check(lib().kvc_score_seq(ctypes.byref(c), slot, pq, q_nb, pi, hq, w, float(scale), pl, ps,
                               pr, _arg(ws, "ws", None, 0), ws_bytes, _stream(stream)),
           "kvc_score_seq")


def kvc_select_ws_bytes(nb, n_kv_heads, t_len):
    out = ctypes.c_size_t()
    _check(lib().kvc_select_ws_bytes(nb, n_kv_heads, t_len, ctypes.byref(out)),
           "kvc_select_ws_bytes")
    return out.value


def _select_args(score, rng, kept, nb, n_kv_heads, t_len, budget_k, recent_b):
    per_row = nb * n_kv_heads * t_len
    n_keep = nb * n_kv_heads * min(t_len, budget_k + recent_b)
    ptrs = (_arg(score, "score", torch.float32, per_row),
            _arg(rng, "range", torch.float32, per_row),
            _arg(kept, "kept", torch.int32, n_keep))
    _on_device(score=score, range=rng, kept=kept)
    return ptrs


def kvc_select(score, rng, nb, n_kv_heads, t_len, budget_k, recent_b, n_v, seed, layer_id,
               kept, ws=None, stream=None):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    ps, pr, pk = _select_args(score, rng, kept, nb, n_kv_heads, t_len, budget_k, recent_b)
    _check(lib().kvc_select(ps, pr, nb, n_kv_heads, t_len, budget_k, recent_b,
                            n_v, int(seed) & (2**64 - 1), layer_id, pk, _arg(ws, "ws", None, 0),
                            ws_bytes, _stream(stream)), "kvc_select")


def kvc_select_seq(score, rng, nb, n_kv_heads, t_len, seq_len, seq_id, budget_k, recent_b, n_v,
                   seed, layer_id, kept, ws=None, stream=None):
    """seq_len, seq_id: device int32 [nb] or None."""
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    ps, pr, pk = _select_args(score, rng, kept, nb, n_kv_heads, t_len, budget_k, recent_b)
    _check(lib().kvc_select_seq(ps, pr, nb, n_kv_heads, t_len,
                                _arg(seq_len, "seq_len", torch.int32, nb),
                                _arg(seq_id, "seq_id", torch.int32, nb), budget_k, recent_b, n_v,
                                int(seed) & (2**64 - 1), layer_id, pk, _arg(ws, "ws", None, 0),
                                ws_bytes, _stream(stream)),
           "kvc_select_seq")


def kvc_compact(src, slot, kept, n_keep, dst, stream=None):
    """kept: device int32 [nb][hkv][n_keep], or None for rows [0, n_keep)."""
    cs, cd = src.desc(), dst.desc()
    pk = _arg(kept, "kept", torch.int32, src.nb * src.n_kv_heads * n_keep)
    _on_device(kept=kept)
    _check(lib().kvc_compact(ctypes.byref(cs), slot, pk, n_keep, ctypes.byref(cd),
                             _stream(stream)), "kvc_compact")


def kvc_philox_words(n, c1, c2, c3, seed, out, stream=None):
    _check(lib().kvc_philox_words(n, c1, c2, c3, int(seed) & (2**64 - 1), _ptr(out),
                                  _stream(stream)), "kvc_philox_words")


PROBE_BLOCKS = 256
ATTN_COUNTERS = 16384      # arrival counters at the head of a kvc_decode_attn workspace


def kvc_read_probe(buf, out, stream=None):
    """Stream the device tensor buf once (its bytes, a multiple of 16) and
    write one XOR checksum word per probe workgroup into out (device int32 or
    uint32, PROBE_BLOCKS elements)."""
    nbytes = buf.numel() * buf.element_size()
    _on_device(buf=buf, out=out)
    if not buf.is_contiguous():
        raise ValueError("kvc_read_probe: buf must be contiguous")
    if out.dtype not in (torch.int32, torch.uint32) or not out.is_contiguous() \
            or out.numel() < PROBE_BLOCKS:
        raise ValueError(f"kvc_read_probe: out must be {PROBE_BLOCKS} contiguous 32-bit words")
    _check(lib().kvc_read_probe(_ptr(buf), nbytes, _ptr(out), _stream(stream)), "kvc_read_probe")


def kvc_dkv_ws_bytes(cache, rank):
    c = cache.desc()
    out = ctypes.c_size_t()
    _check(lib().kvc_dkv_ws_bytes(ctypes.byref(c), rank, ctypes.byref(out)), "kvc_dkv_ws_bytes")
    return out.value


def kvc_dkv_score(cache, slot, g, score, rng=None, ws=None, stream=None):
    """g: bf16 [rank][2*head_dim] (row n = sketch column n)."""
    c = cache.desc()
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    per_row = cache.nb * cache.n_kv_heads * int(cache.t_len)
    _on_device(g=g, score=score, range=rng, ws=ws)
    _check(lib().kvc_dkv_score(ctypes.byref(c), slot,
                               _arg(g, "g", torch.bfloat16, g.shape[0] * 2 * HEAD_DIM),
                               g.shape[0], _arg(score, "score", torch.float32, per_row),
                               _arg(rng, "range", torch.float32, per_row),
                               _arg(ws, "ws", None, 0), ws_bytes, _stream(stream)),
           "kvc_dkv_score")


def kvc_gaussian_bf16(n, seed, c1, c2, out, stream=None):
    _check(lib().kvc_gaussian_bf16(n, int(seed) & (2**64 - 1), c1, c2, _ptr(out),
                                   _stream(stream)), "kvc_gaussian_bf16")


def kvc_q8_quantize(src, slot, protect, n_protect, dst, stream=None):
    """protect: device int32 [nb][hkv][n_protect] ascending (None if 0).
    Sets dst.t_len and dst.p_len before the call."""
    dst.t_len, dst.p_len = src.t_len, n_protect
    cs, cd = src.desc(), dst.desc()
    _check(lib().kvc_q8_quantize(ctypes.byref(cs), slot, _ptr(protect), n_protect,
                                 ctypes.byref(cd), _stream(stream)), "kvc_q8_quantize")


def kvc_q8_append(cache, slot, k_new, v_new, stream=None):
    c = cache.desc()
    _check(lib().kvc_q8_append(ctypes.byref(c), slot, _ptr(k_new), _ptr(v_new), _stream(stream)),
           "kvc_q8_append")


def kvc_q8_decode_attn_ws_bytes(cache, n_q_layers, n_q_heads):
    c = cache.desc()
    out = ctypes.c_size_t()
    _check(lib().kvc_q8_decode_attn_ws_bytes(ctypes.byref(c), n_q_layers, n_q_heads,
                                             ctypes.byref(out)), "kvc_q8_decode_attn_ws_bytes")
    return out.value


def kvc_q8_decode_attn(cache, q, q_slot, out, lse, ws, n_q_heads=None, scale=0.0,
                       q_layer_stride=0, out_layer_stride=0, lse_layer_stride=0, stream=None):
    """q: bf16 [nq][nb][Hq][d] (or strided); out float32 like q."""
    c = cache.desc()
    nq = len(q_slot)
    hq = n_q_heads if n_q_heads is not None else q.shape[-2]
    slots = (ctypes.c_int32 * max(1, nq))(*[int(x) for x in q_slot])
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    per = cache.nb * hq * HEAD_DIM
    _on_device(q=q, out=out, lse=lse, ws=ws)
    _check(lib().kvc_q8_decode_attn(ctypes.byref(c),
                                    _arg(q, "q", torch.bfloat16, per, nq, q_layer_stride),
                                    q_layer_stride, nq, slots, hq, float(scale),
                                    _arg(out, "out", torch.float32, per, nq, out_layer_stride),
                                    out_layer_stride,
                                    _arg(lse, "lse", torch.float32, cache.nb * hq, nq,
                                         lse_layer_stride),
                                    lse_layer_stride, _arg(ws, "ws", None, 0), ws_bytes,
                                    _stream(stream)),
           "kvc_q8_decode_attn")


def kvc_xkv_factor_ws_bytes(store):
    x = store.desc()
    out = ctypes.c_size_t()
    _check(lib().kvc_xkv_factor_ws_bytes(ctypes.byref(x), ctypes.byref(out)),
           "kvc_xkv_factor_ws_bytes")
    return out.value


def kvc_xkv_factor(cache, slot0, store, ws, iters=12, seed=0, stream=None):
    """Factorise slots [slot0, slot0 + store.window) of `cache` into `store`
    (sets store.t_len = cache.t_len first)."""
    store.t_len = cache.t_len
    c, x = cache.desc(), store.desc()
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().kvc_xkv_factor(ctypes.byref(c), slot0, iters, int(seed) & (2**64 - 1),
                                ctypes.byref(x), _ptr(ws), ws_bytes, _stream(stream)),
           "kvc_xkv_factor")


def kvc_xkv_decode_ws_bytes(store, n_q_heads, n_select=256):
    x = store.desc()
    out = ctypes.c_size_t()
    _check(lib().kvc_xkv_decode_ws_bytes(ctypes.byref(x), n_q_heads, n_select, ctypes.byref(out)),
           "kvc_xkv_decode_ws_bytes")
    return out.value


def kvc_xkv_decode_attn(store, layer, q, out, lse=None, n_select=256, scale=0.0, o_in=None,
                        lse_in=None, selected=None, n_q_heads=None, ws=None, stream=None):
    """q: bf16 [nb][Hq][d]; out float32 like q (o_in / lse_in: a second part
    to merge, e.g. attention over rows appended after the factorisation);
    ws: kvc_xkv_decode_ws_bytes bytes of device memory, allocated zeroed
    (its arrival counters start at zero; every call leaves them zero)."""
    x = store.desc()
    hq = q.shape[-2] if n_q_heads is None else n_q_heads
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    nb = store.nb
    per = nb * hq * HEAD_DIM
    n_sel = store.nb * store.n_kv_heads * n_select
    _on_device(q=q, o_in=o_in, lse_in=lse_in, out=out, lse=lse, selected=selected, ws=ws)
    _check(lib().kvc_xkv_decode_attn(ctypes.byref(x), layer, _arg(q, "q", torch.bfloat16, per),
                                     hq, float(scale), n_select,
                                     _arg(o_in, "o_in", torch.float32, per),
                                     _arg(lse_in, "lse_in", torch.float32, nb * hq),
                                     _arg(out, "out", torch.float32, per),
                                     _arg(lse, "lse", torch.float32, nb * hq),
                                     _arg(selected, "selected", torch.int32, n_sel),
                                     _arg(ws, "ws", None, 0), ws_bytes, _stream(stream)),
           "kvc_xkv_decode_attn")
