"""Python binding of libkvq: decode attention over a rotated, 2/4-bit quantized, paged KV cache.

Argument marshalling only: every step of the write and decode paths runs in the HIP kernels of
libkvq.so (see include/kvq.h for the operations, layouts and error behaviour).  The functions take
torch tensors (device memory and streams) and pass their pointers through the C ABI.  There is no
CPU fallback: importing this package fails if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
# KVQ_LIBRARY may name another build of the same library (for side-by-side timing of two builds);
# by default the in-tree libkvq.so is loaded.
LIB_PATH = os.environ.get("KVQ_LIBRARY") or os.path.join(HERE, "libkvq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")

# torch ships its own HIP runtime (libamdhip64.so.7).  Load it before libkvq.so so that the library's
# dependency on that soname resolves to the same runtime: a second HIP runtime in the process would
# not know torch's device memory, streams or device initialisation.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

# enums (include/kvq.h)
KVQ_OK, KVQ_EINVAL, KVQ_ERANGE, KVQ_ENOSPACE, KVQ_EUNSUPPORTED, KVQ_EDEVICE = 0, -1, -2, -3, -4, -5
INT2_CHANNEL, INT4_TOKEN, INT2_TOKEN, INT4_CHANNEL = 0, 1, 2, 3
F32, BF16 = 0, 1
ROT_DENSE, ROT_HADAMARD = 0, 1
DECODE_AUTO, DECODE_F32, DECODE_MFMA = 0, 1, 2
STAGE_QPREP, STAGE_SPLITK, STAGE_MERGE, STAGE_ALL = 1, 2, 4, 7


class Config(ctypes.Structure):
    _fields_ = [
        ("head_dim", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("scheme", ctypes.c_int32), ("rotation", ctypes.c_int32), ("page_tokens", ctypes.c_int32),
        ("group_tokens", ctypes.c_int32), ("n_sink", ctypes.c_int32), ("n_recent", ctypes.c_int32),
        ("clip_k", ctypes.c_float), ("clip_v", ctypes.c_float), ("split_tokens", ctypes.c_int32),
        ("decode_impl", ctypes.c_int32), ("key_only_rotation", ctypes.c_int32), ("hadamard_block", ctypes.c_int32),
    ]


class Cache(ctypes.Structure):
    _fields_ = [
        ("pages", ctypes.c_void_p), ("n_pages", ctypes.c_int64), ("band", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p), ("max_pages_per_seq", ctypes.c_int32), ("seq_lens", ctypes.c_void_p),
        ("rot_k", ctypes.c_void_p), ("rot_v", ctypes.c_void_p), ("batch", ctypes.c_int32),
    ]


_P = ctypes.c_void_p
_CFG = ctypes.POINTER(Config)
_CACHE = ctypes.POINTER(Cache)


def _sig(name, res, *args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_lib_page_bytes = _sig("kvq_page_bytes", ctypes.c_size_t, _CFG)
_lib_band_slots = _sig("kvq_band_slots", ctypes.c_int32, _CFG)
_lib_band_bytes = _sig("kvq_band_bytes", ctypes.c_size_t, _CFG, ctypes.c_int32)
_lib_pages_for_len = _sig("kvq_pages_for_len", ctypes.c_int32, _CFG, ctypes.c_int32)
_lib_ws_bytes = _sig("kvq_decode_workspace_bytes", ctypes.c_size_t, _CFG, ctypes.c_int32, ctypes.c_int32)
_lib_bpe = _sig("kvq_bits_per_element", ctypes.c_double, _CFG, ctypes.c_int64)
_lib_check = _sig("kvq_check_config", ctypes.c_int, _CFG)
_lib_build_oscar = _sig("kvq_build_oscar_rotation", ctypes.c_int, _P, _P)
_lib_compose_oscar = _sig("kvq_compose_oscar_rotation", ctypes.c_int, _P, _P)
_lib_build_hadamard = _sig("kvq_build_hadamard_rotation", ctypes.c_int, _P, _P)
_lib_prefill_ws = _sig("kvq_prefill_workspace_bytes", ctypes.c_size_t, _CFG, ctypes.c_int32)
_lib_prefill = _sig("kv_prefill_attn", ctypes.c_int, _CFG, _CACHE, _P, ctypes.c_int32, _P, ctypes.c_int32,
                    ctypes.c_int32, _P, _P, ctypes.c_size_t, _P)
_lib_query_cov = _sig("kvq_query_covariance", ctypes.c_int, _P, ctypes.c_int64, _P)
_lib_sv_cov = _sig("kvq_score_value_covariance", ctypes.c_int, _P, ctypes.c_int64, _P, ctypes.c_int64, _P)
_lib_eigenbasis = _sig("kvq_eigenbasis", ctypes.c_int, _P, _P, _P)
_lib_oscar_from_cov = _sig("kvq_build_oscar_rotation_from_covariance", ctypes.c_int, _P, _P)
_lib_write = _sig("kv_rotate_quant_write", ctypes.c_int, _CFG, _CACHE, _P, _P, ctypes.c_int32, _P, ctypes.c_int32,
                  ctypes.c_int32, _P)
_lib_build_pt = _sig("kvq_build_page_table", ctypes.c_int, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                     ctypes.c_uint64, _P)
_lib_check_pt = _sig("kvq_check_page_table", ctypes.c_int, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64)
_lib_debug_unpack = _sig("kvq_debug_unpack", ctypes.c_int, _CFG, _CACHE, ctypes.c_int32, ctypes.c_int32,
                         ctypes.c_int32, _P, _P, _P)
_lib_decode = _sig("kv_decode_attn", ctypes.c_int, _CFG, _CACHE, _P, ctypes.c_int32, _P, ctypes.c_int32, _P,
                   ctypes.c_size_t, _P)
class DecodeShape(ctypes.Structure):
    _fields_ = [("chunk_units", ctypes.c_int32), ("n_chunks", ctypes.c_int32), ("walks", ctypes.c_int32),
                ("span", ctypes.c_int32),
                ("splitk_workgroups", ctypes.c_int32), ("band_first", ctypes.c_int32),
                ("matrix_cores", ctypes.c_int32), ("balanced", ctypes.c_int32), ("max_chunks", ctypes.c_int32)]


_lib_decode_shape = _sig("kvq_decode_shape_of", ctypes.c_int, _CFG, ctypes.c_int32, ctypes.c_int32,
                         ctypes.POINTER(DecodeShape))
_lib_decode_noalloc = _sig("kv_decode_attn_noalloc", ctypes.c_int, _CFG, _CACHE, _P, ctypes.c_int32, _P,
                           ctypes.c_int32, _P)
NOALLOC_SCRATCH_BYTES = 64 << 20
_lib_decode_timed = _sig("kv_decode_attn_timed", ctypes.c_int, _CFG, _CACHE, _P, ctypes.c_int32, _P, ctypes.c_int32,
                         _P, ctypes.c_size_t, _P, _P, _P)
_lib_read_probe = _sig("kvq_read_probe", ctypes.c_int, _CFG, _CACHE, _P, ctypes.c_int32, _P)
_lib_decode_stages = _sig("kv_decode_attn_stages", ctypes.c_int, _CFG, _CACHE, _P, ctypes.c_int32, _P, ctypes.c_int32,
                          _P, ctypes.c_size_t, ctypes.c_int32, _P)
_lib_debug_rotate = _sig("kvq_debug_rotate", ctypes.c_int, _CFG, _CACHE, ctypes.c_int32, _P, ctypes.c_int32,
                         ctypes.c_int32, ctypes.c_float, _P, _P)
_lib_strerror = _sig("kvq_strerror", ctypes.c_char_p, ctypes.c_int)
_lib_version = _sig("kvq_version", ctypes.c_char_p)
_lib_last_error = _sig("kvq_last_error", ctypes.c_char_p)

EXPORTED = [
    "kvq_page_bytes", "kvq_band_slots", "kvq_band_bytes", "kvq_pages_for_len", "kvq_decode_workspace_bytes",
    "kvq_bits_per_element", "kvq_check_config", "kvq_build_oscar_rotation", "kvq_compose_oscar_rotation",
    "kvq_build_hadamard_rotation", "kvq_query_covariance", "kvq_score_value_covariance", "kvq_eigenbasis",
    "kvq_build_oscar_rotation_from_covariance", "kvq_prefill_workspace_bytes", "kv_prefill_attn",
    "kv_rotate_quant_write", "kv_decode_attn", "kv_decode_attn_stages", "kv_decode_attn_noalloc",
    "kv_decode_attn_timed",
    "kvq_decode_shape_of", "kvq_read_probe",
    "kvq_debug_rotate", "kvq_debug_unpack", "kvq_build_page_table", "kvq_check_page_table",
    "kvq_strerror", "kvq_version", "kvq_last_error",
]


class KvqError(RuntimeError):
    def __init__(self, status: int, what: str):
        detail = f" [{last_error()}]" if status == KVQ_EDEVICE else ""
        super().__init__(f"{what}: {strerror(status)} ({status}){detail}")
        self.status = status


def strerror(status: int) -> str:
    return _lib_strerror(status).decode()


def version() -> str:
    return _lib_version().decode()


def last_error() -> str:
    """HIP error text of the last KVQ_EDEVICE failure on this thread ("" if none)."""
    return _lib_last_error().decode()


def _check(status: int, what: str) -> None:
    if status != KVQ_OK:
        raise KvqError(status, what)


def make_config(n_kv_heads: int, n_q_heads: int, scheme: int = INT2_CHANNEL, rotation: int = ROT_DENSE,
                n_sink: int = 4, n_recent: int = 128, clip_k: float = 0.96, clip_v: float = 0.92,
                split_tokens: int = 0, decode_impl: int = DECODE_AUTO, key_only_rotation: bool = False,
                hadamard_block: int = 0) -> Config:
    return Config(128, n_kv_heads, n_q_heads, scheme, rotation, 64, 128, n_sink, n_recent, clip_k, clip_v,
                  split_tokens, decode_impl, int(key_only_rotation), hadamard_block)


def check_config(cfg: Config) -> int:
    return _lib_check(ctypes.byref(cfg))


def page_bytes(cfg: Config) -> int:
    return _lib_page_bytes(ctypes.byref(cfg))


def band_slots(cfg: Config) -> int:
    return _lib_band_slots(ctypes.byref(cfg))


def band_bytes(cfg: Config, batch: int) -> int:
    return _lib_band_bytes(ctypes.byref(cfg), batch)


def pages_for_len(cfg: Config, seq_len: int) -> int:
    return _lib_pages_for_len(ctypes.byref(cfg), seq_len)


def decode_workspace_bytes(cfg: Config, batch: int, max_seq_len: int) -> int:
    return _lib_ws_bytes(ctypes.byref(cfg), batch, max_seq_len)


def bits_per_element(cfg: Config, seq_len: int) -> float:
    return _lib_bpe(ctypes.byref(cfg), seq_len)


def _host_f64(a):
    import numpy as np
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def build_oscar_rotation(gaussian):
    """R = QR(gaussian).Q . H . P_br in fp64 (host)."""
    import numpy as np
    g, gp = _host_f64(gaussian)
    out = np.empty((128, 128), dtype=np.float64)
    _check(_lib_build_oscar(gp, out.ctypes.data_as(ctypes.c_void_p)), "kvq_build_oscar_rotation")
    return out


def compose_oscar_rotation(U):
    import numpy as np
    u, up = _host_f64(U)
    out = np.empty((128, 128), dtype=np.float64)
    _check(_lib_compose_oscar(up, out.ctypes.data_as(ctypes.c_void_p)), "kvq_compose_oscar_rotation")
    return out


def build_hadamard_rotation(sign):
    import numpy as np
    s = np.ascontiguousarray(sign, dtype=np.float32)
    out = np.empty((128, 128), dtype=np.float64)
    _check(_lib_build_hadamard(s.ctypes.data_as(ctypes.c_void_p), out.ctypes.data_as(ctypes.c_void_p)),
           "kvq_build_hadamard_rotation")
    return out


def _vp(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def query_covariance(q):
    """C_Q = (1/N) sum_n q_n^T q_n of query rows q [N][128] (host fp32 in, fp64 [128][128] out)."""
    import numpy as np
    qa = np.ascontiguousarray(q, dtype=np.float32).reshape(-1, 128)
    out = np.empty((128, 128), dtype=np.float64)
    _check(_lib_query_cov(_vp(qa), qa.shape[0], _vp(out)), "kvq_query_covariance")
    return out


def score_value_covariance(v, s):
    """C_S = (1/N) (S V)^T (S V) for values v [n_keys][128] and scores s [N][n_keys]."""
    import numpy as np
    va = np.ascontiguousarray(v, dtype=np.float32).reshape(-1, 128)
    sa = np.ascontiguousarray(s, dtype=np.float32)
    if sa.ndim != 2 or sa.shape[1] != va.shape[0]:
        raise ValueError("scores must be [N][n_keys] with n_keys = len(v)")
    out = np.empty((128, 128), dtype=np.float64)
    _check(_lib_sv_cov(_vp(va), va.shape[0], _vp(sa), sa.shape[0], _vp(out)), "kvq_score_value_covariance")
    return out


def eigenbasis(C):
    """(U, lambda): C = U diag(lambda) U^T, lambda descending, columns sign-fixed (largest entry positive)."""
    import numpy as np
    ca, cp = _host_f64(C)
    if ca.shape != (128, 128):
        raise ValueError("C must be 128 x 128")
    U = np.empty((128, 128), dtype=np.float64)
    lam = np.empty(128, dtype=np.float64)
    _check(_lib_eigenbasis(cp, _vp(U), _vp(lam)), "kvq_eigenbasis")
    return U, lam


def build_oscar_rotation_from_covariance(C):
    """R = U . H . P_br with U the eigenbasis of the covariance C."""
    import numpy as np
    ca, cp = _host_f64(C)
    if ca.shape != (128, 128):
        raise ValueError("C must be 128 x 128")
    out = np.empty((128, 128), dtype=np.float64)
    _check(_lib_oscar_from_cov(cp, _vp(out)), "kvq_build_oscar_rotation_from_covariance")
    return out


# ----------------------------------------------------------------------------- device-side objects


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return BF16
    raise ValueError(f"unsupported dtype {t.dtype}: expected float32 or bfloat16")


@dataclass
class DeviceCache:
    """Device tensors of one layer's cache and the C struct that points at them."""
    cfg: Config
    pages: "object"
    band: "object"
    page_table: "object"
    seq_lens: "object"
    rot_k: "object"
    rot_v: "object"
    batch: int

    def c_struct(self) -> Cache:
        n_pages = self.pages.numel() // max(1, page_bytes(self.cfg))
        return Cache(_ptr(self.pages), n_pages, _ptr(self.band), _ptr(self.page_table), self.page_table.shape[1],
                     _ptr(self.seq_lens), _ptr(self.rot_k), _ptr(self.rot_v), self.batch)


def allocate_cache(cfg: Config, batch: int, page_table, rot_k, rot_v, n_pages: Optional[int] = None,
                   device: str = "cuda") -> DeviceCache:
    """Allocate pages, band and lengths (torch, device) for a page table [batch, max_pages] (int32).
    rot_v may be None under key-only rotation."""
    import torch
    _check(check_config(cfg), "config")
    pt = page_table.to(device=device, dtype=torch.int32).contiguous()
    if n_pages is None:
        n_pages = int(pt.max().item()) + 1 if pt.numel() else 1
    pages = torch.empty(n_pages * page_bytes(cfg), dtype=torch.uint8, device=device)
    nb = band_bytes(cfg, batch)
    band = torch.zeros(max(nb, 2) // 2, dtype=torch.int16, device=device)
    seq_lens = torch.zeros(batch, dtype=torch.int32, device=device)
    rv = None if rot_v is None else rot_v.to(device).float().contiguous()
    return DeviceCache(cfg, pages, band, pt, seq_lens, rot_k.to(device).float().contiguous(), rv, batch)


def kv_rotate_quant_write(cache: DeviceCache, k, v, cu_new, max_new: int, max_len: Optional[int] = None,
                          stream=None) -> None:
    """Append tokens: k, v [total_new, n_kv, 128] (fp32 or bf16), cu_new int32 [batch+1] (device).
    max_len bounds every sequence's length after the append (host); if None it is taken as the longest
    current length plus max_new, read from the device (a synchronizing copy)."""
    assert k.is_contiguous() and v.is_contiguous() and cu_new.is_contiguous()
    assert k.shape == v.shape and k.shape[1:] == (cache.cfg.n_kv_heads, 128)
    assert cu_new.numel() == cache.batch + 1
    if max_len is None:
        max_len = int(cache.seq_lens.max().item()) + int(max_new)
    cs = cache.c_struct()
    _check(_lib_write(ctypes.byref(cache.cfg), ctypes.byref(cs), _ptr(k), _ptr(v), _dtype_code(k), _ptr(cu_new),
                      int(max_new), int(max_len), _stream(stream)), "kv_rotate_quant_write")


def kv_decode_attn(cache: DeviceCache, q, out, max_seq_len: int, workspace, stream=None) -> None:
    """One decode step: q [batch, n_q, 128] (fp32/bf16) -> out fp32 [batch, n_q, 128]."""
    assert q.is_contiguous() and out.is_contiguous() and workspace.is_contiguous()
    assert q.shape == (cache.batch, cache.cfg.n_q_heads, 128) and out.shape == q.shape
    cs = cache.c_struct()
    _check(_lib_decode(ctypes.byref(cache.cfg), ctypes.byref(cs), _ptr(q), _dtype_code(q), _ptr(out),
                       int(max_seq_len), _ptr(workspace), workspace.numel() * workspace.element_size(),
                       _stream(stream)), "kv_decode_attn")


def decode_shape(cfg: Config, batch: int, max_seq_len: int) -> dict:
    """How kv_decode_attn splits a batch of sequences up to max_seq_len tokens (host only)."""
    sh = DecodeShape()
    _check(_lib_decode_shape(ctypes.byref(cfg), int(batch), int(max_seq_len), ctypes.byref(sh)), "decode_shape")
    return {name: int(getattr(sh, name)) for name, _ in DecodeShape._fields_}


def read_probe(cache: DeviceCache, xor_out, max_seq_len: int, stream=None) -> None:
    """The decode's read pattern with no arithmetic: xor_out (uint32-sized int32 [batch, n_kv, slots]) gets the
    XOR of the 32-bit words each walk of the split-K decode reads; slots = walks, or max_chunks under balanced
    chunking."""
    assert xor_out.is_contiguous() and xor_out.element_size() == 4
    shape = decode_shape(cache.cfg, cache.batch, max_seq_len)
    slots = shape["max_chunks"] if shape["balanced"] else shape["walks"]
    assert xor_out.numel() == cache.batch * cache.cfg.n_kv_heads * slots
    cs = cache.c_struct()
    _check(_lib_read_probe(ctypes.byref(cache.cfg), ctypes.byref(cs), _ptr(xor_out), int(max_seq_len),
                           _stream(stream)), "kvq_read_probe")


def kv_decode_attn_noalloc(cache: DeviceCache, q, out, max_seq_len: int, stream=None) -> None:
    """kv_decode_attn with the library's own per-GPU scratch as workspace (no allocation)."""
    assert q.is_contiguous() and out.is_contiguous()
    assert q.shape == (cache.batch, cache.cfg.n_q_heads, 128) and out.shape == q.shape
    cs = cache.c_struct()
    _check(_lib_decode_noalloc(ctypes.byref(cache.cfg), ctypes.byref(cs), _ptr(q), _dtype_code(q), _ptr(out),
                               int(max_seq_len), _stream(stream)), "kv_decode_attn_noalloc")


def kv_decode_attn_stages(cache: DeviceCache, q, out, max_seq_len: int, workspace, stages: int, stream=None) -> None:
    """The decode step limited to some of its kernels (bitmask of STAGE_*), for timing one kernel alone."""
    cs = cache.c_struct()
    _check(_lib_decode_stages(ctypes.byref(cache.cfg), ctypes.byref(cs), _ptr(q), _dtype_code(q), _ptr(out),
                              int(max_seq_len), _ptr(workspace), workspace.numel() * workspace.element_size(),
                              int(stages), _stream(stream)), "kv_decode_attn_stages")


def kv_decode_attn_timed(cache: DeviceCache, q, out, max_seq_len: int, workspace, split_begin, split_end,
                         stream=None) -> None:
    """kv_decode_attn with torch.cuda.Event(enable_timing=True) events that the split-K dispatch records at
    the kernel's start and end.  torch creates an event's HIP event at its first record, so an event never
    recorded before is recorded once here first (a marker on the stream, no device work)."""
    for ev in (split_begin, split_end):
        if not ev.cuda_event:
            ev.record()
    cs = cache.c_struct()
    _check(_lib_decode_timed(ctypes.byref(cache.cfg), ctypes.byref(cs), _ptr(q), _dtype_code(q), _ptr(out),
                             int(max_seq_len), _ptr(workspace), workspace.numel() * workspace.element_size(),
                             split_begin.cuda_event, split_end.cuda_event, _stream(stream)), "kv_decode_attn_timed")


def kvq_debug_rotate(cache: DeviceCache, which: int, x, rho: float, out, stream=None) -> None:
    cs = cache.c_struct()
    _check(_lib_debug_rotate(ctypes.byref(cache.cfg), ctypes.byref(cs), which, _ptr(x), _dtype_code(x),
                             x.shape[0], float(rho), _ptr(out), _stream(stream)), "kvq_debug_rotate")


def build_page_table(batch: int, max_pages_per_seq: int, n_pages: Optional[int] = None, seed: int = 0):
    """[batch, max_pages_per_seq] int32 page table (host numpy) over a pool of n_pages (default: exactly
    batch * max_pages_per_seq): seed 0 the identity layout, else a seeded random permutation of the pool."""
    import numpy as np
    n_pages = batch * max_pages_per_seq if n_pages is None else n_pages
    out = np.empty((batch, max_pages_per_seq), dtype=np.int32)
    _check(_lib_build_pt(int(batch), int(max_pages_per_seq), int(n_pages), int(seed) & (2 ** 64 - 1), _vp(out)),
           "kvq_build_page_table")
    return out


def check_page_table(table, n_pages: int) -> int:
    """Status of a host page table [batch, max_pages_per_seq] against a pool of n_pages (KVQ_OK, KVQ_ERANGE
    for an entry outside the pool, KVQ_EINVAL for a physical page named twice)."""
    import numpy as np
    t = np.ascontiguousarray(table, dtype=np.int32)
    return _lib_check_pt(_vp(t), int(t.shape[0]), int(t.shape[1]), int(n_pages))


def kvq_debug_unpack(cache: DeviceCache, seq: int, kv_head: int, n_tokens: int, stream=None):
    """(codes uint8 [n_tokens, 2, 128], scales/zeros bf16 bits) of one (sequence, kv head), read back from the
    pages by the library (device tensors); see include/kvq.h for the scale/zero layout."""
    import torch
    dev = cache.pages.device
    codes = torch.empty((n_tokens, 2, 128), dtype=torch.uint8, device=dev)
    per_channel = cache.cfg.scheme in (INT2_CHANNEL, INT4_CHANNEL)
    sz = torch.empty(((n_tokens // 128, 2, 2, 128) if per_channel else (n_tokens, 2, 2)), dtype=torch.int16,
                     device=dev)
    cs = cache.c_struct()
    _check(_lib_debug_unpack(ctypes.byref(cache.cfg), ctypes.byref(cs), int(seq), int(kv_head), int(n_tokens),
                             _ptr(codes), _ptr(sz), _stream(stream)), "kvq_debug_unpack")
    return codes, sz


def workspace_for(cfg: Config, batch: int, max_seq_len: int, device: str = "cuda"):
    import torch
    n = decode_workspace_bytes(cfg, batch, max_seq_len)
    if n == 0:
        raise KvqError(KVQ_EINVAL, "decode_workspace_bytes")
    return torch.empty((n + 3) // 4, dtype=torch.float32, device=device)


def prefill_workspace_bytes(cfg: Config, total_q: int) -> int:
    return int(_lib_prefill_ws(ctypes.byref(cfg), int(total_q)))


def kv_prefill_attn(cache: DeviceCache, q, cu_q, max_q: int, out, workspace, stream=None) -> None:
    """Prefill attention of the chunk just written: q [total_q, n_q, 128] (fp32/bf16), cu_q [batch + 1]
    int32 (device) prefix sums of each sequence's chunk length -> out fp32 [total_q, n_q, 128]."""
    assert q.is_contiguous() and out.is_contiguous() and workspace.is_contiguous() and cu_q.is_contiguous()
    assert q.dim() == 3 and q.shape[1:] == (cache.cfg.n_q_heads, 128) and out.shape == q.shape
    cs = cache.c_struct()
    _check(_lib_prefill(ctypes.byref(cache.cfg), ctypes.byref(cs), _ptr(q), _dtype_code(q), _ptr(cu_q), int(q.shape[0]),
                        int(max_q), _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                        _stream(stream)), "kv_prefill_attn")


def prefill_workspace_for(cfg: Config, total_q: int, device: str = "cuda"):
    import torch
    n = prefill_workspace_bytes(cfg, total_q)
    return torch.empty(max(1, (n + 3) // 4), dtype=torch.float32, device=device)
