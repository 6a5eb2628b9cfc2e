"""Python binding of libkvcodec (include/kvcodec.h): argument marshalling only.

Every function has the C entry point's name. Device buffers are torch
tensors on the GPU (contiguous; bf16 tensors for K/V, uint8 for pools and
cards); the work is enqueued on `stream` (a torch.cuda.Stream, a raw
hipStream_t integer, or None for torch's current stream). Errors from the
library raise KvcError. If libkvcodec.so is missing the import fails: there
is no fallback path.
"""

import ctypes
import os

import numpy as np
# torch first: it ships its own HIP runtime (SONAME libamdhip64.so.7) and
# names it by file name, so if libkvcodec.so were loaded first the process
# would hold two HIP runtimes and our launches would not see torch's memory
# or streams. Loaded in this order, libkvcodec binds to torch's runtime.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvcodec.so")

KVC_OK = 0
KVC_E_NULL, KVC_E_SHAPE, KVC_E_SIZE, KVC_E_ALIGN = -1, -2, -3, -4
KVC_E_ALIAS, KVC_E_FORMAT, KVC_E_RANGE, KVC_E_HIP, KVC_E_SCRATCH = -5, -6, -7, -8, -9
KVC_DEV_BAD_HEADER, KVC_DEV_BAD_WIDTH, KVC_DEV_CAPACITY = 1, 2, 4
KVC_DEV_ENCODE_TIMEOUT = 8
KVC_MAX_AGENTS = 64


class KvcError(RuntimeError):
    def __init__(self, code, what):
        super().__init__(f"{what}: {kvc_strerror(code)} ({code})")
        self.code = code


class kvc_shape(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_uint32), ("num_kv_heads", ctypes.c_uint32),
                ("num_tokens", ctypes.c_uint32), ("head_dim", ctypes.c_uint32)]


class kvc_card_meta(ctypes.Structure):
    _fields_ = [("model_id", ctypes.c_char * 64), ("position_offset", ctypes.c_int64),
                ("group_size", ctypes.c_uint32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "(hipcc --offload-arch=gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    sz, i32, u32, p = ctypes.c_size_t, ctypes.c_int, ctypes.c_uint32, ctypes.c_void_p
    sp = ctypes.POINTER(kvc_shape)
    sig = {
        "kvpool_bytes": (sz, [sp]),
        "kvpool_workspace_bytes": (sz, [sp]),
        "kvpool_encode": (i32, [sp, p, p, p, sz, p, sz, p, p]),
        "kvpool_encode_noalloc": (i32, [sp, p, p, p, sz, p, p]),
        "kvpool_decode": (i32, [sp, p, sz, u32, u32, ctypes.POINTER(p), ctypes.POINTER(p), u32, p, p]),
        "cachecard_record_bytes": (sz, [u32, u32]),
        "cachecard_max_bytes": (sz, [sp]),
        "cachecard_bytes_host": (sz, [sp, p]),
        "cachecard_workspace_bytes": (sz, [sp]),
        "cachecard_pack": (i32, [sp, p, p, p, ctypes.POINTER(kvc_card_meta), p, sz, p, p, p, sz, p]),
        "cachecard_unpack": (i32, [sp, p, sz, p, p, p, p, sz, p]),
        "cachecard_transcode_workspace_bytes": (sz, [sp]),
        "cachecard_transcode": (i32, [sp, p, sz, p, p, sz, p, p, p, sz, p]),
        "kvc_realign_keys": (i32, [sp, p, p, ctypes.c_int64, p, u32, p]),
        "kvc_lowrank_materialize": (i32, [sp, u32, u32, p, p, p, p, p, p]),
        "kvc_lowrank_factor_workspace_bytes": (sz, [sp, u32]),
        "kvc_lowrank_factor": (i32, [sp, u32, p, p, p, ctypes.c_uint64, p, ctypes.c_uint64, p, p, sz, p]),
        "kvc_parse_header": (i32, [p, sz, sp, ctypes.POINTER(u32)]),
        "kvc_strerror": (ctypes.c_char_p, [i32]),
        "kvc_codebook": (None, [p, p]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()
EXPORTED = ("kvpool_bytes", "kvpool_workspace_bytes", "kvpool_encode", "kvpool_encode_noalloc", "kvpool_decode",
            "cachecard_record_bytes", "cachecard_max_bytes", "cachecard_bytes_host",
            "cachecard_workspace_bytes", "cachecard_pack", "cachecard_unpack",
            "cachecard_transcode_workspace_bytes", "cachecard_transcode", "kvc_realign_keys",
            "kvc_lowrank_materialize", "kvc_lowrank_factor_workspace_bytes", "kvc_lowrank_factor",
            "kvc_parse_header",
            "kvc_strerror", "kvc_codebook")


def library():
    return _lib


def _shape(shape):
    if isinstance(shape, kvc_shape):
        return shape
    L, H, T, d = (int(x) for x in shape)
    return kvc_shape(L, H, T, d)


def _ptr(t):
    """Device address of a torch tensor (or None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a GPU tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr())


def _nbytes(t):
    return t.numel() * t.element_size()


def _want(t, dtype, numel, what):
    """Argument check before any device work: a GPU tensor of this dtype
    and element count (numel None: any count), contiguous."""
    if t is None:
        raise ValueError(f"{what}: tensor required")
    if t.dtype != dtype:
        raise ValueError(f"{what}: expected {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{what}: expected {numel} elements, got {t.numel()}")
    return _ptr(t)


def _kv_numel(shape, layers=None):
    L, H, T, d = (int(x) for x in shape)
    return (L if layers is None else layers) * H * T * d


def _opt(t, dtype, numel, what):
    return None if t is None else _want(t, dtype, numel, what)


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(rc, what):
    if rc != KVC_OK:
        raise KvcError(rc, what)


def kvc_strerror(code):
    return _lib.kvc_strerror(int(code)).decode()


# ------------------------------------------------------------------ pool mode

def kvpool_bytes(shape):
    return int(_lib.kvpool_bytes(ctypes.byref(_shape(shape))))


def kvpool_workspace_bytes(shape):
    return int(_lib.kvpool_workspace_bytes(ctypes.byref(_shape(shape))))


def kvpool_encode(shape, k, v, pool, ws, dev_status=None, stream=None):
    """k, v: bf16 [L, H, T, d]; pool, ws: uint8 device buffers (ws zeroed
    before its first use, e.g. torch.zeros); dev_status: int32 device
    tensor of 1 element or None."""
    n = _kv_numel(shape)
    args = (_want(k, torch.bfloat16, n, "k"), _want(v, torch.bfloat16, n, "v"),
            _want(pool, torch.uint8, None, "pool"))
    wsp, st = _want(ws, torch.uint8, None, "ws"), _opt(dev_status, torch.int32, 1, "dev_status")
    _check(_lib.kvpool_encode(ctypes.byref(_shape(shape)), *args, _nbytes(pool), wsp, _nbytes(ws), st,
                              _stream(stream)), "kvpool_encode")


def kvpool_encode_noalloc(shape, k, v, pool, dev_status=None, stream=None):
    """kvpool_encode with the library's own per-GPU scratch as workspace
    (no allocation anywhere in the call)."""
    n = _kv_numel(shape)
    args = (_want(k, torch.bfloat16, n, "k"), _want(v, torch.bfloat16, n, "v"),
            _want(pool, torch.uint8, None, "pool"))
    _check(_lib.kvpool_encode_noalloc(ctypes.byref(_shape(shape)), *args, _nbytes(pool),
                                      _opt(dev_status, torch.int32, 1, "dev_status"), _stream(stream)),
           "kvpool_encode_noalloc")


def kvpool_decode(shape, pool, layer_begin, layer_end, k_outs, v_outs, dev_status=None, stream=None):
    """k_outs, v_outs: lists of bf16 [layer_end-layer_begin, H, T, d] tensors
    (one pair per agent); dev_status: int32 device tensor of 1 element or None."""
    n = len(k_outs)
    if len(v_outs) != n:
        raise ValueError("k_outs and v_outs must have the same length")
    m = _kv_numel(shape, max(int(layer_end) - int(layer_begin), 0))
    for i, t in enumerate(list(k_outs) + list(v_outs)):
        _want(t, torch.bfloat16, m, f"decode output {i}")
    karr = (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in k_outs])
    varr = (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in v_outs])
    _check(_lib.kvpool_decode(ctypes.byref(_shape(shape)), _want(pool, torch.uint8, None, "pool"), _nbytes(pool),
                              int(layer_begin), int(layer_end), karr, varr, n,
                              _opt(dev_status, torch.int32, 1, "dev_status"), _stream(stream)),
           "kvpool_decode")


# ------------------------------------------------------------------ CacheCard mode

def cachecard_record_bytes(head_dim, bits):
    return int(_lib.cachecard_record_bytes(int(head_dim), int(bits)))


def cachecard_max_bytes(shape):
    return int(_lib.cachecard_max_bytes(ctypes.byref(_shape(shape))))


def cachecard_bytes_host(shape, widths_host):
    w = np.ascontiguousarray(widths_host, np.uint8)
    return int(_lib.cachecard_bytes_host(ctypes.byref(_shape(shape)), w.ctypes.data_as(ctypes.c_void_p)))


def cachecard_workspace_bytes(shape):
    return int(_lib.cachecard_workspace_bytes(ctypes.byref(_shape(shape))))


def cachecard_pack(shape, k, v, widths, card, ws, model_id=b"", position_offset=0,
                   dev_card_bytes=None, dev_status=None, stream=None):
    """widths: uint8 [T] device tensor; card, ws: uint8 device buffers;
    dev_card_bytes: int64 device tensor of 1 element or None."""
    meta = kvc_card_meta()
    mid = model_id.encode() if isinstance(model_id, str) else bytes(model_id)
    meta.model_id = mid[:63]
    meta.position_offset = int(position_offset)
    meta.group_size = 32
    n = _kv_numel(shape)
    args = (_want(k, torch.bfloat16, n, "k"), _want(v, torch.bfloat16, n, "v"),
            _want(widths, torch.uint8, int(shape[2]), "widths"))
    _check(_lib.cachecard_pack(ctypes.byref(_shape(shape)), *args, ctypes.byref(meta),
                               _want(card, torch.uint8, None, "card"), _nbytes(card),
                               _opt(dev_card_bytes, torch.int64, 1, "dev_card_bytes"),
                               _opt(dev_status, torch.int32, 1, "dev_status"), _want(ws, torch.uint8, None, "ws"),
                               _nbytes(ws), _stream(stream)), "cachecard_pack")


def cachecard_unpack(shape, card, k_out, v_out, ws, card_bytes=None, dev_status=None, stream=None):
    n = _nbytes(card) if card_bytes is None else int(card_bytes)
    if n > _nbytes(card):
        raise ValueError("card_bytes exceeds the card tensor")
    m = _kv_numel(shape)
    _check(_lib.cachecard_unpack(ctypes.byref(_shape(shape)), _want(card, torch.uint8, None, "card"), n,
                                 _want(k_out, torch.bfloat16, m, "k_out"), _want(v_out, torch.bfloat16, m, "v_out"),
                                 _opt(dev_status, torch.int32, 1, "dev_status"), _want(ws, torch.uint8, None, "ws"),
                                 _nbytes(ws), _stream(stream)), "cachecard_unpack")


def cachecard_transcode_workspace_bytes(shape):
    return int(_lib.cachecard_transcode_workspace_bytes(ctypes.byref(_shape(shape))))


def cachecard_transcode(shape, card_in, new_widths, card_out, ws, card_in_bytes=None, dev_card_bytes=None,
                        dev_status=None, stream=None):
    """card_in, card_out, ws: uint8 device buffers; new_widths: uint8 [T]
    device tensor; dev_card_bytes: int64 device tensor of 1 element or None."""
    n = _nbytes(card_in) if card_in_bytes is None else int(card_in_bytes)
    if n > _nbytes(card_in):
        raise ValueError("card_in_bytes exceeds the card_in tensor")
    _check(_lib.cachecard_transcode(ctypes.byref(_shape(shape)), _want(card_in, torch.uint8, None, "card_in"), n,
                                    _want(new_widths, torch.uint8, int(shape[2]), "new_widths"),
                                    _want(card_out, torch.uint8, None, "card_out"), _nbytes(card_out),
                                    _opt(dev_card_bytes, torch.int64, 1, "dev_card_bytes"),
                                    _opt(dev_status, torch.int32, 1, "dev_status"),
                                    _want(ws, torch.uint8, None, "ws"), _nbytes(ws), _stream(stream)),
           "cachecard_transcode")


KVC_ROPE_HALVES, KVC_ROPE_ADJACENT = 0, 1


def kvc_realign_keys(shape, k_in, k_out, delta, inv_freq, pairing=KVC_ROPE_HALVES, stream=None):
    """k_in, k_out: bf16 device tensors [L, H, T, d] (the same tensor for in
    place); inv_freq: d/2 host floats."""
    f = np.ascontiguousarray(inv_freq, np.float32)
    if f.size != shape[3] // 2:
        raise ValueError("inv_freq must hold d/2 values")
    n = _kv_numel(shape)
    _want(k_in, torch.bfloat16, n, "k_in")
    _want(k_out, torch.bfloat16, n, "k_out")
    _check(_lib.kvc_realign_keys(ctypes.byref(_shape(shape)), _ptr(k_in), _ptr(k_out), int(delta),
                                 f.ctypes.data_as(ctypes.c_void_p), int(pairing), _stream(stream)),
           "kvc_realign_keys")


def kvc_lowrank_materialize(shape, rank, n_anchors, src, a, r, weights, out, stream=None):
    """src, out: bf16 device tensors [L, H, T, d] (the same tensor for in
    place); a: bf16 [L, V, T, rank]; r: bf16 [L, V, H*d, rank]; weights:
    float32 device tensor [L, V]."""
    L, H, T, d = (int(x) for x in shape)
    V, r_ = int(n_anchors), int(rank)
    _want(src, torch.bfloat16, _kv_numel(shape), "src")
    _want(out, torch.bfloat16, _kv_numel(shape), "out")
    _want(a, torch.bfloat16, L * V * T * r_, "a")
    _want(r, torch.bfloat16, L * V * H * d * r_, "r")
    _want(weights, torch.float32, L * V, "weights")
    _check(_lib.kvc_lowrank_materialize(ctypes.byref(_shape(shape)), int(rank), int(n_anchors), _ptr(src),
                                        _ptr(a), _ptr(r), _ptr(weights), _ptr(out), _stream(stream)),
           "kvc_lowrank_materialize")


LOWRANK_SKETCH = 48


def kvc_lowrank_factor_workspace_bytes(shape, rank=32):
    return int(_lib.kvc_lowrank_factor_workspace_bytes(ctypes.byref(_shape(shape)), int(rank)))


def kvc_lowrank_factor(shape, rank, z, omega, a_out, r_out, ws, a_stride=None, r_stride=None, sigma_out=None,
                       stream=None):
    """z: bf16 device tensor [L, H, T, d]; omega: float32 device tensor
    [H*d, 48]; a_out / r_out: bf16 device tensors holding A (T x rank) and R
    (H*d x rank) of matrix l at element offset l * a_stride / l * r_stride
    (defaults: packed); ws: device bytes; sigma_out: float32 [L, rank] or
    None."""
    L, H, T, d = shape
    a_stride = T * rank if a_stride is None else a_stride
    r_stride = H * d * rank if r_stride is None else r_stride

    def base(t, row):
        # a view of strided outputs (e.g. anchor v of [L][V][T][r]): its own
        # rows must be contiguous; the layer stride is the explicit argument
        if not t.is_cuda:
            raise ValueError("expected a GPU tensor")
        if t.dim() != 3 or t.shape[0] != L or t.shape[2] != rank or t.stride(2) != 1 or t.stride(1) != rank \
                or t.shape[1] != row:
            raise ValueError("expected a [L, rows, rank] view with contiguous rows")
        return ctypes.c_void_p(t.data_ptr())

    _want(z, torch.bfloat16, _kv_numel(shape), "z")
    _want(omega, torch.float32, H * d * LOWRANK_SKETCH, "omega")
    _want(ws, torch.uint8, None, "ws")
    _opt(sigma_out, torch.float32, L * rank, "sigma_out")
    if a_out.dtype != torch.bfloat16 or r_out.dtype != torch.bfloat16:
        raise ValueError("a_out and r_out must be bfloat16")
    a_ptr, r_ptr = base(a_out, T), base(r_out, H * d)
    if L > 1 and (a_out.stride(0) != a_stride or r_out.stride(0) != r_stride):
        raise ValueError("layer strides of the views differ from a_stride / r_stride")
    _check(_lib.kvc_lowrank_factor(ctypes.byref(_shape(shape)), int(rank), _ptr(z), _ptr(omega), a_ptr,
                                   int(a_stride), r_ptr, int(r_stride), _ptr(sigma_out), _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream(stream)),
           "kvc_lowrank_factor")


# ------------------------------------------------------------------ host utils

def kvc_parse_header(host_bytes):
    """bytes-like header -> ((L, H, T, d), kind) with kind 1 = pool, 2 = card."""
    b = np.frombuffer(bytes(host_bytes), np.uint8)
    s = kvc_shape()
    kind = ctypes.c_uint32()
    _check(_lib.kvc_parse_header(b.ctypes.data_as(ctypes.c_void_p), b.size, ctypes.byref(s), ctypes.byref(kind)),
           "kvc_parse_header")
    return (s.num_layers, s.num_kv_heads, s.num_tokens, s.head_dim), int(kind.value)


def kvc_codebook():
    lv = np.zeros(8, np.float32)
    th = np.zeros(7, np.float32)
    _lib.kvc_codebook(lv.ctypes.data_as(ctypes.c_void_p), th.ctypes.data_as(ctypes.c_void_p))
    return lv, th


# ------------------------------------------------------------------ object wrappers

class SharedKVPool:
    """The shared pool of the write-once, read-many cache (PolyKV §2.A: the
    shared document's K/V compressed once into one object that every agent
    decodes layer by layer into its own cache). Holds the pool bytes and
    the shape; allocates buffers on the inputs' device and calls
    kvpool_encode / kvpool_decode on torch's current stream."""

    def __init__(self, shape, pool):
        self.shape = tuple(int(x) for x in shape)
        self.pool = pool

    @classmethod
    def encode(cls, k, v, ws=None, dev_status=None):
        """k, v: bf16 [L, H, T, d] device tensors. ws: a zeroed workspace to
        reuse across encodes, or None for a new one."""
        shape = tuple(k.shape)
        pool = torch.empty(kvpool_bytes(shape), dtype=torch.uint8, device=k.device)
        if ws is None:
            ws = torch.zeros(kvpool_workspace_bytes(shape), dtype=torch.uint8, device=k.device)
        kvpool_encode(shape, k, v, pool, ws, dev_status)
        return cls(shape, pool)

    def decode_layers(self, layer_begin=0, layer_end=None, k_outs=None, v_outs=None, n_agents=1, dev_status=None):
        """Layers [layer_begin, layer_end) into each agent's K and V buffers
        (new bf16 tensors for n_agents agents when k_outs / v_outs are None);
        returns (k_outs, v_outs)."""
        L, H, T, d = self.shape
        layer_end = L if layer_end is None else int(layer_end)
        n = max(layer_end - int(layer_begin), 0)
        if k_outs is None:
            k_outs = [torch.empty((n, H, T, d), dtype=torch.bfloat16, device=self.pool.device) for _ in range(n_agents)]
        if v_outs is None:
            v_outs = [torch.empty((n, H, T, d), dtype=torch.bfloat16, device=self.pool.device) for _ in range(n_agents)]
        kvpool_decode(self.shape, self.pool, layer_begin, layer_end, k_outs, v_outs, dev_status)
        return k_outs, v_outs


class CacheCard:
    """A CacheCard (QKVShare: quantised groups, per-token widths and
    metadata in one buffer). Holds the card bytes, their exact size and the
    shape; allocates buffers on the inputs' device and calls
    cachecard_pack / cachecard_unpack / cachecard_transcode on torch's
    current stream. Data errors (a width outside {2, 4, 8, 16}, a refused
    header) land in the status word, read by status()."""

    def __init__(self, shape, card, nbytes, dev_status):
        self.shape = tuple(int(x) for x in shape)
        self.card = card
        self.nbytes = int(nbytes)
        self.dev_status = dev_status

    @staticmethod
    def _widths(widths, device, T):
        w_host = widths.cpu().numpy() if isinstance(widths, torch.Tensor) else np.asarray(widths, np.uint8)
        w_host = np.ascontiguousarray(w_host, np.uint8).reshape(-1)
        if w_host.size != T:
            raise ValueError(f"widths: expected {T} values, got {w_host.size}")
        return w_host, torch.from_numpy(w_host).to(device)

    @classmethod
    def pack(cls, k, v, widths, model_id=b"", position_offset=0):
        """k, v: bf16 [L, H, T, d] device tensors; widths: T values in
        {2, 4, 8, 16} (host array or tensor)."""
        shape = tuple(k.shape)
        w_host, w_dev = cls._widths(widths, k.device, shape[2])
        n = cachecard_bytes_host(shape, w_host)
        card = torch.empty(max(n, 1), dtype=torch.uint8, device=k.device)
        ws = torch.empty(cachecard_workspace_bytes(shape), dtype=torch.uint8, device=k.device)
        status = torch.zeros(1, dtype=torch.int32, device=k.device)
        cachecard_pack(shape, k, v, w_dev, card, ws, model_id, position_offset, None, status)
        return cls(shape, card, n, status)

    def unpack(self, k_out=None, v_out=None):
        """Full-width bf16 K and V (new tensors when k_out / v_out are None)."""
        dev = self.card.device
        if k_out is None:
            k_out = torch.empty(self.shape, dtype=torch.bfloat16, device=dev)
        if v_out is None:
            v_out = torch.empty(self.shape, dtype=torch.bfloat16, device=dev)
        ws = torch.empty(cachecard_workspace_bytes(self.shape), dtype=torch.uint8, device=dev)
        cachecard_unpack(self.shape, self.card, k_out, v_out, ws, self.nbytes, self.dev_status)
        return k_out, v_out

    def transcode(self, new_widths):
        """The card at new per-token widths (one hop), as a new CacheCard."""
        dev = self.card.device
        w_host, w_dev = self._widths(new_widths, dev, self.shape[2])
        n = cachecard_bytes_host(self.shape, w_host)
        card = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
        ws = torch.empty(cachecard_transcode_workspace_bytes(self.shape), dtype=torch.uint8, device=dev)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        cachecard_transcode(self.shape, self.card, w_dev, card, ws, self.nbytes, None, status)
        return CacheCard(self.shape, card, n, status)

    def status(self):
        """The card's device status word (synchronises): 0, or KVC_DEV_* bits."""
        return int(self.dev_status.item())
