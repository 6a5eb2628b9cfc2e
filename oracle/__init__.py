"""CPU oracle of the compressed KV-cache codec.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this package. The product path (the HIP library
and its binding) never touches it.

The C part (kvoracle.c) is compiled with gcc into oracle/libkvoracle.so by
build(); the level table comes from codebook.py. All arrays are numpy:
bf16 tensors are carried as their raw uint16 bit patterns.
"""

import ctypes
import os
import subprocess

import numpy as np

from . import codebook

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvoracle.so")
SRC_PATH = os.path.join(_HERE, "kvoracle.c")
CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
          "-std=c99", "-Wall", "-Wextra"]

_lib = None


def build(verbose=False):
    """Compile kvoracle.c with gcc (always recompiles)."""
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc"] + CFLAGS + [SRC_PATH, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        u32, u64, i64, p = ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
        L.or_pool_bytes.restype = u64
        L.or_pool_bytes.argtypes = [u32] * 4
        L.or_pool_layout.restype = ctypes.c_int
        L.or_pool_layout.argtypes = [u32] * 4 + [p]
        L.or_pool_encode.restype = ctypes.c_int
        L.or_pool_encode.argtypes = [u32] * 4 + [p, p, p, p]
        L.or_pool_decode.restype = ctypes.c_int
        L.or_pool_decode.argtypes = [u32] * 4 + [p, u64, u32, u32, p, p, p]
        L.or_pool_v_codes.restype = ctypes.c_int
        L.or_pool_v_codes.argtypes = [u32] * 4 + [p, u64, p]
        L.or_v_encode_vector.restype = None
        L.or_v_encode_vector.argtypes = [p, u32, p, p, p]
        L.or_v_decode_vector.restype = None
        L.or_v_decode_vector.argtypes = [p, ctypes.c_uint16, u32, p, p]
        L.or_pool_near_boundary.restype = ctypes.c_int
        L.or_pool_near_boundary.argtypes = [u32] * 4 + [p, p, p, ctypes.c_double, p]
        L.or_k_layer_absmax.restype = ctypes.c_float
        L.or_k_layer_absmax.argtypes = [p, u64]
        L.or_card_record_bytes.restype = u32
        L.or_card_record_bytes.argtypes = [u32, u32]
        L.or_card_bytes.restype = u64
        L.or_card_bytes.argtypes = [u32] * 4 + [p]
        L.or_card_layout.restype = ctypes.c_int
        L.or_card_layout.argtypes = [u32] * 4 + [p, p]
        L.or_card_pack.restype = ctypes.c_int
        L.or_card_pack.argtypes = [u32] * 4 + [p, p, p, ctypes.c_char_p, i64, p]
        L.or_card_unpack.restype = ctypes.c_int
        L.or_card_unpack.argtypes = [u32] * 4 + [p, u64, p, p]
        L.or_card_dequant.restype = ctypes.c_uint16
        L.or_card_dequant.argtypes = [u32, ctypes.c_uint16, ctypes.c_uint16]
        L.or_realign_keys.restype = ctypes.c_int
        L.or_realign_keys.argtypes = [u32] * 4 + [p, p, i64, p, u32]
        L.or_set_threads.restype = None
        L.or_set_threads.argtypes = [ctypes.c_int]
        L.or_max_threads.restype = ctypes.c_int
        L.or_max_threads.argtypes = []
        L.or_f64_to_bf16.restype = ctypes.c_uint16
        L.or_f64_to_bf16.argtypes = [ctypes.c_double]
        L.or_f32_to_f16.restype = ctypes.c_uint16
        L.or_f32_to_f16.argtypes = [ctypes.c_float]
        L.or_f16_to_f32.restype = ctypes.c_float
        L.or_f16_to_f32.argtypes = [ctypes.c_uint16]
        _lib = L
    return _lib


def set_threads(n):
    lib().or_set_threads(int(n))


def max_threads():
    return int(lib().or_max_threads())


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _table():
    levels, thr = codebook.codec_table()
    return np.asarray(levels, np.float32), np.asarray(thr, np.float32)


def _check_bf16(a, shape):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16 or a.shape != tuple(shape):
        raise ValueError(f"expected uint16 bf16 bits of shape {shape}, got {a.dtype} {a.shape}")
    return a


# ---------------------------------------------------------------- pool mode

def pool_layout(L, H, T, d):
    off = np.zeros(5, np.uint64)
    rc = lib().or_pool_layout(L, H, T, d, _ptr(off))
    if rc:
        raise ValueError("bad pool shape")
    return [int(x) for x in off]


def pool_bytes(L, H, T, d):
    return int(lib().or_pool_bytes(L, H, T, d))


def pool_encode(k, v):
    """k, v: uint16 [L, H, T, d] bf16 bits -> pool bytes (uint8)."""
    L, H, T, d = k.shape
    k = _check_bf16(k, (L, H, T, d))
    v = _check_bf16(v, (L, H, T, d))
    _, thr = _table()
    pool = np.zeros(pool_bytes(L, H, T, d), np.uint8)
    rc = lib().or_pool_encode(L, H, T, d, _ptr(k), _ptr(v), _ptr(thr), _ptr(pool))
    if rc:
        raise ValueError(f"or_pool_encode failed: {rc}")
    return pool


def pool_decode(pool, shape, l0=0, l1=None):
    """Decode layers [l0, l1) -> (k, v) uint16 bf16 bits [l1-l0, H, T, d]."""
    L, H, T, d = shape
    l1 = L if l1 is None else l1
    levels, _ = _table()
    pool = np.ascontiguousarray(pool, np.uint8)
    ko = np.zeros((l1 - l0, H, T, d), np.uint16)
    vo = np.zeros((l1 - l0, H, T, d), np.uint16)
    rc = lib().or_pool_decode(L, H, T, d, _ptr(pool), pool.size, l0, l1, _ptr(levels),
                              _ptr(ko), _ptr(vo))
    if rc:
        raise ValueError(f"or_pool_decode failed: {rc}")
    return ko, vo


def pool_v_codes(pool, shape):
    L, H, T, d = shape
    pool = np.ascontiguousarray(pool, np.uint8)
    codes = np.zeros((L, H, T, d), np.uint8)
    rc = lib().or_pool_v_codes(L, H, T, d, _ptr(pool), pool.size, _ptr(codes))
    if rc:
        raise ValueError(f"or_pool_v_codes failed: {rc}")
    return codes


def v_encode_vector(v):
    """One bf16 vector (uint16 [d]) -> (fp16 scale bits, codes uint8 [d])."""
    v = np.ascontiguousarray(v, np.uint16)
    d = v.size
    _, thr = _table()
    sh = np.zeros(1, np.uint16)
    codes = np.zeros(d, np.uint8)
    lib().or_v_encode_vector(_ptr(v), d, _ptr(thr), _ptr(sh), _ptr(codes))
    return int(sh[0]), codes


def v_decode_vector(codes, scale_bits):
    codes = np.ascontiguousarray(codes, np.uint8)
    levels, _ = _table()
    out = np.zeros(codes.size, np.uint16)
    lib().or_v_decode_vector(_ptr(codes), int(scale_bits), codes.size, _ptr(levels), _ptr(out))
    return out


def pool_near_boundary(k, v, eps=1e-5):
    """(keys, value coordinates) whose encoding decision lies within eps:
    x * 127 / m within eps of a half-integer, z within eps of a threshold."""
    L, H, T, d = k.shape
    k = _check_bf16(k, (L, H, T, d))
    v = _check_bf16(v, (L, H, T, d))
    _, thr = _table()
    out = np.zeros(2, np.uint64)
    rc = lib().or_pool_near_boundary(L, H, T, d, _ptr(k), _ptr(v), _ptr(thr), float(eps), _ptr(out))
    if rc:
        raise ValueError(f"or_pool_near_boundary failed: {rc}")
    return int(out[0]), int(out[1])


def k_layer_absmax(k_layer):
    k_layer = np.ascontiguousarray(k_layer, np.uint16)
    return float(lib().or_k_layer_absmax(_ptr(k_layer), k_layer.size))


# ---------------------------------------------------------------- CacheCard mode

def card_record_bytes(d, b):
    return int(lib().or_card_record_bytes(d, b))


def card_layout(L, H, T, d, widths):
    widths = np.ascontiguousarray(widths, np.uint8)
    off = np.zeros(3, np.uint64)
    rc = lib().or_card_layout(L, H, T, d, _ptr(widths), _ptr(off))
    if rc:
        raise ValueError(f"bad card shape or widths ({rc})")
    return [int(x) for x in off]


def card_bytes(L, H, T, d, widths):
    widths = np.ascontiguousarray(widths, np.uint8)
    return int(lib().or_card_bytes(L, H, T, d, _ptr(widths)))


def card_pack(k, v, widths, model_id=b"", position_offset=0):
    L, H, T, d = k.shape
    k = _check_bf16(k, (L, H, T, d))
    v = _check_bf16(v, (L, H, T, d))
    widths = np.ascontiguousarray(widths, np.uint8)
    n = card_bytes(L, H, T, d, widths)
    if n == 0:
        raise ValueError("bad card shape or widths")
    card = np.zeros(n, np.uint8)
    rc = lib().or_card_pack(L, H, T, d, _ptr(k), _ptr(v), _ptr(widths), model_id,
                            int(position_offset), _ptr(card))
    if rc:
        raise ValueError(f"or_card_pack failed: {rc}")
    return card


def card_unpack(card, shape):
    L, H, T, d = shape
    card = np.ascontiguousarray(card, np.uint8)
    ko = np.zeros((L, H, T, d), np.uint16)
    vo = np.zeros((L, H, T, d), np.uint16)
    rc = lib().or_card_unpack(L, H, T, d, _ptr(card), card.size, _ptr(ko), _ptr(vo))
    if rc:
        raise ValueError(f"or_card_unpack failed: {rc}")
    return ko, vo


def card_dequant(q, scale_f16_bits, min_bf16_bits):
    """One dequantised card value: bf16 bits of q * s + mn rounded once."""
    return int(lib().or_card_dequant(int(q), int(scale_f16_bits), int(min_bf16_bits)))


def card_meta(card):
    """(model ID bytes, position offset) from a card's header."""
    card = np.ascontiguousarray(card, np.uint8)
    model_id = bytes(card[72:136]).split(b"\0", 1)[0]
    position_offset = int.from_bytes(bytes(card[32:40]), "little", signed=True)
    return model_id, position_offset


def card_transcode(card, shape, new_widths):
    """One hop of a handoff chain (QKVShare, problem statement and method:
    each agent passes the cache on as a card at its own per-token widths):
    the card rebuilt to full width, then packed again at new_widths, with
    the model ID and position offset carried over. This is the definition
    itself, written as the composition of unpack and pack."""
    k, v = card_unpack(card, shape)
    model_id, position_offset = card_meta(card)
    return card_pack(k, v, new_widths, model_id, position_offset)


# ---------------------------------------------------------------- key re-alignment

def realign_keys(k, delta, inv_freq, pairing=0):
    """k: uint16 bf16 bits [L, H, T, d]; rotate every channel pair j by
    delta * inv_freq[j] (pairs (j, j + d/2) for pairing 0, (2j, 2j + 1) for
    pairing 1); returns new bf16 bits."""
    L, H, T, d = k.shape
    k = _check_bf16(k, (L, H, T, d))
    f = np.ascontiguousarray(inv_freq, np.float32)
    if f.size != d // 2 or d > 256:
        raise ValueError("inv_freq must hold d/2 values, d <= 256")
    out = np.zeros_like(k)
    rc = lib().or_realign_keys(L, H, T, d, _ptr(k), _ptr(out), int(delta), _ptr(f), int(pairing))
    if rc:
        raise ValueError(f"or_realign_keys failed: {rc}")
    return out


# ---------------------------------------------------------------- scalar formats

def f64_to_bf16(x):
    return int(lib().or_f64_to_bf16(float(x)))


def f32_to_f16(x):
    return int(lib().or_f32_to_f16(float(np.float32(x))))


def f16_to_f32(h):
    return float(lib().or_f16_to_f32(int(h)))
