"""Seeded synthetic inputs for the CSA2 layer step.

A module of its own, shared by the HIP path and by the CPU oracle: it draws
random numbers and shapes them like the method's inputs, and holds none of the
method's arithmetic (no quantisation, scoring, selection or attention).

The generator itself is C (``synth.c``, counter-based SplitMix64 + Box-Muller);
this file loads it through ctypes and exposes numpy-returning helpers.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile libsynth.so with gcc (OpenMP, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        u64, i64, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
        for name in ("synth_normal_f32", "synth_uniform_f32", "synth_normal_bf16"):
            getattr(lib, name).argtypes = [u64, u64, u64, i64, vp]
            getattr(lib, name).restype = None
        lib.synth_latent_rows.argtypes = [u64, u64, i64, i64, ctypes.c_int, ctypes.c_int, i64, vp]
        lib.synth_latent_rows.restype = None
        lib.synth_hash.argtypes = [u64, u64, u64]
        lib.synth_hash.restype = u64
        _lib = lib
    return _lib


# tensor kinds: each (kind, layer, sequence) triple is an independent stream
MAIN_LATENT, INDEX_Q, INDEX_W, ATTN_Q, SWA_LATENT, INDEX_PROJ = 1, 3, 4, 5, 6, 7   # tensor kinds


def tensor_id(kind: int, layer: int = 0, seq: int = 0) -> int:
    return (kind << 40) | (layer << 24) | seq


def hash64(seed: int, tensor: int, index: int) -> int:
    return int(_load().synth_hash(seed, tensor, index))


def normal_f32(seed: int, tensor: int, first: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.float32)
    _load().synth_normal_f32(seed, tensor, first, count, out.ctypes.data)
    return out


def uniform_f32(seed: int, tensor: int, first: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.float32)
    _load().synth_uniform_f32(seed, tensor, first, count, out.ctypes.data)
    return out


def normal_bf16_bits(seed: int, tensor: int, first: int, count: int) -> np.ndarray:
    """N(0,1) rounded to bf16 (RNE); returned as the uint16 bit patterns."""
    out = np.empty(count, dtype=np.uint16)
    _load().synth_normal_bf16(seed, tensor, first, count, out.ctypes.data)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def latent_rows(seed: int, tensor: int, row0: int, rows: int, dim: int,
                rope_dims: int = 64, pos_mult: int = 1, out: np.ndarray | None = None) -> np.ndarray:
    """Rows [row0, row0+rows) of an RMS-normalised, rotary-embedded N(0,1) latent."""
    if dim > 4096 or rope_dims > dim or rope_dims % 2:
        raise ValueError("bad latent shape")
    if out is None:
        out = np.empty((rows, dim), dtype=np.float32)
    assert out.dtype == np.float32 and out.flags.c_contiguous and out.size >= rows * dim
    _load().synth_latent_rows(seed, tensor, row0, rows, dim, rope_dims, pos_mult, out.ctypes.data)
    return out
