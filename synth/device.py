"""Device-side drawing of the seeded inputs (leaves and codes) into torch
tensors, through libpmsynth.so.  Bit-identical to the host generator in
synth/__init__.py for every slice; used to fill expert pools that are too
large to draw on the host."""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import KIND_CODES, KIND_LEAVES, KIND_POISON, leaf_quantiles, stream_key

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpmsynth.so")


class DeviceSynth:
    def __init__(self, device="cuda"):
        import torch
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run bitplane_quantized_expert_amd/build.py")
        self.torch = torch
        self.lib = ctypes.CDLL(LIB_PATH)
        P, I, U32, U64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint32, ctypes.c_uint64
        self.lib.pmsynth_leaves.argtypes = [U32, U32, I, I, I, P, P, P, P]
        self.lib.pmsynth_codes.argtypes = [U32, U32, I, I, I, P, P]
        self.lib.pmsynth_words.argtypes = [U32, U32, U64, P, P]
        for f in (self.lib.pmsynth_leaves, self.lib.pmsynth_codes, self.lib.pmsynth_words):
            f.restype = I
        q, gap = leaf_quantiles()
        self.q = torch.tensor(q, dtype=torch.float64, device=device)
        self.gap = torch.tensor(gap, dtype=torch.float64, device=device)
        self.device = device

    def _stream(self, stream):
        s = stream if stream is not None else self.torch.cuda.current_stream()
        return s.cuda_stream

    def leaves_into(self, out, seed, cfg, layer, expert, matrix, ngroups, row0, nrows, stream=None):
        k0, k1 = stream_key(seed, KIND_LEAVES, cfg, layer, expert, matrix)
        assert out.numel() >= nrows * ngroups * 256 and out.dtype == self.torch.float32
        rc = self.lib.pmsynth_leaves(k0, k1, ngroups, row0, nrows, self.q.data_ptr(),
                                     self.gap.data_ptr(), out.data_ptr(), self._stream(stream))
        if rc:
            raise RuntimeError(f"pmsynth_leaves failed ({rc})")
        return out

    def codes_into(self, out, seed, cfg, layer, expert, matrix, cols, row0, nrows, stream=None):
        k0, k1 = stream_key(seed, KIND_CODES, cfg, layer, expert, matrix)
        assert out.numel() >= nrows * cols and out.dtype == self.torch.uint8
        rc = self.lib.pmsynth_codes(k0, k1, cols, row0, nrows, out.data_ptr(), self._stream(stream))
        if rc:
            raise RuntimeError(f"pmsynth_codes failed ({rc})")
        return out

    def poison_into(self, out_u32, seed, unit, stream=None):
        """Fill a uint32 view (numel % 4 == 0) with raw stream words."""
        k0, k1 = stream_key(seed, KIND_POISON, 0, 0, unit, 0)
        rc = self.lib.pmsynth_words(k0, k1, out_u32.numel(), out_u32.data_ptr(), self._stream(stream))
        if rc:
            raise RuntimeError(f"pmsynth_words failed ({rc})")
        return out_u32
