"""Fill a plane store with seeded synthetic experts on the device: the
device generator draws each matrix's leaves and codes, the library's device
encoder writes the tree levels and bitplanes straight into the store slot.
Harness glue only: the arithmetic is the library's."""
from __future__ import annotations

from . import Workload, matrix_shape
from .device import DeviceSynth


class PoolFiller:
    def __init__(self, wl: Workload, device="cuda"):
        import torch
        import bitplane_quantized_expert_amd as pm
        self.pm = pm
        self.torch = torch
        self.wl = wl
        self.syn = DeviceSynth(device)
        self.e = pm.eshape(wl.hidden, wl.inter, wl.group)
        self.pw = pm.pm_expert_plane_words(self.e)
        n_leaf = max(matrix_shape(wl, m)[0] * (matrix_shape(wl, m)[1] // wl.group) * 256
                     for m in range(3))
        n_code = max(matrix_shape(wl, m)[0] * matrix_shape(wl, m)[1] for m in range(3))
        self.leaf_buf = torch.empty(n_leaf, dtype=torch.float32, device=device)
        self.code_buf = torch.empty(n_code, dtype=torch.uint8, device=device)
        self.offsets = [pm.pm_expert_matrix_offsets(self.e, m) for m in range(3)]

    def fill(self, store, layer, expert, gen_layer=None, gen_expert=None, stream=None):
        """Encode the seeded expert (gen_layer, gen_expert) -- by default the
        slot's own (layer, expert) -- into slot (layer, expert), all planes."""
        pm, wl = self.pm, self.wl
        gl = layer if gen_layer is None else gen_layer
        ge = expert if gen_expert is None else gen_expert
        pp, lp = pm.pm_store_slot(store, layer, expert)
        for m in range(3):
            rows, cols = matrix_shape(wl, m)
            po, lo, sh = self.offsets[m]
            self.syn.leaves_into(self.leaf_buf, wl.seed, wl.cfg, gl, ge, m, cols // wl.group, 0,
                                 rows, stream)
            self.syn.codes_into(self.code_buf, wl.seed, wl.cfg, gl, ge, m, cols, 0, rows, stream)
            pm.pm_encode_matrix_device(sh, self.code_buf, self.leaf_buf, None, pp + 4 * po,
                                       self.pw, lp + 4 * lo, stream)
        pm.pm_store_set_resident(store, layer, expert, 8)
        return pp, lp
