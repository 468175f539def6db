"""A multi-layer VBR cache: layers start at the top of a codec ladder and
are moved down, one layer one rung at a time, whenever the cache would no
longer fit its byte budget (VBR announcement thread, opening posts).

The plan comes from the library's controller (``kvq_vbr_plan``); every step
is carried out on the device with ``kvq_transcode_layer`` into a new layer
that shares the old one's binary16 tail, after which the old planes are
released.  Appending tokens (generated or injected) is what pushes degrades.
"""

from . import lib
from .cache import LayerCache, PlaneSpec


class VBRCache:
    def __init__(self, n_layers, batch, n_kv_heads, capacity, tail_len, ladder, floor, order,
                 budget_bytes, device="cuda"):
        self.ladder, self.floor = list(ladder), floor
        self.policy = lib.vbr_policy(ladder, floor, order, batch, n_kv_heads, tail_len, budget_bytes)
        self.level = [0] * n_layers
        self.layers = [LayerCache(batch, n_kv_heads, capacity, tail_len, PlaneSpec(ladder[0]),
                                  PlaneSpec(ladder[0]), device) for _ in range(n_layers)]
        self.history = []          # (n_tokens, layer, from codec, to codec)

    @property
    def n_tokens(self):
        return self.layers[0].n_tokens

    def codec(self, layer):
        return self.ladder[self.level[layer]]

    def bytes(self, n_tokens=None):
        return lib.vbr_bytes(self.policy, self.level, self.n_tokens if n_tokens is None else n_tokens)

    def fit(self, n_tokens, stream=None):
        """Degrade as needed so that n_tokens fit; returns the steps taken.
        Raises KvqError (KVQ_ERR_CAPACITY) when even the floor does not fit."""
        status, level, steps = lib.vbr_plan(self.policy, n_tokens, self.level)
        for (layer, src, dst) in steps:
            old = self.layers[layer]
            new = LayerCache(old.batch, old.n_kv_heads, old.capacity, old.tail_len,
                             PlaneSpec(dst), PlaneSpec(dst), old.device, share_tail_with=old,
                             tail_format=old.tail_format)
            old.transcode_into(new, stream=stream)
            self.layers[layer] = new
            self.history.append((n_tokens, layer, src, dst))
        self.level = level
        lib.check(status)
        return steps

    def append(self, layer, k_new, v_new, stream=None):
        """Append to one layer (call fit() for the new token count first)."""
        self.layers[layer].append(k_new, v_new, stream=stream)
