"""A seeded weights-only model for the decode-token tests (device tensors, and
host copies of the matrices for the oracle)."""
import numpy as np
import torch

import synth
import bit_weight_streaming_q4f16_amd as q4
from gpuhelp import dev_half

EPS = 1e-5


class Weights:
    """Seeded weights of a model with D, F, V and n blocks (host copies kept for
    the oracle when `host`)."""

    def __init__(self, tag, n, D, F, V, host=True):
        self.D, self.F, self.V, self.n = D, F, V, n
        self.mats = {}

        def w(name, N, K, sigma):
            m = synth.Matrix(f"tok/{tag}/{name}", N, K, sigma=sigma, floor=sigma / 4)
            self.mats[name] = m if host else None
            return (m.words_torch("cuda"), dev_half(m.scales()))

        def g(name):
            v = (1.0 + 0.1 * synth.normal(f"tok/{tag}/{name}", 0, 0, D)).astype(np.float16)
            return dev_half(v.view(np.uint16))
        self.embed = w("embed", V, D, 0.05)
        self.lm_head = w("lm_head", V, D, 2.0 / D)
        self.final_norm = g("final_norm")
        self.blocks = [dict(qkv=w(f"{b}/qkv", 3 * D, D, 2.0 / D), o=w(f"{b}/o", D, D, 2.0 / D),
                            gate_up=w(f"{b}/gate_up", 2 * F, D, 2.0 / D),
                            down=w(f"{b}/down", D, F, 2.0 / F),
                            attn_norm=g(f"{b}/attn_norm"), ffn_norm=g(f"{b}/ffn_norm"))
                       for b in range(n)]
        self.model = q4.Model(self.embed, self.blocks, self.final_norm, self.lm_head, EPS)
        self.fmodel = q4.Model(self.embed, self.blocks, self.final_norm, self.lm_head, EPS,
                               options=q4.MODEL_FACTORED_NORM)
