"""Grouped decode sweeps: every BitLinear projection of every layer of a model,
packed once on the GPU and run as one grouped forward per token step.

The 70B-shaped sweep holds 80 layers x 7 projections (q, o 8192->8192; k, v
8192->1024; gate, up 8192->28672; down 28672->8192), 17.1 GB of packed
ternary weights resident in HBM.  Each latent matrix is drawn on the GPU
(seeded), packed by ``bitlinear_pack_weights`` and freed, so the 274 GB of
float32 latents never exist at once.  Activations are float32 ``[M][K]`` per
(layer, projection), drawn on the host and uploaded once.

One step = ``bitlinear_forward_grouped``: a grouped activation-quantize
kernel over all 560 inputs, then one grouped contraction kernel over all
work units (dequant fused).
"""
from __future__ import annotations

import ctypes
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

from . import synthetic as S


class DecodeSweep:
    def __init__(self, layers: int = S.C4_LAYERS, projs: Sequence[S.Proj] = S.C4_PROJS,
                 Ms: Iterable[int] = (1, 16), keep_int: Iterable[Tuple[int, str]] = (),
                 progress=None):
        import torch
        from . import bitlinear as L

        self.torch, self.L = torch, L
        self.layers, self.projs, self.Ms = layers, list(projs), list(Ms)
        self.keep_int = set(keep_int)
        dev = "cuda"
        self.packed: Dict[Tuple[int, str], "torch.Tensor"] = {}
        self.gamma: Dict[Tuple[int, str], float] = {}
        ws_bytes = max(L.bitlinear_workspace_bytes(0, p.N, p.K) for p in self.projs)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        g_host = ctypes.c_float()
        for layer in range(layers):
            for p in self.projs:
                W = S.c4_weight_device(layer, p, dev)
                buf = torch.empty(L.bitlinear_packed_bytes(p.N, p.K), dtype=torch.uint8, device=dev)
                L.bitlinear_pack_weights(W, p.N, p.K, buf, None, g_host, ws, ws_bytes)
                del W
                self.packed[(layer, p.name)] = buf
                self.gamma[(layer, p.name)] = g_host.value
            if progress and (layer % 10 == 9 or layer == layers - 1):
                progress(f"packed {layer + 1}/{layers} layers")
        del ws
        # activations, outputs and one plan per token count
        self.x, self.xq, self.eta, self.y, self.y_int, self.plans, self.tables = {}, {}, {}, {}, {}, {}, {}
        for M in self.Ms:
            specs = []
            for layer in range(layers):
                for p in self.projs:
                    key = (layer, p.name, M)
                    x = torch.from_numpy(S.c4_x(layer, p, M)).to(dev)
                    self.x[key] = x
                    self.xq[key] = torch.empty((M, p.K), dtype=torch.int8, device=dev)
                    self.eta[key] = torch.empty(M, dtype=torch.float32, device=dev)
                    self.y[key] = torch.empty((M, p.N), dtype=torch.float32, device=dev)
                    if (layer, p.name) in self.keep_int:
                        self.y_int[key] = torch.empty((M, p.N), dtype=torch.int32, device=dev)
                    specs.append(dict(x=x, xq=self.xq[key], eta=self.eta[key],
                                      packed=self.packed[(layer, p.name)], y=self.y[key],
                                      y_int=self.y_int.get(key), gamma=self.gamma[(layer, p.name)],
                                      N=p.N, K=p.K))
            probs = L.make_problems(specs)
            tb = L.bitlinear_grouped_table_bytes(probs, len(specs), M)
            table = torch.empty(tb, dtype=torch.uint8, device=dev)
            self.tables[M] = table
            self.plans[M] = L.bitlinear_grouped_plan_init(probs, len(specs), M, table, tb)
            if progress:
                progress(f"plan M={M}: {self.plans[M].units} units, {self.plans[M].quant_rows} rows")
        torch.cuda.synchronize()

    def step(self, M: int, stream=None) -> None:
        self.L.bitlinear_forward_grouped(self.plans[M], stream)

    # ---- algorithmic work per step
    def weight_bytes(self) -> int:
        return sum(int(self.L.bitlinear_packed_bytes(p.N, p.K)) for p in self.projs) * self.layers

    def algorithmic_bytes(self, M: int) -> int:
        """Packed weights + float32 x in + float32 y out + eta (the fused step reads
        float32 activations; the int8 round trip inside the step is overhead)."""
        per_layer = sum(p.N * p.K // 4 + 4 * M * p.K + 4 * M * p.N + 4 * M for p in self.projs)
        return per_layer * self.layers

    def contraction_bytes(self, M: int) -> int:
        """What the contraction kernel alone must move: packed weights + int8 xq +
        eta + float32 y."""
        per_layer = sum(p.N * p.K // 4 + M * p.K + 4 * M + 4 * M * p.N for p in self.projs)
        return per_layer * self.layers

    def ops(self, M: int) -> int:
        return 2 * M * sum(p.N * p.K for p in self.projs) * self.layers
