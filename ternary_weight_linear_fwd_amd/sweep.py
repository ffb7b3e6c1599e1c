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


FORMATS = ("2bit", "base3")


class DecodeSweep:
    """formats: which weight layouts to pack and plan ("2bit": the device
    layout, 2 bits per weight; "base3": the base-3 layout, 1.6 bits per weight
    and at most 8 tokens).  Ms: token counts planned for the 2-bit layout,
    base3_Ms those for the base-3 layout; plans of one token count share
    their activation and output buffers."""

    def __init__(self, layers: int = S.C4_LAYERS, projs: Sequence[S.Proj] = S.C4_PROJS,
                 Ms: Iterable[int] = (1, 16), keep_int: Iterable[Tuple[int, str]] = (),
                 progress=None, formats: Sequence[str] = ("2bit",), base3_Ms: Iterable[int] = (1,)):
        import torch
        from . import bitlinear as L

        assert formats and all(f in FORMATS for f in formats)
        self.torch, self.L = torch, L
        self.layers, self.projs, self.formats = layers, list(projs), tuple(formats)
        self.Ms = {"2bit": list(Ms) if "2bit" in formats else [],
                   "base3": list(base3_Ms) if "base3" in formats else []}
        self.keep_int = set(keep_int)
        dev = "cuda"
        self.packed: Dict[Tuple[str, int, str], "torch.Tensor"] = {}
        self.gamma: Dict[Tuple[int, str], float] = {}
        ws_bytes = max(L.bitlinear_workspace_bytes(0, p.N, p.K) for p in self.projs)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        g_host = ctypes.c_float()
        for layer in range(layers):
            for p in self.projs:
                W = S.c4_weight_device(layer, p, dev)
                for fmt in self.formats:
                    if fmt == "2bit":
                        buf = torch.empty(L.bitlinear_packed_bytes(p.N, p.K), dtype=torch.uint8, device=dev)
                        L.bitlinear_pack_weights(W, p.N, p.K, buf, None, g_host, ws, ws_bytes)
                    else:
                        buf = torch.empty(L.bitlinear_packed3_bytes(p.N, p.K), dtype=torch.uint8, device=dev)
                        L.bitlinear_pack_weights3(W, p.N, p.K, buf, None, g_host, ws, ws_bytes)
                    self.packed[(fmt, layer, p.name)] = buf
                    self.gamma[(layer, p.name)] = g_host.value   # the same absmean scale either way
                del W
            if progress and (layer % 10 == 9 or layer == layers - 1):
                progress(f"packed {layer + 1}/{layers} layers ({', '.join(self.formats)})")
        del ws
        # activations and outputs per token count, one plan per (layout, token count)
        self.x, self.xq, self.eta, self.y, self.y_int = {}, {}, {}, {}, {}
        self.plans, self.tables = {}, {}
        for fmt in self.formats:
            for M in self.Ms[fmt]:
                specs = []
                for layer in range(layers):
                    for p in self.projs:
                        key = (layer, p.name, M)
                        if key not in self.x:
                            self.x[key] = torch.from_numpy(S.c4_x(layer, p, M)).to(dev)
                            self.xq[key] = torch.empty((M, p.K), dtype=torch.int8, device=dev)
                            self.eta[key] = torch.empty(M, dtype=torch.float32, device=dev)
                            self.y[key] = torch.empty((M, p.N), dtype=torch.float32, device=dev)
                            if (layer, p.name) in self.keep_int:
                                self.y_int[key] = torch.empty((M, p.N), dtype=torch.int32, device=dev)
                        specs.append(dict(x=self.x[key], xq=self.xq[key], eta=self.eta[key],
                                          packed=self.packed[(fmt, layer, p.name)], y=self.y[key],
                                          y_int=self.y_int.get(key), gamma=self.gamma[(layer, p.name)],
                                          N=p.N, K=p.K,
                                          format=L.BITLINEAR_FORMAT_2BIT if fmt == "2bit"
                                          else L.BITLINEAR_FORMAT_BASE3))
                probs = L.make_problems(specs)
                tb = L.bitlinear_grouped_table_bytes(probs, len(specs), M)
                table = torch.empty(tb, dtype=torch.uint8, device=dev)
                self.tables[(fmt, M)] = table
                plan = L.bitlinear_grouped_plan_init(probs, len(specs), M, table, tb)
                self.plans[(fmt, M)] = plan
                if progress:
                    progress(f"plan {fmt} M={M}: {plan.units} units, {plan.quant_rows} rows, kernel {plan.kernel}")
        torch.cuda.synchronize()

    def step(self, M: int, stream=None, fmt: str = "2bit") -> None:
        self.L.bitlinear_forward_grouped(self.plans[(fmt, M)], stream)

    # ---- algorithmic work per step
    def weight_bytes(self, fmt: str = "2bit") -> int:
        size = self.L.bitlinear_packed_bytes if fmt == "2bit" else self.L.bitlinear_packed3_bytes
        return sum(int(size(p.N, p.K)) for p in self.projs) * self.layers

    @staticmethod
    def _weight_bytes_alg(p, fmt: str) -> int:
        return p.N * p.K // 4 if fmt == "2bit" else p.N * p.K // 5   # 2 or 1.6 bits per weight

    def algorithmic_bytes(self, M: int, fmt: str = "2bit") -> int:
        """Packed weights + float32 x in + float32 y out + eta (the fused step reads
        float32 activations; the int8 round trip inside the step is overhead)."""
        per_layer = sum(self._weight_bytes_alg(p, fmt) + 4 * M * p.K + 4 * M * p.N + 4 * M for p in self.projs)
        return per_layer * self.layers

    def contraction_bytes(self, M: int, fmt: str = "2bit") -> int:
        """What the contraction kernel alone must move: packed weights + int8 xq +
        eta + float32 y."""
        per_layer = sum(self._weight_bytes_alg(p, fmt) + M * p.K + 4 * M + 4 * M * p.N for p in self.projs)
        return per_layer * self.layers

    def ops(self, M: int) -> int:
        return 2 * M * sum(p.N * p.K for p in self.projs) * self.layers
