"""A decode-layer chain of GEMVs captured in one HIP graph.

"Resumo Tecnico: Llamas na Web", sections "Inferencia Local Eficiente em
Memoria" and "Biblioteca de Kernels Portatil em Desempenho", allocates every
buffer once at start-up and submits the kernels of a forward pass in batches
with little CPU-GPU synchronization. The chain here is the GEMV part of one
7B-class decode layer in Q4_0 at batch 1: fused QKV (12288 x 4096), output
projection (4096 x 4096), fused gate/up (22016 x 4096) and down projection
(4096 x 11008), each GEMV reading (a prefix of) the previous one's output as
its activations, so the launches depend on each other the way a layer's do.
Every buffer is allocated when the chain is built; the calls go through the
allocation-free entry point, so the whole chain can be captured in a HIP
graph and replayed with one launch per layer group.
"""
from __future__ import annotations

import numpy as np

LAYER = [  # (name, N, K): weight rows x inputs of each GEMV of the layer
    ("qkv", 12288, 4096),
    ("o", 4096, 4096),
    ("gate_up", 22016, 4096),
    ("down", 4096, 11008),
]


class DecodeChain:
    """`layers` decode layers of Q4_0 weights (distinct per layer), their
    activation buffers, and the launches of one pass over all of them."""

    def __init__(self, torch, layers=1, seed=0, device="cuda:0"):
        import synth
        self.torch = torch
        self.dev = torch.device(device)
        self.layers = []
        rng_seed = seed
        for _ in range(layers):
            ws = []
            for name, N, K in LAYER:
                # scales |N(0,1)| / (3.7 sqrt(K)) keep the activations near unit
                # size from one GEMV to the next (no normalization between them)
                c = synth.q4_0_case(N, K, 0, seed=rng_seed, scale=1.0 / (3.7 * K ** 0.5))
                rng_seed += 1
                ws.append(torch.from_numpy(c.W.reshape(-1)).to(self.dev))
            self.layers.append(ws)
        x0 = np.random.default_rng(seed + 10**6).standard_normal((1, LAYER[0][2]))
        self.x = torch.from_numpy(x0.astype(np.float32)).to(self.dev)
        self.outs = [torch.empty((1, N), dtype=torch.float32, device=self.dev)
                     for _, N, _ in LAYER]
        self.weight_bytes = sum(w.numel() for ws in self.layers for w in ws)

    def run(self):
        """One pass: every layer's four GEMVs, each reading the first K
        outputs of the previous GEMV (the first reads x, and the first GEMV of
        the next layer reads the last output)."""
        import block_quantized_matmul_amd as bq
        src = self.x
        for ws in self.layers:
            for w, (name, N, K), out in zip(ws, LAYER, self.outs):
                xin = src[:, :K] if src.shape[1] >= K else src
                if xin.shape[1] != K:
                    raise ValueError(f"{name}: needs {K} inputs, has {xin.shape[1]}")
                bq.lqmm_gemv_q4_0_noalloc(w, xin, N, out=out)
                src = out
        return src

    def capture(self):
        """A HIP graph of one pass (the library allocates nothing inside)."""
        g = self.torch.cuda.CUDAGraph()
        # (1, N)[:, :K] of a row-major (1, N) tensor is contiguous: no copy
        # kernel enters the graph
        with self.torch.cuda.graph(g):
            self.run()
        return g
