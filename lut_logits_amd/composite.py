"""A per-token decode loop over the compressed parts of a Gemma-2-2B-shaped model, built from the
library's entry points only: the current token's embedding row (rq_decode_rows, fp32, times sqrt(D)
as Gemma scales its embeddings), the MLP blocks chained one into the next (rq_lut_mlp), and the tied
head on the last output (rq_build_lut + rq_lut_logits: softcap and argmax, no logits written). The
argmax id stays on the device and is the next token's row id, so a run of tokens is enqueued with no
host synchronisation.

Attention, norms and residual connections are not part of it (they need the model's weights); the
sqrt(D) scale is plain torch arithmetic and keeps the activations at unit scale through the chain."""
import math

import torch

from . import binding as B


class DecodeLoop:
    """head: DeviceMatrix of the tied embedding / head; layers: list of (gate, up, down) DeviceMatrix."""

    def __init__(self, head, layers, softcap=30.0, max_tokens=128, device="cuda", keep_layers=False):
        """keep_layers: keep every block's output of the last step (xs[i] is block i's input,
        xs[i + 1] its output) instead of two alternating buffers."""
        self.head, self.layers, self.softcap = head, list(layers), softcap
        self.scale = math.sqrt(head.D)
        self.ids = torch.zeros(max_tokens + 1, dtype=torch.int32, device=device)
        self.row = torch.empty((1, head.D), dtype=torch.float32, device=device)
        nbuf = len(self.layers) + 1 if keep_layers else 2
        self.xs = [torch.empty((1, head.D), dtype=torch.float32, device=device) for _ in range(nbuf)]
        self.lut = torch.empty(B.lut_bytes(head, 1) // 4, dtype=torch.float32, device=device)
        mlp_ws = max([B.lut_mlp_workspace(*lay, 1) for lay in self.layers] + [256])
        self.ws_mlp = B.workspace(mlp_ws, device)
        self.ws_head = B.workspace(B.lut_logits_workspace(head, 1), device)

    def step(self, t):
        """Token t: row of ids[t] -> MLP chain -> head argmax into ids[t + 1]. Returns the last hidden vector."""
        B.decode_rows(self.head, self.ids[t:t + 1], "f32", out=self.row)
        x = self.xs[0]
        torch.mul(self.row, self.scale, out=x)
        for i, (gate, up, down) in enumerate(self.layers):
            y = self.xs[(i + 1) % len(self.xs)]
            B.lut_mlp(gate, up, down, x, ws=self.ws_mlp, out=y)
            x = y
        B.build_lut(self.head, x, out=self.lut)
        B.lut_logits(self.head, self.lut, 1, softcap=self.softcap, logits=False, ws=self.ws_head,
                     argmax_out=self.ids[t + 1:t + 2])
        return x

    def run(self, first_id, n_tokens):
        """Enqueue n_tokens steps starting from token first_id; the ids are in self.ids[:n_tokens + 1]."""
        self.ids[0] = int(first_id)
        for t in range(n_tokens):
            self.step(t)
        return self.ids[:n_tokens + 1]
