"""A per-token decode loop over the compressed parts of a Gemma-2-2B-shaped model, built from the
library's entry points: the current token's embedding row (rq_decode_rows, fp32, times sqrt(D) as
Gemma scales its embeddings), the MLP blocks (rq_lut_mlp) on a residual stream, and the tied head on
the last hidden vector (rq_build_lut + rq_lut_logits: softcap and argmax, no logits written). The
argmax id stays on the device and is the next token's row id, so a run of tokens is enqueued with no
host synchronisation.

Around each block sits Gemma-2's own glue, outside the method: an RMSNorm before the block and one
after it, the block's output added to the residual stream, and a final RMSNorm before the head. One
rq_residual_norm launch per block does it (h += rms(y), then the next input rms(h)). The norms carry
unit scales (Gemma-2 stores each RMSNorm scale as 1 + w, and w starts at zero). Without them the chain diverges on these synthetic weights: a block maps an input of
scale s to about 1.3 s^2, so an unnormalised chain of 26 blocks overflows fp32 within ten. Attention is
not part of the loop (it needs the model's weights)."""
import math

import torch

from . import binding as B

RMS_EPS = 1e-6


class DecodeLoop:
    """head: DeviceMatrix of the tied embedding / head; layers: list of (gate, up, down) DeviceMatrix."""

    def __init__(self, head, layers, softcap=30.0, max_tokens=128, device="cuda", keep_layers=False):
        """keep_layers: keep every block's input (ins[i], after the pre-norm) and output (outs[i]) of
        the last step, instead of one buffer each."""
        self.head, self.layers, self.softcap = head, list(layers), softcap
        self.scale = math.sqrt(head.D)
        self.ids = torch.zeros(max_tokens + 1, dtype=torch.int32, device=device)
        D = head.D

        def buf():
            return torch.empty((1, D), dtype=torch.float32, device=device)

        self.row = buf()
        self.h = buf()       # residual stream
        self.last = buf()    # final-norm output: the head's hidden vector
        n = len(self.layers) if keep_layers else 1
        self.ins = [buf() for _ in range(n)]
        self.outs = [buf() for _ in range(n)]
        self.lut = torch.empty(B.lut_bytes(head, 1) // 4, dtype=torch.float32, device=device)
        mlp_ws = max([B.lut_mlp_workspace(*lay, 1) for lay in self.layers] + [256])
        self.ws_mlp = B.workspace(mlp_ws, device)
        self.ws_head = B.workspace(B.lut_logits_workspace(head, 1), device)

    def step(self, t):
        """Token t: row of ids[t] -> blocks on the residual stream -> final norm -> head argmax into
        ids[t + 1]. Returns the head's hidden vector."""
        B.decode_rows(self.head, self.ids[t:t + 1], "f32", out=self.row)
        torch.mul(self.row, self.scale, out=self.h)
        n = len(self.layers)

        def block_input(i):   # block i's input buffer; past the last block, the head's vector
            return self.ins[i % len(self.ins)] if i < n else self.last

        B.residual_norm(self.h, block_input(0), eps=RMS_EPS)
        for i, (gate, up, down) in enumerate(self.layers):
            y = self.outs[i % len(self.outs)]
            B.lut_mlp(gate, up, down, block_input(i), ws=self.ws_mlp, out=y)
            B.residual_norm(self.h, block_input(i + 1), y, eps=RMS_EPS)
        B.build_lut(self.head, self.last, out=self.lut)
        B.lut_logits(self.head, self.lut, 1, softcap=self.softcap, logits=False, ws=self.ws_head,
                     argmax_out=self.ids[t + 1:t + 2])
        return self.last

    def run(self, first_id, n_tokens):
        """Enqueue n_tokens steps starting from token first_id; the ids are in self.ids[:n_tokens + 1]."""
        self.ids[0] = int(first_id)
        for t in range(n_tokens):
            self.step(t)
        return self.ids[:n_tokens + 1]
