"""Workload shapes for multi-scale retention.

The shapes follow the model shapes the RetNet pages name: head dimension 256
and chunk 512 ("Retentive Network: A Successor to Transformer for Large
Language Models", Elamur summary, Key points items four and five), hidden size
1024 for the 200M comparison (Key points, third item), 2,048-token context
(Spiral-RetNet-3b model card, Model Description) and 8k-token inputs for the
7B decode claim (Elamur summary, Key points, first item).
"""

from dataclasses import dataclass, field

from .inputs import draw


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    heads: int
    dk: int
    dv: int
    chunk: int
    dtype: str  # "f32" or "bf16"
    qkv_scale: float
    gate_scale: float | None  # None: no GroupNorm / gate
    rotary_base: float  # 0: no rotation
    seed: int
    forms: tuple = field(default=("chunkwise",))
    decode_steps: int = 0
    decode_batches: tuple = ()

    def specs(self, batch=None, seqlen=None):
        """(shape, scale) list in draw order Q, K, V[, G]."""
        b = self.batch if batch is None else batch
        n = self.seqlen if seqlen is None else seqlen
        qk = (b, n, self.heads, self.dk)
        vv = (b, n, self.heads, self.dv)
        out = [(qk, self.qkv_scale), (qk, self.qkv_scale), (vv, self.qkv_scale)]
        if self.gate_scale is not None:
            out.append((vv, self.gate_scale))
        return out

    def inputs(self, batch=None, seqlen=None, seed=None):
        """Seeded Q, K, V[, G] as synth Tensors (G is None without a gate)."""
        ts = draw(self.seed if seed is None else seed, self.specs(batch, seqlen), self.dtype)
        if len(ts) == 3:
            ts.append(None)
        return ts


CONFIGS = {
    # batch 1, 256 tokens, 2 heads x 64, chunk 64, fp32, N(0,1)/sqrt(64), rotary on
    "tiny_fp32": Workload("tiny_fp32", 1, 256, 2, 64, 64, 64, "f32", 1 / 8, None, 10000.0, 1,
                          forms=("parallel", "recurrent", "chunkwise")),
    # hidden 1024 = 4 heads x 256, batch 8, 2048 tokens, chunk 512, bf16, gate N(0,1)
    "retention_200m": Workload("retention_200m", 8, 2048, 4, 256, 256, 512, "bf16", 1 / 16, 1.0, 0.0, 2),
    # hidden 2560 = 10 heads x 256, batch 4, 2048 tokens, rotary on, gate
    "retention_3b": Workload("retention_3b", 4, 2048, 10, 256, 256, 512, "bf16", 1 / 16, 1 / 16, 10000.0, 3,
                             forms=("parallel", "chunkwise")),
    # hidden 4096 = 16 heads x 256, batch 2, 8192 tokens, chunk 512, gate, state out
    "retention_7b_8k": Workload("retention_7b_8k", 2, 8192, 16, 256, 256, 512, "bf16", 1 / 16, 1 / 16, 0.0, 4),
    # 16 heads x 256 decode after an 8192-token chunkwise prefill at batch 64
    "retention_7b_decode": Workload("retention_7b_decode", 64, 8192, 16, 256, 256, 512, "bf16", 1 / 16, 1 / 16,
                                    0.0, 5, forms=("recurrent",), decode_steps=256,
                                    decode_batches=(1, 8, 64, 256)),
}


def get(name):
    return CONFIGS[name]
