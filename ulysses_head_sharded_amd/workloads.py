"""The synthetic Ulysses per-rank workloads (shapes only; no arithmetic).

Every workload is one rank's share of a Ulysses attention layer: P emulated
ranks, global sequence s, batch b, h query heads and h_kv KV heads of size
d_h.  The rank holds a [s/P, b, h, d_h] shard before the exchange and
computes attention for h/P heads over the whole s after it.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    c: int  # seed family: Q = 100c+1, K = 100c+2, V = 100c+3
    P: int
    s: int
    b: int
    h: int
    h_kv: int
    d: int
    dtype: str  # "f32" or "bf16"
    causal: bool
    about: str

    @property
    def hp(self) -> int:
        return self.h // self.P

    @property
    def hkvp(self) -> int:
        """KV heads of the share: h_kv/P, or 1 when h_kv < P (each KV head replicated)."""
        return self.h_kv // self.P if self.h_kv % self.P == 0 else 1

    @property
    def elt(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def pairs(self) -> int:
        return self.s * (self.s + 1) // 2 if self.causal else self.s * self.s

    def attn_flops(self) -> float:
        """Algorithmic FLOPs: 2 per multiply-add of QK^T and of PV over visible pairs."""
        return 4.0 * self.d * self.b * self.hp * self.pairs()

    def attn_bwd_flops(self) -> float:
        """Algorithmic FLOPs of the attention backward: the five products over
        visible pairs (S = QK^T recomputed, dP = dO V^T, dV = P^T dO, dQ = dS K,
        dK = dS^T Q), 2 per multiply-add; 2.5 times the forward."""
        return 10.0 * self.d * self.b * self.hp * self.pairs()

    def shard_bytes(self, kv: bool = False) -> int:
        """Bytes of one rank-local [s/P, b, heads, d] shard."""
        heads = self.h_kv if kv else self.h
        return (self.s // self.P) * self.b * heads * self.d * self.elt

    def kv_blocks_bytes(self) -> int:
        """Bytes of one K or V send buffer [P, s/P, b, hkvp, d] (larger than the
        shard when heads are replicated)."""
        return self.s * self.b * self.hkvp * self.d * self.elt

    def layout_bytes(self) -> int:
        """Algorithmic HBM bytes of pack(Q), pack(K), pack(V), unpack(O): read + write."""
        return 4 * self.shard_bytes() + 2 * (self.shard_bytes(kv=True) + self.kv_blocks_bytes())


WORKLOADS = {
    "tiny": Workload("tiny", 1, 4, 16, 1, 8, 8, 64, "f32", False,
                     "tiny share: P=4, 16 tokens, 8 heads, d_h=64, fp32, dense"),
    "gpt1.2b-32k": Workload("gpt1.2b-32k", 2, 8, 32768, 1, 16, 16, 128, "bf16", True,
                            "GPT-1.2B-like share: 16 MHA heads, s=32768, P=8, causal"),
    "mha-128k": Workload("mha-128k", 3, 8, 131072, 1, 32, 32, 128, "bf16", True,
                         "MHA long share: 32 heads, s=131072, P=8, causal"),
    "gqa-64k": Workload("gqa-64k", 4, 8, 65536, 2, 32, 8, 128, "bf16", True,
                        "GQA share: 32 Q / 8 KV heads, s=65536, b=2, P=8, causal"),
    # an extra share beside the ones above: the GQA share at twice the ranks it
    # has KV heads for, possible only with KV-head replication (each rank gets
    # one KV head)
    "gqa-64k-p16": Workload("gqa-64k-p16", 6, 16, 65536, 2, 32, 8, 128, "bf16", True,
                            "GQA share with fewer KV heads than ranks: 32 Q / 8 KV heads, "
                            "s=65536, b=2, P=16 (KV heads replicated), causal"),
    "mtok-1m": Workload("mtok-1m", 5, 64, 1048576, 1, 64, 64, 128, "bf16", True,
                        "million-token share: 64 heads, s=1048576, P=64, causal"),
    "dit-256k": Workload("dit-256k", 5, 8, 262144, 1, 32, 32, 128, "bf16", False,
                         "DiT-style dense share: 32 heads, s=262144, P=8, non-causal"),
}
