"""The five synthetic workloads (sizes, token-row counts, value distributions).

Plain data; no arithmetic of the method lives here.

  worked   the wiki's column-parallel example: X fp32 [32, 1024], one
           1024 -> 2048 weight split into 2 column shards, plus the
           row-parallel variant (2 row shards of [512, 2048]); N(0, 1) draws
           and an integer copy with values in {-3..3}.
  llama2k  one rank of tp=4 of a Llama-style dense layer, bf16: hidden 2048,
           32 Q / 8 KV heads of 64, FFN 8192; M = 1, 16, 256.
  dec7b    decode with 4-bit weights, one rank of tp=4 of a 7B-class layer:
           hidden 3584, FFN 18944, 28 Q / 4 KV heads of 128; M = 1, 4, 16.
  pre27b   prefill with 4-bit weights, one rank of tp=4 of a 27B-class layer:
           hidden 5120, FFN 17408, 64 Q / 8 KV heads of 128; M = 2048.
  gqa8     the GQA replication case: tp=8, hidden 4096, 32 Q / 4 KV heads of
           128 (K/V replicated), FFN 14336, bf16; M = 64 (decode) and 512
           (prefill).
Vocabulary-parallel workloads (embedding table and LM head split over the
vocabulary, which the pages recommend past about 100k tokens):
  vocab7b  vocabulary 152064 at dec7b's width (hidden 3584), tp=4: a 4-bit
           LM head at decode (M = 1, 4, 16 token rows of N(0, 1) bf16
           activations) and a bf16 N(0, 0.02) embedding table looked up by
           M = 2048 uniformly drawn token ids.
"""
from dataclasses import dataclass, field

F32, BF16, Q4 = "f32", "bf16", "q4g64"


@dataclass(frozen=True)
class Layer:
    name: str
    index: int            # config number used in the input seeds
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    tp: int
    wdtype: str
    ms: tuple             # token-row counts
    w_std: float = 0.02   # dense weights ~ N(0, w_std^2)
    x_std: float = 1.0    # activations ~ N(0, x_std^2)
    # 4-bit format: scales ~ U(lo, hi), biases ~ N(0, bias_std^2)
    scale_lo: float = 0.005
    scale_hi: float = 0.02
    bias_std: float = 0.05
    measured: tuple = field(default=("q", "k", "v", "o", "gate", "up", "down"))

    @property
    def group(self):
        return 64 if self.wdtype == Q4 else 0


@dataclass(frozen=True)
class Worked:
    """The wiki example: one linear layer 1024 -> 2048 on 2 ranks."""
    name: str = "worked"
    index: int = 0
    K: int = 1024
    N: int = 2048
    tp: int = 2
    M: int = 32
    wdtype: str = F32


WORKED = Worked()
LLAMA2K = Layer("llama2k", 1, 2048, 32, 8, 64, 8192, 4, BF16, (1, 16, 256))
DEC7B = Layer("dec7b", 2, 3584, 28, 4, 128, 18944, 4, Q4, (1, 4, 16))
PRE27B = Layer("pre27b", 3, 5120, 64, 8, 128, 17408, 4, Q4, (2048,),
               measured=("gate", "up", "down", "o"))
GQA8 = Layer("gqa8", 4, 4096, 32, 4, 128, 14336, 8, BF16, (64, 512))

LAYERS = (LLAMA2K, DEC7B, PRE27B, GQA8)
PROJS = ("q", "k", "v", "o", "gate", "up", "down")


@dataclass(frozen=True)
class Vocab:
    """A vocabulary-parallel embedding + LM head workload."""
    name: str
    index: int           # config number used in the input seeds
    vocab: int
    hidden: int
    tp: int
    head_ms: tuple       # LM-head token rows (decode)
    lookup_m: int        # embedding lookups per call
    e_std: float = 0.02  # embedding table ~ N(0, e_std^2), bf16
    scale_lo: float = 0.005
    scale_hi: float = 0.02
    bias_std: float = 0.05


VOCAB7B = Vocab("vocab7b", 5, 152064, 3584, 4, (1, 4, 16), 2048)


@dataclass(frozen=True)
class Moe:
    """A mixture-of-experts FFN workload."""
    name: str
    index: int           # config number used in the input seeds
    n_experts: int
    top_k: int
    hidden: int
    expert_ffn: int
    tp: int
    tokens: tuple        # token counts T
    x_std: float = 1.0
    scale_lo: float = 0.005
    scale_hi: float = 0.02
    bias_std: float = 0.05


MOE30B = Moe("moe30b", 6, 128, 8, 2048, 768, 4, (2048, 16))
MOE_SMALL = Moe("moe_small", 7, 16, 4, 384, 256, 2, (37, 5))
