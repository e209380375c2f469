"""The five KDA workloads: shapes, dtypes and input distributions.

q and k are drawn N(0, 1) and L2-normalised per (token, head); v ~ N(0, 1);
beta = sigmoid(N(0, 1)) per (token, head); alpha = sigmoid(N(mu, 1)) per
(token, head, key channel); the initial state ~ N(0, std) with std the second
number of "N(0, x)" read as a standard deviation.
"""
from dataclasses import dataclass, field
from typing import Optional


@dataclass(frozen=True)
class Config:
    name: str
    kind: str                 # "chunk" or "decode"
    dtype: str                # storage dtype of q, k, v and o: "f32" or "bf16"
    B: int
    T: int
    H: int
    dk: int
    dv: int
    alpha_mu: float
    s0_std: Optional[float]   # None = zero initial state
    num_seqs: int = 0         # varlen: number of packed sequences (B == 1)
    len_range: tuple = ()     # varlen: inclusive length range
    steps: int = 0            # decode: consecutive steps
    seed: int = 0
    notes: str = field(default="")


CONFIGS = [
    Config("fp32_B1_H2_T256_d64", "chunk", "f32", 1, 256, 2, 64, 64, 4.0, None, seed=0,
           notes="fp32 forward, zero initial state"),
    Config("bf16_B4_H16_T4096_d128", "chunk", "bf16", 4, 4096, 16, 128, 128, 4.0, 0.02, seed=1,
           notes="chunked forward, nonzero initial state"),
    Config("bf16_B1_H32_T65536_d128", "chunk", "bf16", 1, 65536, 32, 128, 128, 5.0, None, seed=2,
           notes="long context, slow forgetting, zero initial state"),
    Config("decode_N256_H32_d128", "decode", "bf16", 256, 1, 32, 128, 128, 4.0, 0.05, steps=100,
           seed=3, notes="single-token decode, fp32 state in place, 100 consecutive steps"),
    Config("varlen_N64_H16_d128", "chunk", "bf16", 1, 0, 16, 128, 128, 4.0, 0.02, num_seqs=64,
           len_range=(128, 8192), seed=4, notes="packed variable-length sequences"),
]
