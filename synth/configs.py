"""The five workloads the loss head is measured and checked on.

Shapes follow the language-model heads the pages talk about: page 3
("Complete Guide to Liger Kernel", LigerFusedLinearCrossEntropyLoss section)
uses hidden size 4096 and the 128256-token Llama-3 vocabulary; page 2
("Liger-Kernel: Triton kernels that replace Hugging Face training ops", the
problem section) quotes LLaMA 3-8B at batch 8 and contexts up to 16K.  The
distributions are synthetic stand-ins for real hidden states, weights and
labels, which are not available here.
"""

from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Config:
    idx: int            # 1-based workload number
    name: str
    N: int              # tokens
    H: int              # hidden size
    V: int              # vocabulary size
    dtype: str          # "f32" or "bf16": dtype of h, W and grad_h
    h_dist: str         # "normal" | "rms_normal" | "normal_outliers"
    targets: str        # "uniform" | "zipf"
    w_std: float = 0.02
    zipf_s: float = 1.1
    outlier_frac: float = 0.001
    outlier_scale: float = 20.0
    rms_eps: float = 1e-6
    default_chunk: int = 0   # token chunk used by the benchmark (0: N)

    @property
    def flops(self) -> float:
        """Dense work of one forward+backward: three N*V*H contractions."""
        return 6.0 * self.N * self.V * self.H

    @property
    def naive_logits_bytes(self) -> int:
        """Bytes an unfused head would spend on an fp32 [N, V] logit tensor."""
        return 4 * self.N * self.V


CONFIGS = {
    1: Config(1, "tiny_fp32", N=256, H=128, V=1000, dtype="f32",
              h_dist="normal", targets="uniform", default_chunk=256),
    2: Config(2, "llama2_7b_head", N=2048, H=4096, V=32000, dtype="bf16",
              h_dist="normal", targets="uniform", default_chunk=2048),
    3: Config(3, "llama3_8b_head", N=8192, H=4096, V=128256, dtype="bf16",
              h_dist="rms_normal", targets="uniform", default_chunk=4096),
    4: Config(4, "llama3_8b_long_context", N=16384, H=4096, V=128256,
              dtype="bf16", h_dist="normal", targets="uniform",
              default_chunk=4096),
    5: Config(5, "large_vocab_256k", N=8192, H=3584, V=256000, dtype="bf16",
              h_dist="normal_outliers", targets="zipf", default_chunk=4096),
}


def config_by_name(name: str) -> Config:
    for c in CONFIGS.values():
        if c.name == name or str(c.idx) == str(name):
            return c
    raise KeyError(name)
