"""The five synthetic workloads, described by shape and value distribution only.

Shapes stand in for the models the pages train with GRPO (Qwen2.5-1.5B,
Llama-3.1-8B at the pages' 20K context with 8 generations per prompt, and
Phi-4) [Long-context GRPO, §1 and §2; Unsloth R1 reasoning page, §2].  No
dataset or checkpoint is involved: every tensor is drawn from the recipe below.

Readings where the description of a workload is silent or ambiguous:
  * "N(0, 0.1)" reward noise of the long-context workload is read as variance
    0.1 (standard deviation sqrt(0.1)), since the other normals are written
    with their squared scale spelled out.
  * Completion lengths "uniform in [a, b]" are discrete and inclusive; the
    mask is 1 on [prefix, prefix + length) and 0 elsewhere.
  * Zipf(1.1) target ids are truncated to [0, V): P(y = k) is proportional to
    (k + 1) ** -1.1.
  * Rewards of the trainable-head and fp16 workloads (unstated) are uniform
    floats in [0, 3], as in the Qwen-shaped workload.
  * fp16 outliers: each element of X_q and X_p independently becomes +-30
    (uniform sign) with probability 0.001.
  * "All unmasked" in the long-context workload means every one of the 20224
    completion positions is a loss token; the 256 prompt positions stay masked.
"""

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" | "bf16" | "f16": storage type of X_q, X_p, W
    G: int                # generations (sequences) per prompt; one prompt
    L: int                # positions per sequence
    H: int                # hidden size
    V: int                # vocabulary size
    prefix: int           # masked prompt positions at the start of each sequence
    comp_min: int         # completion length range, inclusive
    comp_max: int
    x_std: float          # X_q, X_p ~ N(0, x_std^2)
    w_std: float          # W ~ N(0, w_std^2)
    targets: str          # "uniform" | "zipf"
    rewards: str          # "int012" | "uniform03" | "bern_noise"
    need_dW: bool
    loss_scale: float = 1.0
    outlier_p: float = 0.0
    outlier_val: float = 0.0
    zipf_s: float = 1.1
    K: int = 1            # reward functions, summed before normalisation
    beta: float = 0.04
    eps: float = 1e-4
    seed: int = 0

    @property
    def B(self) -> int:
        return 1

    @property
    def S(self) -> int:
        return self.B * self.G

    @property
    def N(self) -> int:
        return self.S * self.L

    @property
    def expected_tokens(self) -> float:
        return self.S * (self.comp_min + self.comp_max) / 2.0


WORKLOADS = (
    Workload("tiny-f32", "f32", G=4, L=64, H=64, V=1000, prefix=16, comp_min=8, comp_max=48,
             x_std=1.0, w_std=0.02, targets="uniform", rewards="int012", need_dW=False, seed=1),
    Workload("qwen2.5-1.5b-bf16", "bf16", G=8, L=1024, H=1536, V=151936, prefix=256,
             comp_min=128, comp_max=768, x_std=1.0, w_std=0.02, targets="uniform",
             rewards="uniform03", need_dW=False, seed=2),
    Workload("llama3.1-8b-train-bf16", "bf16", G=8, L=4096, H=4096, V=128256, prefix=256,
             comp_min=512, comp_max=3840, x_std=1.0, w_std=0.02, targets="zipf",
             rewards="uniform03", need_dW=True, seed=3),
    Workload("llama3.1-8b-long-bf16", "bf16", G=8, L=20480, H=4096, V=128256, prefix=256,
             comp_min=20224, comp_max=20224, x_std=1.0, w_std=0.02, targets="uniform",
             rewards="bern_noise", need_dW=False, seed=4),
    Workload("phi4-f16", "f16", G=8, L=8192, H=5120, V=100352, prefix=512, comp_min=1024,
             comp_max=7680, x_std=1.5, w_std=0.02, targets="uniform", rewards="uniform03",
             need_dW=False, loss_scale=65536.0, outlier_p=0.001, outlier_val=30.0, seed=5),
)


def workload_by_name(name: str) -> Workload:
    for w in WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(f"unknown workload {name!r}; known: {[w.name for w in WORKLOADS]}")
