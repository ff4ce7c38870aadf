"""Seeded synthetic workloads for tests and the benchmark.

Shapes, value distributions and hyperparameters of the five workloads the mask
path is measured and checked on.  This module holds no arithmetic of the method
itself: it only draws inputs (with torch's seeded generators) and names
shapes.  Both the GPU library's callers and the CPU oracle's callers take their
inputs from here; the oracle never imports it.

Stand-ins: trained LLaMA-2-7B / Nemotron-4-15B weights are not available, so
weights are Gaussian at the published layer shapes (the kernels have no
data-dependent control flow apart from argmax and top-N).  Hyperparameters
follow the MaskLLM summary page, section 3.4 (Table 7 and the kappa / tau /
alpha / lambda sweeps): kappa 100 -> 500, tau 4 -> 0.05, alpha 3, lambda 1e-5,
logit init N(0, 0.01) (read as standard deviation 0.01).
"""
from __future__ import annotations

from dataclasses import dataclass, field

LLAMA2_7B = dict(hidden=4096, ffn=11008, layers=32)
NEMOTRON4_15B = dict(hidden=6144, ffn=24576)


@dataclass
class TensorSpec:
    name: str
    rows: int
    cols: int
    tensor_id: int


@dataclass
class Workload:
    key: str
    n: int
    m: int
    tensors: list
    w_dtype: str            # "f32" | "bf16"
    w_std: float
    z_std: float
    g_std: float
    g_dtype: str
    kappa: float = 100.0
    tau: float = 4.0
    lam: float = 1e-5
    steps: int = 1
    kappa_end: float | None = None
    tau_end: float | None = None
    prior_alpha: float | None = None  # magnitude-prior seeding of base logits
    description: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def k(self) -> int:
        return {(2, 4): 6, (4, 8): 70}[(self.n, self.m)]

    def nblocks(self) -> int:
        return sum(t.rows * t.cols // self.m for t in self.tensors)

    def schedule(self, s: int):
        """(kappa_s, tau_s) of step s: linear with both endpoints included."""
        if self.steps <= 1 or self.kappa_end is None:
            return self.kappa, self.tau
        f = s / (self.steps - 1)
        return (self.kappa + (self.kappa_end - self.kappa) * f,
                self.tau + (self.tau_end - self.tau) * f)


def llama7b_layer(layer: int):
    h, f = LLAMA2_7B["hidden"], LLAMA2_7B["ffn"]
    shapes = [("q_proj", h, h), ("k_proj", h, h), ("v_proj", h, h), ("o_proj", h, h),
              ("gate_proj", f, h), ("up_proj", f, h), ("down_proj", h, f)]
    return [TensorSpec(f"layers.{layer}.{n}", r, c, 7 * layer + i)
            for i, (n, r, c) in enumerate(shapes)]


def nemotron15b_layer():
    h, f = NEMOTRON4_15B["hidden"], NEMOTRON4_15B["ffn"]
    shapes = [("q_proj", h, h), ("k_proj", h, h), ("v_proj", h, h), ("o_proj", h, h),
              ("up_proj", f, h), ("down_proj", h, f)]
    return [TensorSpec(n, r, c, i) for i, (n, r, c) in enumerate(shapes)]


WORKLOADS = {
    "single256_f32": Workload(
        "single256_f32", 2, 4, [TensorSpec("w", 256, 256, 0)], "f32", 0.02, 1.0, 1.0, "f32",
        description="one 256x256 fp32 weight, 2:4, fwd+bwd+hard argmax"),
    "llama7b_qproj_prior": Workload(
        "llama7b_qproj_prior", 2, 4, [TensorSpec("q_proj", 4096, 4096, 0)], "bf16", 0.02, 0.01,
        1e-3, "bf16", prior_alpha=3.0,
        description="LLaMA-2-7B q_proj 4096x4096 bf16, logits N(0,0.01) seeded by a magnitude "
                    "top-2 prior (alpha 3)"),
    "llama7b_mlp_anneal": Workload(
        "llama7b_mlp_anneal", 2, 4,
        [TensorSpec("gate_proj", 11008, 4096, 0), TensorSpec("up_proj", 11008, 4096, 1),
         TensorSpec("down_proj", 4096, 11008, 2)], "bf16", 0.02, 1.0, 1e-3, "bf16",
        steps=8, kappa_end=500.0, tau_end=0.05,
        description="LLaMA-2-7B MLP trio, tau 4 -> 0.05 and kappa 100 -> 500 over 8 steps"),
    "llama7b_all_linear": Workload(
        "llama7b_all_linear", 2, 4,
        [t for layer in range(LLAMA2_7B["layers"]) for t in llama7b_layer(layer)], "bf16", 0.02,
        1.0, 1e-3, "bf16",
        description="all 224 linear weights of a 32-layer LLaMA-2-7B-shaped model, swept per "
                    "tensor: fwd+bwd, then hard-mask extract + 2:4 compaction"),
    "nemotron15b_layer_48": Workload(
        "nemotron15b_layer_48", 4, 8, nemotron15b_layer(), "bf16", 0.015, 1.0, 1e-3, "bf16",
        tau=2.0, description="Nemotron-4-15B-shaped layer set (hidden 6144, FFN 24576), 4:8"),
}


def _gen(device, seed):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def seed_for(tensor_id: int, what: str) -> int:
    """Generator seed of one input stream: 1000 + 16*tensor_id + {W,z,G,base,pi}."""
    return 1000 + 16 * tensor_id + {"w": 0, "z": 1, "g": 2, "base": 3, "pi": 4}[what]


def draw(shape, std, dtype, device, seed):
    """N(0, std^2) samples; bf16 values are fp32 samples rounded to nearest even."""
    import torch
    x = torch.randn(shape, generator=_gen(device, seed), device=device, dtype=torch.float32)
    x.mul_(std)
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    return x


def tensor_inputs(wl: Workload, spec: TensorSpec, device, rows=None):
    """W, z (or the base logits before prior seeding) and G of one tensor."""
    rows = spec.rows if rows is None else rows
    B = rows * spec.cols // wl.m
    w = draw((rows, spec.cols), wl.w_std, wl.w_dtype, device, seed_for(spec.tensor_id, "w"))
    z = draw((B, wl.k), wl.z_std, "f32", device, seed_for(spec.tensor_id, "z"))
    g = draw((rows, spec.cols), wl.g_std, wl.g_dtype, device, seed_for(spec.tensor_id, "g"))
    return w, z, g


# Linear-space logits (one per weight, the MaskPro variant): N(0, 1), a spread
# at which the draws of a block vary from step to step.
PI_STD = 1.0


def linear_logits(wl: Workload, spec: TensorSpec, device, rows=None):
    """fp32 [B, M] logits of one tensor for the linear-space variant."""
    rows = spec.rows if rows is None else rows
    B = rows * spec.cols // wl.m
    return draw((B, wl.m), PI_STD, "f32", device, seed_for(spec.tensor_id, "pi"))
