"""The five synthetic workloads of the zero-computation-expert MoE layer.

Every shape, distribution and routing structure used by the tests, the smoke check and
the benchmark lives here and nowhere else.  Notation follows the LongCat-Flash article
(itouyu.top, section "Zero-computation experts"): T tokens x_t of width d, a pool of N
FFN experts plus Z zero-computation (identity) experts, each token choosing K of the
N+Z.  I is the SwiGLU intermediate width of one FFN expert.

Index convention: FFN experts are 0..N-1, zero-computation experts are N..N+Z-1.

Bias recipes (``bias`` field):
  ("uniform", a)                   b_i ~ U(-a, a) for every expert, used as drawn.
  ("uniform+shift", a, share)      b_i ~ U(-a, a); a constant beta is added to every
                                   zero-expert bias, beta chosen offline so that the
                                   fraction of picks that land on zero experts is
                                   ``share`` (within 0.002).
  ("exclude_zero", a)              FFN biases ~ U(-a, a); every zero-expert bias is -2,
                                   so a zero expert can never enter the top K (p <= 1).
  ("zipf+shift", s, c, a, share)   FFN bias b_e = c * r_e^(-s) with r a seeded
                                   permutation of 1..N (heavy-tailed expert load); zero
                                   experts get beta + U(-a, a), beta tuned to ``share``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    N: int
    Z: int
    K: int
    I: int
    dtype: str                 # "f32" or "bf16": x, expert weights and y
    seed_key: tuple            # SeedSequence entropy words of this workload
    expert_std: float          # standard deviation of every expert weight
    bias: tuple                # bias recipe, see module docstring
    plant_frac: float = 0.0    # fraction of "easy" and of "hard" tokens planted
    plant_scale: float = 3.0
    description: str = ""
    weight_key: tuple = None   # seed words of the expert weights (default: seed_key)

    @property
    def weight_seed_key(self) -> tuple:
        return self.weight_key if self.weight_key is not None else self.seed_key

    @property
    def E(self) -> int:
        return self.N + self.Z

    @property
    def router_std(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def target_share(self):
        if self.bias[0] in ("uniform+shift",):
            return self.bias[2]
        if self.bias[0] == "zipf+shift":
            return self.bias[4]
        if self.bias[0] == "exclude_zero":
            return 0.0
        return None

    @property
    def tuned(self) -> bool:
        """True when the bias carries an offline-tuned zero-expert shift."""
        return self.bias[0] in ("uniform+shift", "zipf+shift")

    def weight_bytes(self) -> int:
        es = 4 if self.dtype == "f32" else 2
        return 3 * self.N * self.I * self.d * es


def _tiny() -> Workload:
    return Workload(
        name="tiny", T=64, d=128, N=8, Z=4, K=2, I=256, dtype="f32", seed_key=(0,),
        # N(0, 0.02) is read with 0.02 as the variance, like N(0, 1/d) beside it.
        expert_std=math.sqrt(0.02), bias=("uniform", 0.1),
        description="tiny fp32 layer T=64 d=128 N=8 Z=4 K=2 I=256")


def _small() -> Workload:
    return Workload(
        name="small", T=4096, d=2048, N=64, Z=32, K=6, I=1024, dtype="bf16", seed_key=(1,),
        expert_std=1.0 / math.sqrt(2048), bias=("uniform", 0.05),
        description="small bf16 layer T=4096 d=2048 N=64 Z=32 K=6 I=1024")


PREFILL_SEED = (2,)


def _prefill() -> Workload:
    E = 768
    return Workload(
        name="prefill", T=16384, d=6144, N=512, Z=256, K=12, I=2048, dtype="bf16",
        seed_key=PREFILL_SEED, expert_std=1.0 / math.sqrt(6144),
        bias=("uniform+shift", 0.1 / E, 1.0 / 3.0),
        description="prefill bf16 layer T=16384 d=6144 N=512 Z=256 K=12 I=2048, "
                    "mean 8 FFN experts per token")


def decode(T: int, share_pct: int) -> Workload:
    """Decode-step workload: the prefill layer itself (same expert weights) run on a batch
    of T in {64,128,256} tokens; its own tokens, router weights and biases."""
    E = 768
    a = 0.1 / E
    bias = ("exclude_zero", a) if share_pct == 0 else ("uniform+shift", a, share_pct / 100.0)
    return Workload(
        name=f"decode_T{T}_z{share_pct}", T=T, d=6144, N=512, Z=256, K=12, I=2048,
        dtype="bf16", seed_key=(3, T, share_pct), expert_std=1.0 / math.sqrt(6144),
        bias=bias, weight_key=PREFILL_SEED,
        description=f"decode bf16 layer T={T} d=6144 N=512 Z=256 K=12 I=2048, "
                    f"zero-expert share {share_pct}%")


def _skewed() -> Workload:
    E = 384
    return Workload(
        name="skewed", T=32768, d=4096, N=256, Z=128, K=8, I=1536, dtype="bf16",
        seed_key=(4,), expert_std=1.0 / math.sqrt(4096),
        bias=("zipf+shift", 1.1, 7.68 / E, 0.1 / E, 1.0 / 3.0), plant_frac=0.01,
        description="skewed bf16 layer T=32768 d=4096 N=256 Z=128 K=8 I=1536, "
                    "Zipf(1.1) FFN bias, 1% easy and 1% hard tokens")


DECODE_T = (64, 128, 256)
DECODE_SHARES = (0, 33, 66)


def all_workloads() -> dict:
    w = {"tiny": _tiny(), "small": _small(), "prefill": _prefill(), "skewed": _skewed()}
    for T in DECODE_T:
        for s in DECODE_SHARES:
            dw = decode(T, s)
            w[dw.name] = dw
    return w


WORKLOADS = all_workloads()


def get(name: str) -> Workload:
    return WORKLOADS[name]
