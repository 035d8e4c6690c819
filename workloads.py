"""Seeded synthetic inputs for the DeepSeekMoE layer forward.

This module only draws random tensors and holds the workload shapes.  It does
none of the layer's arithmetic: no routing, no quantisation, no GEMM.  Both the
CPU oracle (``oracle/``) and the HIP library are fed from the tensors it makes.

Workloads (shapes of the DeepSeek-V3 MoE layer: 256 routed experts, top-8, one
shared expert, tiles of 128; see "DeepSeek-V3 Technical Report" notes at
learn.ifs.name, MoE-routing and FP8 paragraphs, and the nlp-lineage summary,
"The idea"):

  tiny      T=128,   d=512,  E=16,  K=4, I=256, 1 shared
  rdc       T=8192,  d=7168, E=256, K=8, router + dispatch + permute + combine,
            identity experts, no shared term, bias update gamma=1e-3
  decode    T=256,   d=7168, E=256, K=8, I=2048, 1 shared, 0.1% outliers x100
  prefill   T=16384, d=7168, E=256, K=8, I=2048, 1 shared, 0.1% outliers x100,
            bias calibrated so the expert load is Zipf(1.1)-like, max/mean ~4
  dense     M=8192, N=7168, K in {4096, 16384}: block-scaled FP8 GEMM alone

Seeding: every tensor gets its own 63-bit seed from
numpy SeedSequence([BASE_SEED, workload_id, tensor_id, expert_id]).  On the CPU
it is drawn with numpy's PCG64 generator of that seed (activations, centroids
and biases are always drawn there: identical bytes on every machine); expert
weights that live on the GPU are drawn per expert with a torch CUDA generator
of the same seed, and tests copy the FP32 masters of the experts they check
back to the host for the oracle.
"""
from __future__ import annotations

import os
from dataclasses import dataclass, field

import numpy as np
import torch

BASE_SEED = 20241227

_WORKLOAD_IDS = {"tiny": 1, "rdc": 2, "decode": 3, "prefill": 4, "dense": 5, "custom": 9}
_TENSOR_IDS = {"u": 1, "centroids": 2, "bias": 3, "w1": 4, "w3": 5, "w2": 6,
               "outlier_pos": 7, "a": 8, "b": 9, "a_outlier": 10, "b_outlier": 11,
               "rank_perm": 12, "dh": 13}

HERE = os.path.dirname(os.path.abspath(__file__))
PREFILL_BIAS_FILE = os.path.join(HERE, "tests", "golden", "prefill_bias_zipf.txt")


@dataclass(frozen=True)
class MoEShape:
    name: str
    T: int
    d: int
    E: int
    K: int
    I: int            # expert intermediate size (0: no expert FFN, identity experts)
    shared: int       # number of shared experts (0 or 1)
    outliers: bool    # 0.1% of u entries scaled x100 before bf16 rounding
    gamma: float = 1e-3
    zipf_bias: bool = False
    extra: dict = field(default_factory=dict)


SHAPES = {
    "tiny": MoEShape("tiny", T=128, d=512, E=16, K=4, I=256, shared=1, outliers=False),
    "rdc": MoEShape("rdc", T=8192, d=7168, E=256, K=8, I=0, shared=0, outliers=False),
    "decode": MoEShape("decode", T=256, d=7168, E=256, K=8, I=2048, shared=1, outliers=True),
    "prefill": MoEShape("prefill", T=16384, d=7168, E=256, K=8, I=2048, shared=1,
                        outliers=True, zipf_bias=True),
}

DENSE = {"M": 8192, "N": 7168, "K": (4096, 16384)}


def seed_for(workload: str, tensor: str, expert: int = 0) -> int:
    wid = _WORKLOAD_IDS[workload] if workload in _WORKLOAD_IDS else _WORKLOAD_IDS["custom"]
    ss = np.random.SeedSequence([BASE_SEED, wid, _TENSOR_IDS[tensor], int(expert)])
    return int(ss.generate_state(1, np.uint64)[0] & np.uint64((1 << 63) - 1))


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


_CHUNK = 1 << 20


def _cpu_normal(shape, seed: int) -> np.ndarray:
    """Standard normals in fixed chunks of 2^20 values, chunk c drawn from
    PCG64(SeedSequence([seed, c])); the chunks are filled by a thread pool, so
    the bytes do not depend on the number of threads."""
    from concurrent.futures import ThreadPoolExecutor
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    nchunk = (n + _CHUNK - 1) // _CHUNK

    def fill(c):
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, c])))
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        rng.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])

    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(fill, range(nchunk)))
    return out.reshape(shape)


def normal(shape, std: float, seed: int, device="cpu") -> torch.Tensor:
    """FP32 N(0, std^2) drawn from a generator of the given seed (numpy PCG64
    on the CPU, torch's generator on a GPU)."""
    if torch.device(device).type == "cpu":
        x = torch.from_numpy(_cpu_normal(shape, seed))
    else:
        g = _gen(device, seed)
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def add_outliers(x: torch.Tensor, seed: int, frac: float = 1e-3, factor: float = 100.0) -> torch.Tensor:
    """Scale exactly round(frac * numel) entries, chosen uniformly without
    replacement (numpy PCG64 of the given seed), by ``factor`` (in place,
    before any rounding to bf16)."""
    n = x.numel()
    cnt = int(round(frac * n))
    if cnt == 0:
        return x
    rng = np.random.Generator(np.random.PCG64(seed))
    pos = torch.from_numpy(rng.choice(n, size=cnt, replace=False).astype(np.int64)).to(x.device)
    x.view(-1)[pos] *= factor
    return x


def activations(shape: MoEShape, workload: str | None = None) -> torch.Tensor:
    """u: bf16 [T, d] on the CPU, N(0,1) (+ outliers when the workload has them)."""
    wl = workload or shape.name
    x = normal((shape.T, shape.d), 1.0, seed_for(wl, "u"))
    if shape.outliers:
        add_outliers(x, seed_for(wl, "outlier_pos"))
    return x.to(torch.bfloat16)


def centroids(shape: MoEShape, workload: str | None = None) -> torch.Tensor:
    """Expert centroids e: bf16 [E, d] on the CPU, N(0, 1/d)."""
    wl = workload or shape.name
    return normal((shape.E, shape.d), shape.d ** -0.5, seed_for(wl, "centroids")).to(torch.bfloat16)


def uniform_bias(shape: MoEShape, workload: str | None = None) -> torch.Tensor:
    """b: FP32 [E] on the CPU, U(-0.05, 0.05)."""
    wl = workload or shape.name
    rng = np.random.Generator(np.random.PCG64(seed_for(wl, "bias")))
    return torch.from_numpy((rng.random(shape.E, dtype=np.float32) - np.float32(0.5)) * np.float32(0.1))


def load_prefill_bias() -> torch.Tensor:
    """The calibrated prefill bias (256 FP32 values stored as hex bit patterns)."""
    vals = []
    with open(PREFILL_BIAS_FILE) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            vals.append(int(line.split()[0], 16))
    return torch.tensor(np.array(vals, dtype=np.uint32).view(np.float32))


def bias(shape: MoEShape, workload: str | None = None) -> torch.Tensor:
    if shape.zipf_bias:
        return load_prefill_bias()
    return uniform_bias(shape, workload)


def expert_weights(shape: MoEShape, expert: int, device="cpu", workload: str | None = None):
    """FP32 masters of one expert (routed 0..E-1, shared = E): W1, W3 [I, d] and
    W2 [d, I], each N(0, 1/d)."""
    wl = workload or shape.name
    std = shape.d ** -0.5
    w1 = normal((shape.I, shape.d), std, seed_for(wl, "w1", expert), device)
    w3 = normal((shape.I, shape.d), std, seed_for(wl, "w3", expert), device)
    w2 = normal((shape.d, shape.I), std, seed_for(wl, "w2", expert), device)
    return w1, w3, w2


def zipf_target_profile(E: int, s: float = 1.1, q: float = 31.334190744039795) -> np.ndarray:
    """Relative load target (rank r = 1..E) proportional to (r + q)^-s, with q
    solved so that max/mean = 4 for E = 256.  Normalised to mean 1."""
    r = np.arange(1, E + 1, dtype=np.float64)
    p = (r + q) ** (-s)
    return p / p.mean()


def rank_permutation(E: int, workload: str = "prefill") -> np.ndarray:
    """Seeded map rank -> expert index for the skewed load profile."""
    rng = np.random.Generator(np.random.PCG64(seed_for(workload, "rank_perm")))
    return rng.permutation(E)


def dense_operands(M: int, N: int, K: int, device="cpu"):
    """A [M, K], B [N, K] FP32 ~ N(0,1) with 0.1% outliers x100."""
    a = normal((M, K), 1.0, seed_for("dense", "a", K), device)
    add_outliers(a, seed_for("dense", "a_outlier", K))
    b = normal((N, K), 1.0, seed_for("dense", "b", K), device)
    add_outliers(b, seed_for("dense", "b_outlier", K))
    return a, b


def custom_shape(T, d, E, K, I, shared=1, outliers=False, name="custom") -> MoEShape:
    return MoEShape(name, T=T, d=d, E=E, K=K, I=I, shared=shared, outliers=outliers)
