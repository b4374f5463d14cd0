"""The five workloads of the ZeRO-1 shard step, as shapes and distributions.

Every workload is seeded synthetic data (seed = 1000 + workload index); no
dataset or trained weight is involved. "N(0, x)" means a zero-mean
distribution of standard deviation x; the generator is the Irwin-Hall-of-8
approximation described in synth_host.c. The model names only give shapes.

Sizes follow the pages' example of a 7.5B-parameter model on 64 ranks
("CS336 Lecture 7: Parallelism 1", section "训练内存的详细分析") and common
GPT-2-small and Llama-7B layer shapes.
"""
from __future__ import annotations

import dataclasses
from typing import List

ADAMW = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


@dataclasses.dataclass(frozen=True)
class TensorSpec:
    name: str
    full: int    # elements of the whole (unsharded) tensor or bucket
    start: int   # first element of this rank's shard within it
    n: int       # elements of the shard
    tensor_id: int


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int
    name: str
    M: int
    tensors: List[TensorSpec]
    grad_std: float
    master_std: float
    m_std: float        # 0: zeros
    v_std: float        # 0: zeros; otherwise |N(0, v_std)|
    step: int
    max_grad_norm: float
    grad_scale: float
    skip_on_nonfinite: int
    inject_rate: float  # per replica element, on odd runs; 0: never
    full_replicas: bool  # replicas hold the whole bucket (shard read at an offset)

    @property
    def seed(self) -> int:
        return 1000 + self.index

    @property
    def n_total(self) -> int:
        return sum(t.n for t in self.tensors)

    @property
    def two_pass(self) -> bool:
        return self.max_grad_norm > 0 or bool(self.skip_on_nonfinite)

    def bytes_per_param(self) -> int:
        """Algorithmic HBM bytes per shard parameter: M bf16 replica reads,
        fp32 master/m/v read and written, bf16 emit; plus the fp32 reduced
        gradient written and read back once when clipping or skipping needs
        the global norm before any update."""
        return 2 * self.M + 26 + (8 if self.two_pass else 0)

    def hparams(self) -> dict:
        return dict(ADAMW, step=self.step, max_grad_norm=self.max_grad_norm, grad_scale=self.grad_scale,
                    skip_on_nonfinite=self.skip_on_nonfinite)


def _shard(full: int, M: int, r: int):
    per = -(-full // M)
    s = min(full, r * per)
    e = min(full, (r + 1) * per)
    return s, e - s


def _llama_layers(M: int, rank: int, layers: int = 32, hidden: int = 4096, inter: int = 11008):
    out = []
    tid = 0
    for layer in range(layers):
        shapes = [("q", hidden * hidden), ("k", hidden * hidden), ("v", hidden * hidden), ("o", hidden * hidden),
                  ("gate", hidden * inter), ("up", hidden * inter), ("down", inter * hidden),
                  ("attn_norm", hidden), ("mlp_norm", hidden)]
        for nm, full in shapes:
            s, n = _shard(full, M, rank)
            out.append(TensorSpec(f"layers.{layer}.{nm}", full, s, n, tid))
            tid += 1
    return out


def workload(i: int) -> Workload:
    if i == 0:
        full, M = 1_048_576, 4
        s, n = _shard(full, M, 0)
        return Workload(0, "tiny single tensor, N=1,048,576, M=4, shard 0", M, [TensorSpec("w", full, s, n, 0)],
                        1e-3, 0.02, 0.0, 0.0, 1, 0.0, 1.0, 0, 0.0, True)
    if i == 1:
        full, M = 124_439_808, 8
        s, n = _shard(full, M, 3)
        return Workload(1, "GPT-2-small flat bucket, 124,439,808 params, M=8, shard 3", M,
                        [TensorSpec("bucket", full, s, n, 0)], 1e-4, 0.02, 1e-5, 1e-8, 100, 1.0, 1.0, 0, 0.0, True)
    if i == 2:
        M = 64
        n = 7_500_000_000 // M
        return Workload(2, "7.5B params at 64-way ZeRO-1, one rank's 117,187,500-param shard, M=64", M,
                        [TensorSpec("shard", 7_500_000_000, 0, n, 0)], 1e-4, 0.02, 1e-5, 1e-8, 1000, 0.0, 1.0,
                        0, 0.0, False)
    if i == 3:
        M = 8
        return Workload(3, "ragged Llama-7B-shaped bucket, 32 layers x 9 tensors, M=8, shard 7", M,
                        _llama_layers(M, 7), 1e-4, 0.02, 1e-5, 1e-8, 10, 0.0, 1.0, 0, 0.0, False)
    if i == 4:
        M = 8
        return Workload(4, "AMP edge path, 2e9-param shard, M=8, grads scaled by 65536", M,
                        [TensorSpec("shard", 2_000_000_000 * M, 0, 2_000_000_000, 0)], 1e-4 * 65536, 0.02, 1e-5,
                        1e-8, 5000, 1.0, 2.0**-16, 1, 1e-9, False)
    raise ValueError(i)


# Gradient buckets of the ZeRO-2 streaming step (gsyq.cn/news/457874 section
# 4.2: reduce_bucket_size 5e7 elements). Backward produces a layer's
# gradients in the reverse of the order the forward pass uses its tensors,
# from the last layer to the first.
REDUCE_BUCKET_ELEMS = 50_000_000
_LLAMA_FORWARD = ("attn_norm", "q", "k", "v", "o", "mlp_norm", "gate", "up", "down")


def backward_order(w: Workload) -> List[int]:
    """Tensor indices of w in the order backward produces their gradients."""
    if len(w.tensors) == 1:
        return [0]
    by_name = {t.name: i for i, t in enumerate(w.tensors)}
    layers = sorted({int(t.name.split(".")[1]) for t in w.tensors}, reverse=True)
    return [by_name[f"layers.{L}.{nm}"] for L in layers for nm in reversed(_LLAMA_FORWARD)]


def zero2_buckets(w: Workload, bucket_elems: int = REDUCE_BUCKET_ELEMS) -> List[List[int]]:
    """Tensor indices grouped into buckets in backward order; a bucket closes
    once the whole (unsharded) tensors in it reach bucket_elems elements."""
    out, cur, size = [], [], 0
    for i in backward_order(w):
        cur.append(i)
        size += w.tensors[i].full
        if size >= bucket_elems:
            out.append(cur)
            cur, size = [], 0
    if cur:
        out.append(cur)
    return out


WORKLOADS = [workload(i) for i in range(5)]
