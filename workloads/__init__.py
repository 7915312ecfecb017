"""Seeded synthetic workloads shared by the tests, the smoke check and the benchmark.

This module holds the workload shapes, the seeded input generators and the
benchmark's FLOP accounting.  It holds none of the attention arithmetic: it
never computes a score, a softmax or an output.  Both the CPU oracle and the HIP
path receive the arrays it produces; neither imports the other.

Input recipe (the pages give shapes and "i.i.d. N(0,1)" but no generator):
a CPU ``torch.Generator`` seeded ``1000 + index`` draws fp32 standard normals
in the order Q, K, V; each tensor is then cast (round-to-nearest-even) to the
workload's dtype.  The stress workload multiplies Q by 8 in fp32 before the cast
(exact: a power of two) so that logits are large.  Both sides consume the cast
values; the oracle widens them exactly to fp64.

FLOP convention of the headline metric: 4*B*H*M*N*D (two matrix products of
2*M*N*D each, as counted in Step 4 of the Module 08 page: 256,000,000 for
N = 1000, d = 64), halved for causal.  For a causal workload with M != N the
halving is not the work done, so :func:`exact_flops` counts visible pairs.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = ["Workload", "WORKLOADS", "BENCH_WORKLOAD", "make_inputs", "make_inputs_device",
           "make_dout_device", "sample_rows",
           "metric_flops", "visible_pairs", "exact_flops", "compulsory_bytes", "DTYPE_CODES",
           "ELT_BYTES"]

# dtype codes of the C ABI (fa_dtype_t)
DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2}
ELT_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    M: int
    N: int
    D: int
    dtype: str          # "f32" | "f16" | "bf16"
    causal: bool
    scale: float
    seed: int
    q_mult: float = 1.0

    def shape_q(self):
        return (self.B, self.H, self.M, self.D)

    def shape_kv(self):
        return (self.B, self.H, self.N, self.D)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _inv_sqrt(d: int) -> float:
    return 1.0 / math.sqrt(d)


WORKLOADS = {
    # single head, no batch: Q 256x64, K/V 1024x64, fp32, non-causal
    "single_head_f32": Workload("single_head_f32", 1, 1, 256, 1024, 64, "f32", False,
                                _inv_sqrt(64), 1001),
    # GPT-2-medium-shaped forward
    "gpt2_medium_f16": Workload("gpt2_medium_f16", 64, 16, 1024, 1024, 64, "f16", False,
                                1.0 / 8.0, 1002),
    # causal LLM prefill, N = 4096, d = 128 (the headline workload)
    "causal_prefill_bf16": Workload("causal_prefill_bf16", 8, 32, 4096, 4096, 128, "bf16", True,
                                    _inv_sqrt(128), 1003),
    # stress: ragged M, N; D = 96; Q * 8 (large logits); non-causal and causal bottom-right
    "stress_f16": Workload("stress_f16", 4, 12, 1000, 3000, 96, "f16", False,
                           _inv_sqrt(96), 1004, 8.0),
    "stress_f16_causal": Workload("stress_f16_causal", 4, 12, 1000, 3000, 96, "f16", True,
                                  _inv_sqrt(96), 1004, 8.0),
    # stress edge: M > N causal bottom-right -> rows 0..1999 see no key
    "stress_f16_causal_mgtn": Workload("stress_f16_causal_mgtn", 4, 12, 3000, 1000, 96, "f16",
                                       True, _inv_sqrt(96), 1004, 8.0),
    # long context: N = 65536 causal, linear memory
    "long_context_bf16": Workload("long_context_bf16", 1, 16, 65536, 65536, 128, "bf16", True,
                                  _inv_sqrt(128), 1005),
}

# The workload the headline throughput metric is quoted on.
BENCH_WORKLOAD = "causal_prefill_bf16"


def make_inputs(w: Workload):
    """Seeded Q, K, V as CPU torch tensors of the workload's dtype ([B,H,M|N,D])."""
    import torch

    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    q = torch.randn(w.shape_q(), generator=g, dtype=torch.float32)
    if w.q_mult != 1.0:
        q.mul_(w.q_mult)
    k = torch.randn(w.shape_kv(), generator=g, dtype=torch.float32)
    v = torch.randn(w.shape_kv(), generator=g, dtype=torch.float32)
    return q.to(tdt), k.to(tdt), v.to(tdt)


def make_inputs_device(w: Workload, device):
    """Seeded Q, K, V generated directly on a GPU, for shapes too large to draw
    on the host in seconds (tensors beyond 2^31 elements).  Same recipe as
    :func:`make_inputs` (fp32 standard normals in the order Q, K, V, then a
    round-to-nearest-even cast) but from a device ``torch.Generator`` seeded
    ``w.seed``, so the values differ from :func:`make_inputs`'.  Callers copy the
    heads they check to the host for the oracle."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(w.seed)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    out = []
    for shape in (w.shape_q(), w.shape_kv(), w.shape_kv()):
        x = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
        if w.q_mult != 1.0 and not out:
            x.mul_(w.q_mult)
        out.append(x.to(tdt))
        del x
    return tuple(out)


def make_dout_device(w: Workload, device):
    """Seeded incoming gradient drawn on a GPU (device generator seeded
    ``w.seed + 500000``), the large-shape counterpart of :func:`make_dout`."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(w.seed + 500000)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    return torch.randn(w.shape_q(), generator=g, dtype=torch.float32, device=device).to(tdt)


def make_dout(w: Workload):
    """Seeded incoming gradient dL/dO for the backward pass: N(0,1) of the
    workload's dtype, shape [B,H,M,D], from its own generator (seed + 500000)
    so that Q, K, V are the same as the forward workload's."""
    import torch

    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed + 500000)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    return torch.randn(w.shape_q(), generator=g, dtype=torch.float32).to(tdt)


def sample_rows(M: int, head: int, n: int = 256, seed_base: int = 5000) -> np.ndarray:
    """Seeded sample of query rows for one head (sorted, unique).

    Rows 0..15 and M-16..M-1 are always included (the first causal rows average
    few keys and have the largest |O|); the rest are drawn uniformly without
    replacement from the middle with ``numpy.random.default_rng(seed_base + head)``.
    """
    if M <= n:
        return np.arange(M)
    edge = np.concatenate([np.arange(16), np.arange(M - 16, M)])
    rng = np.random.default_rng(seed_base + head)
    mid = rng.choice(np.arange(16, M - 16), size=n - 32, replace=False)
    return np.sort(np.concatenate([edge, mid]))


def visible_pairs(M: int, N: int, causal: bool) -> int:
    """Number of (query, key) pairs the mask lets through, for one head.

    Causal (bottom-right): row i sees keys 0 .. i + N - M, clipped to [0, N].
    """
    if not causal:
        return M * N
    total = 0
    off = N - M
    # rows with 0 < i + off + 1 < N see i + off + 1 keys; later rows see all N
    i_full = max(0, min(M, N - off - 1))       # first row that sees every key
    i_any = max(0, min(M, -off))               # first row that sees any key
    if i_full > i_any:
        a, b = i_any + off + 1, i_full - 1 + off + 1
        total += (a + b) * (i_full - i_any) // 2
    total += (M - max(i_full, i_any)) * N if M > max(i_full, i_any) else 0
    return total


def metric_flops(B, H, M, N, D, causal) -> float:
    """Headline FLOP count: 4*B*H*M*N*D, halved for causal."""
    f = 4.0 * B * H * M * N * D
    return f / 2.0 if causal else f


def exact_flops(B, H, M, N, D, causal) -> float:
    """4*D FLOP per visible (query, key) pair, summed over heads."""
    return 4.0 * D * B * H * visible_pairs(M, N, causal)


def compulsory_bytes(w: Workload) -> int:
    """Bytes the forward pass must move: read Q, K, V once; write O and fp32 LSE."""
    e = ELT_BYTES[w.dtype]
    return (w.B * w.H * (2 * w.M * w.D + 2 * w.N * w.D) * e) + 4 * w.B * w.H * w.M
