"""Seeded synthetic inputs for the fused ZeRO Adam step.

Only input generation lives here (parameters, per-worker gradients, decay
flags, tensor lists); none of the step's arithmetic. Tests, the smoke check and
the benchmark draw from these generators and hand copies of the same values to
both the HIP path and the CPU oracle.

Distributions: "N(0, s)" means standard deviation s. Draw order is fixed:
parameters (or master), then per-worker scales, then for each step t and each
worker k in rank order, worker k's gradient; each draw comes from a generator
seeded with (seed, t, k) so that any step can be regenerated on its own.
"""
from dataclasses import dataclass, field, replace
from typing import List, Optional, Tuple

import numpy as np

MODE_F64, MODE_F32, MODE_MIXED, MODE_MIXED_F16 = 0, 1, 2, 3


@dataclass(frozen=True)
class Workload:
    name: str
    mode: int
    n: int                 # parameters in the gathered vector
    n_workers: int
    lr: float
    beta1: float
    beta2: float
    eps: float
    weight_decay: float
    steps: int             # steps the workload is defined for (t = 1..steps)
    param_std: float
    grad_std: float
    rank: int = -1         # -1: all workers in one call; r: worker r's share only
    worker_scale: Optional[Tuple[float, float]] = None  # per-worker U(lo, hi) scale
    zero_frac: float = 0.0  # fraction of gradient entries set exactly to 0
    decay: str = "none"    # "none", "all", "2d" (2-D tensors of `shapes` only)
    shapes: Tuple[Tuple[int, ...], ...] = field(default=())
    seed: int = 0

    @property
    def shard(self):
        """[a, b) of the elements this call updates: the bounds of
        np.array_split(np.arange(n), N)[rank], which the input recipe needs to
        draw a rank's gradient chunks (tests check it against numpy itself)."""
        if self.rank < 0:
            return 0, self.n
        q, rho = divmod(self.n, self.n_workers)
        a = self.rank * q + min(self.rank, rho)
        return a, a + q + (1 if self.rank < rho else 0)

    @property
    def length(self):
        a, b = self.shard
        return b - a


def gpt2_small_shapes(vocab=50257, ctx=1024, d=768, layers=12):
    """Parameter shapes of a GPT-2-small-shaped model in parameters() order, with
    the output head tied to the token embedding."""
    shapes = [(vocab, d), (ctx, d)]
    for _ in range(layers):
        shapes += [(d,), (d,), (d, 3 * d), (3 * d,), (d, d), (d,), (d,), (d,),
                   (d, 4 * d), (4 * d,), (4 * d, d), (d,)]
    shapes += [(d,), (d,)]
    return tuple(shapes)


def tensor_starts(shapes):
    out, pos = [], 0
    for s in shapes:
        out.append(pos)
        pos += int(np.prod(s))
    return out, pos


_GPT2 = gpt2_small_shapes()

# The workloads, named by what they are. Sizes and hyperparameters as stated for
# each; readings of unstated values are listed in the design notes.
WORKLOADS = {
    "fp64-1M-n4": Workload(
        "fp64-1M-n4", MODE_F64, 1_048_579, 4, 1e-2, 0.9, 0.999, 1e-8, 0.0, 10,
        param_std=1.0, grad_std=1.0, seed=20260001),
    "fp32-320M-n8": Workload(
        "fp32-320M-n8", MODE_F32, 320_000_000, 8, 3e-4, 0.9, 0.95, 1e-8, 0.0, 20,
        param_std=0.02, grad_std=1e-3, worker_scale=(0.5, 2.0), seed=20260002),
    "mixed-1B-n8": Workload(
        "mixed-1B-n8", MODE_MIXED, 1_000_000_000, 8, 1e-4, 0.9, 0.95, 1e-8, 0.0, 10,
        param_std=0.02, grad_std=1e-3, zero_frac=0.01, seed=20260003),
    "mixed-rank0-of-8B-n8": Workload(
        "mixed-rank0-of-8B-n8", MODE_MIXED, 8_000_000_000, 8, 3e-4, 0.9, 0.95, 1e-8, 0.1, 5,
        param_std=0.02, grad_std=1e-3, rank=0, decay="all", seed=20260004),
    "mixed-fp16-1B-n8": Workload(
        "mixed-fp16-1B-n8", MODE_MIXED_F16, 1_000_000_000, 8, 1e-4, 0.9, 0.95, 1e-8, 0.0, 10,
        param_std=0.02, grad_std=1e-3, zero_frac=0.01, seed=20260006),
    "gpt2s-fp32-n64": Workload(
        "gpt2s-fp32-n64", MODE_F32, tensor_starts(_GPT2)[1], 64, 3e-4, 0.9, 0.95, 1e-8, 0.1,
        100, param_std=0.02, grad_std=1e-3, decay="2d", shapes=_GPT2, seed=20260005),
}


def scaled(wl: Workload, n: int, name=None, shapes=None, **kw) -> Workload:
    """The same workload at another size (for oracle-sized parity cases)."""
    if shapes:
        n = tensor_starts(shapes)[1]
    shapes = wl.shapes if shapes is None else tuple(shapes)
    return replace(wl, n=n, name=name or f"{wl.name}@{n}", shapes=shapes, **kw)


def decay_flags(wl: Workload) -> Optional[np.ndarray]:
    """Per-element decay flags over [0, n) (bool), or None when no mask is needed."""
    if wl.decay == "none" or wl.decay == "all":
        return None
    if wl.decay == "2d":
        flags = np.zeros(wl.n, dtype=bool)
        starts, total = tensor_starts(wl.shapes)
        assert total == wl.n
        for s, st in zip(wl.shapes, starts):
            if len(s) == 2:
                flags[st:st + int(np.prod(s))] = True
        return flags
    raise ValueError(wl.decay)


def _torch():
    import torch
    return torch


def _gen(device, *key):
    torch = _torch()
    g = torch.Generator(device=device)
    # a 63-bit seed from the key tuple; fixed arithmetic, no hashing of strings
    s = 0
    for k in key:
        s = (s * 1_000_003 + int(k) + 1) % (2 ** 63 - 1)
    g.manual_seed(s)
    return g


_CHUNK = 1 << 28


def _normal(n, std, device, gen, dtype):
    """n draws of N(0, std) in fp32 (fp64 for fp64 workloads), chunked."""
    torch = _torch()
    work_dt = torch.float64 if dtype == torch.float64 else torch.float32
    out = torch.empty(n, dtype=dtype, device=device)
    for i in range(0, n, _CHUNK):
        j = min(n, i + _CHUNK)
        x = torch.randn(j - i, generator=gen, device=device, dtype=work_dt)
        x.mul_(std)
        out[i:j] = x.to(dtype)
    return out


def param_dtype(wl):
    torch = _torch()
    return {MODE_F64: torch.float64, MODE_F32: torch.float32, MODE_MIXED: torch.bfloat16,
            MODE_MIXED_F16: torch.float16}[wl.mode]


def state_dtype(wl):
    torch = _torch()
    return torch.float64 if wl.mode == MODE_F64 else torch.float32


def make_params(wl: Workload, device="cuda"):
    """The gathered parameter vector (n elements) and, in rank mode, the rank's
    fp32/fp64 master chunk drawn N(0, param_std). In full mode the master is
    derived from the parameters by init_states, so it is returned as None.
    Elements outside the rank's shard (rank mode) are zeros."""
    torch = _torch()
    g = _gen(device, wl.seed, 0)
    if wl.rank < 0:
        return _normal(wl.n, wl.param_std, device, g, param_dtype(wl)), None
    a, b = wl.shard
    master = _normal(b - a, wl.param_std, device, g, state_dtype(wl))
    param = torch.zeros(wl.n, dtype=param_dtype(wl), device=device)
    return param, master


def worker_scales(wl: Workload):
    if wl.worker_scale is None:
        return [1.0] * wl.n_workers
    lo, hi = wl.worker_scale
    rng = np.random.default_rng(wl.seed)
    return [float(x) for x in rng.uniform(lo, hi, wl.n_workers)]


def make_grad(wl: Workload, t: int, k: int, device="cuda"):
    """Worker k's gradient at step t: n elements in full mode, the rank's chunk
    of length c_r in rank mode. N(0, grad_std * scale_k), then a zero_frac
    fraction of entries set exactly to 0 (independently per worker)."""
    torch = _torch()
    length = wl.length
    g = _gen(device, wl.seed, t, k + 1)
    scale = worker_scales(wl)[k]
    x = _normal(length, wl.grad_std * scale, device, g, param_dtype(wl))
    if wl.zero_frac > 0:
        for i in range(0, length, _CHUNK):
            j = min(length, i + _CHUNK)
            drop = torch.rand(j - i, generator=g, device=device) < wl.zero_frac
            x[i:j].masked_fill_(drop, 0)
    return x


def make_grads(wl: Workload, t: int, device="cuda") -> List:
    return [make_grad(wl, t, k, device) for k in range(wl.n_workers)]


def sample_indices(wl: Workload, count: int, seed=7) -> np.ndarray:
    """Sorted unique indices into [0, length) for sampled parity at full size:
    the first and last 4096, every shard boundary +-64, every tensor boundary
    +-64, and `count` seeded uniform draws."""
    L = wl.length
    a0, _ = wl.shard
    pts = [np.arange(0, min(L, 4096)), np.arange(max(0, L - 4096), L)]
    if wl.rank < 0:
        q, rho = divmod(wl.n, wl.n_workers)
        for r in range(1, wl.n_workers):
            s = r * q + min(r, rho)
            pts.append(np.arange(max(0, s - 64), min(L, s + 64)))
    if wl.shapes:
        for s in tensor_starts(wl.shapes)[0]:
            s -= a0
            if 0 <= s <= L:
                pts.append(np.arange(max(0, s - 64), min(L, s + 64)))
    rng = np.random.default_rng(seed)
    pts.append(rng.integers(0, L, count))
    return np.unique(np.concatenate(pts)).astype(np.int64)
