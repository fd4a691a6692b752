"""A ZeroOptimizer over the C ABI, with the interface of "Data parallelism and
ZeRO stages 1 to 3" (openlearn L11.3), section "4. The interface":
ZeroOptimizer(..., stage, **kw) with step(), zero_grad(), gather() and
memory_bytes().

On one GPU the N logical workers share one HBM, so the optimizer keeps:
  * one flat gathered parameter buffer in parameters() order; each model
    parameter becomes a view of its slice (so the model reads the gathered
    result directly, and no tensor can be unflattened out of order);
  * one flat gradient buffer per logical worker, with per-parameter views
    (worker_grads(k)) that worker k's backward pass (or a copy) fills;
  * the optimizer state as flat device buffers (fp32 master in mixed precision,
    m, v), each worker's shard being its [a_r, b_r) view.
step() runs one fused zero_step over all of it; step(max_norm=...) first clips
the averaged gradient by its global norm (the same page, section "Going
further": a sum of the chunks' squared norms before the update). The stage only
changes the memory model (memory_bytes), as on the pages: sharding moves
storage between ranks and leaves the arithmetic unchanged, except that stage 1
keeps the averaged full gradient (what the pages leave in .grad): the step
stores it in the same pass (zero_step_with_mean) for 1, 2, 4 or 8 workers, and
for other worker counts runs the mean pass and then the step from that mean
(zero_mean_grad, zero_step_mean: the same result, faster there); averaged_grad()
returns it.

This module is argument marshalling only: every step of the computation runs
in libzero.so's HIP kernels.
"""
from typing import Dict, List, Optional, Sequence

import zero_sharded_optimizer_amd as z

# worker counts the fused step is specialised for; other counts take its any-N path
_FUSED_N = (1, 2, 4, 8)

_MODE_DTYPE = {"fp64": (z.ZERO_MODE_F64, "float64", "float64"),
               "fp32": (z.ZERO_MODE_F32, "float32", "float32"),
               "bf16": (z.ZERO_MODE_MIXED_BF16, "bfloat16", "float32"),
               "fp16": (z.ZERO_MODE_MIXED_F16, "float16", "float32")}


class ZeroOptimizer:
    """ZeRO-sharded Adam/AdamW (or momentum SGD) over N logical workers on one GPU.

    params: the model's parameters (device tensors of the mode's parameter
        dtype), in parameters() order.
    n_workers: N, the logical data-parallel workers (ranks).
    stage: 1, 2 or 3 (0, 4 and no parameters are rejected, as the pages do).
    precision: "fp64", "fp32", "bf16" or "fp16" (the latter two with an fp32
        master, m and v).
    optimizer: "adamw" (lr, betas, eps, weight_decay) or "sgd" (lr, momentum,
        dampening, nesterov, weight_decay). No hyperparameter has a hidden
        default inside the library; the keyword defaults here are torch's.
    decay: None (decay everything when weight_decay > 0) or one bool per
        parameter tensor (e.g. 2-D tensors only).
    keep_averaged_grad: store the averaged gradient during each step (n more
        values of the state dtype in memory, sizeof(state) more bytes per
        parameter per step). None: on in stage 1, whose ranks keep the full
        averaged gradient in .grad, off in stages 2 and 3, which keep only
        their chunk of it.
    """

    def __init__(self, params: Sequence, n_workers: int, stage: int, precision: str = "fp32",
                 optimizer: str = "adamw", lr: float = 1e-3, betas=(0.9, 0.999),
                 eps: float = 1e-8, weight_decay: float = 0.0, momentum: float = 0.0,
                 dampening: float = 0.0, nesterov: bool = False,
                 decay: Optional[Sequence[bool]] = None,
                 keep_averaged_grad: Optional[bool] = None):
        params = list(params)
        if stage not in (1, 2, 3):
            raise ValueError(f"stage must be 1, 2 or 3, got {stage}")
        if not params:
            raise ValueError("no parameters")
        if n_workers < 1 or n_workers > z.ZERO_MAX_WORKERS:
            raise ValueError(f"n_workers must be in [1, {z.ZERO_MAX_WORKERS}], got {n_workers}")
        if precision not in _MODE_DTYPE:
            raise ValueError(f"precision must be one of {sorted(_MODE_DTYPE)}")
        if optimizer not in ("adamw", "sgd"):
            raise ValueError("optimizer must be 'adamw' or 'sgd'")
        if decay is not None and len(decay) != len(params):
            raise ValueError("decay: one flag per parameter tensor")
        if len({id(p) for p in params}) != len(params):
            raise ValueError("a parameter appears more than once")
        spans = sorted((p.data_ptr(), p.data_ptr() + p.numel() * p.element_size(), i)
                       for i, p in enumerate(params) if p.numel())
        for (_, hi, i), (lo, _, j) in zip(spans, spans[1:]):
            if lo < hi:  # each becomes its own slice of the gathered buffer: a tie would break
                raise ValueError(f"params[{i}] and params[{j}] share memory")
        import torch
        mode, pdt, sdt = _MODE_DTYPE[precision]
        pdt, sdt = getattr(torch, pdt), getattr(torch, sdt)
        for i, p in enumerate(params):
            if not p.is_cuda or p.dtype != pdt:
                raise ValueError(f"params[{i}]: expected a GPU tensor of {pdt}")
            if p.device != params[0].device:
                raise ValueError(f"params[{i}] is on {p.device}, params[0] on {params[0].device}")
        self.stage, self.n_workers, self.mode = stage, n_workers, mode
        self.params = params
        self.sizes = [p.numel() for p in params]
        self.offsets = [sum(self.sizes[:i]) for i in range(len(params))]
        n = sum(self.sizes)
        self.n = n
        dev = params[0].device
        # the gathered buffer; each parameter becomes a view of its slice
        self.flat = torch.empty(n, dtype=pdt, device=dev)
        for p, off, size in zip(params, self.offsets, self.sizes):
            self.flat[off:off + size].copy_(p.detach().reshape(-1))
            p.data = self.flat[off:off + size].view_as(p)
        self.grads = [torch.zeros(n, dtype=pdt, device=dev) for _ in range(n_workers)]
        sgd = optimizer == "sgd"
        mixed = mode in (z.ZERO_MODE_MIXED_BF16, z.ZERO_MODE_MIXED_F16)
        self.states = z.States(torch.empty(n, dtype=sdt, device=dev) if mixed else None,
                               torch.empty(n, dtype=sdt, device=dev),
                               None if sgd else torch.empty(n, dtype=sdt, device=dev))
        mask = None
        if decay is not None and weight_decay:
            flags = torch.zeros(n, dtype=torch.bool)
            for f, off, size in zip(decay, self.offsets, self.sizes):
                if f:
                    flags[off:off + size] = True
            mask = z.wd_mask_from_flags(flags, device=dev)
        self.hp = z.HParams(n=n, n_workers=n_workers, mode=mode, lr=lr, beta1=betas[0],
                            beta2=betas[1], eps=eps, weight_decay=weight_decay, wd_mask=mask,
                            optimizer=z.ZERO_OPT_SGD if sgd else z.ZERO_OPT_ADAM,
                            momentum=momentum, dampening=dampening, nesterov=nesterov)
        z.zero_init_states(self.hp, self.flat, self.states)
        self.t = 0
        self._clip_ws = None   # the clipped step's workspace, allocated on first use
        self._sumsq = None     # device double: the last clipped step's squared norm
        keep = stage == 1 if keep_averaged_grad is None else bool(keep_averaged_grad)
        # the averaged gradient of the last step (stage 1's .grad), or None
        self._mean = torch.empty(n, dtype=sdt, device=dev) if keep else None
        self._mean_valid = False

    # -- the training step ------------------------------------------------------
    def worker_grads(self, k: int) -> List:
        """Per-parameter views of worker k's flat gradient buffer (shapes of the
        parameters), to be filled by that worker's backward pass or a copy."""
        g = self.grads[k]
        return [g[off:off + size].view_as(p)
                for p, off, size in zip(self.params, self.offsets, self.sizes)]

    def state_shards(self) -> List:
        """Worker r's (m_shard, v_shard), as views (see state_shards)."""
        return state_shards(self.states, self.n_workers)

    def zero_grad(self) -> None:
        for g in self.grads:
            g.zero_()
        self._mean_valid = False

    def gather(self) -> None:
        """Stage 3's gather of the full parameters before forward. On one GPU every
        worker reads the one gathered buffer, so there is nothing to move."""

    def step(self, max_norm: Optional[float] = None, stream=None) -> None:
        """One fused step (reduce-scatter mean, Adam/SGD on each shard,
        all-gather) over the workers' gradient buffers, enqueued on `stream`.
        With max_norm, the averaged gradient is first scaled by
        min(1, max_norm / (norm + 1e-6)), its global norm taken over every shard;
        grad_norm() then returns that norm. With keep_averaged_grad, the
        averaged gradient (before clipping) is stored as well. The step count
        advances only when the call is accepted."""
        t = self.t + 1
        keep = self._mean is not None
        self._mean_valid = False
        if max_norm is None:
            if keep and self.n_workers not in _FUSED_N:
                # any other worker count: the mean pass, then the step from the
                # stored mean (bit for bit the same result; at N = 64 on MI355X
                # 6 % faster than the any-N fused step with its mean store)
                z.zero_mean_grad(self.hp, self.grads, self._mean, stream=stream)
                z.zero_step_mean(self.hp, self.flat, self._mean, self.states, t, stream=stream)
            elif keep:
                z.zero_step_with_mean(self.hp, self.flat, self.grads, self.states, t, self._mean,
                                      stream=stream)
            else:
                z.zero_step(self.hp, self.flat, self.grads, self.states, t, stream=stream)
        else:
            import torch
            if self._sumsq is None:
                self._sumsq = torch.zeros(1, dtype=torch.float64, device=self.flat.device)
            if keep:
                # the clipped step's own two launches, with the mean kept in place
                # of the workspace: the mean and its squared norm, then the step
                if self._clip_ws is None:
                    nbytes = max(1, z.zero_mean_grad_workspace_bytes(self.hp))
                    self._clip_ws = torch.empty(nbytes, dtype=torch.uint8,
                                                device=self.flat.device)
                z.zero_mean_grad(self.hp, self.grads, self._mean, self._sumsq, self._clip_ws,
                                 stream=stream)
                z.zero_step_mean(self.hp, self.flat, self._mean, self.states, t, self._sumsq,
                                 max_norm, stream=stream)
            else:
                if self._clip_ws is None:
                    nbytes = z.zero_step_clipped_workspace_bytes(self.hp)
                    self._clip_ws = torch.empty(nbytes, dtype=torch.uint8,
                                                device=self.flat.device)
                z.zero_step_clipped(self.hp, self.flat, self.grads, self.states, t, max_norm,
                                    self._clip_ws, sumsq_out=self._sumsq, stream=stream)
        self.t = t
        self._mean_valid = keep

    def buckets(self, bucket_bytes: int = 25 << 20) -> List:
        """(begin, end) buckets of about bucket_bytes of one worker's gradient
        (25 MiB by default, the DDP bucket size "Data Parallelism & ZeRO" names),
        last bucket first: the order in which a backward pass finishes them. Each
        begin is a multiple of 8 elements, as zero_step_buckets requires."""
        esize = self.grads[0].element_size()
        size = max(8, bucket_bytes // esize // 8 * 8)
        edges = list(range(0, self.n, size)) + [self.n]
        return list(reversed(list(zip(edges[:-1], edges[1:]))))

    def step_buckets(self, buckets: Sequence, events: Optional[Sequence] = None,
                     stream=None) -> None:
        """The same step as step(), bucket by bucket in one call
        (zero_step_buckets): bucket i first waits on the device for events[i] (a
        recorded torch.cuda.Event, e.g. after the gradient producer wrote that
        bucket, or None), so the step of early buckets overlaps the production
        of later ones. The buckets must cover [0, n) once; the result is bit for
        bit that of step()."""
        covered = sorted((int(a), int(b)) for a, b in buckets)
        pos = 0
        for a, b in covered:
            if a != pos or b < a:
                raise ValueError("buckets must cover [0, n) exactly once")
            pos = b
        if pos != self.n:
            raise ValueError("buckets must cover [0, n) exactly once")
        t = self.t + 1
        self._mean_valid = False
        z.zero_step_buckets(self.hp, self.flat, self.grads, self.states, t, buckets,
                            events, stream=stream)
        self.t = t

    def grad_norm(self) -> float:
        """The global norm of the averaged gradient of the last clipped step
        (waits for that step to finish)."""
        if self._sumsq is None:
            raise RuntimeError("grad_norm: no clipped step has run")
        return float(self._sumsq.item()) ** 0.5

    def averaged_grad(self, stream=None):
        """The averaged full gradient (1/N) sum_k g_k as a flat device tensor of
        the state dtype: what stage 1 leaves in .grad until zero_grad(). After a
        step() with keep_averaged_grad, it is the buffer that step stored (valid
        until the next step or zero_grad()); otherwise a new
        tensor from a separate pass over the workers' gradients
        (zero_mean_grad). Both use the step's rank-order fold and division, so
        either is bit-identical to the gradient the step used."""
        if self._mean_valid:
            return self._mean
        import torch
        mean = torch.empty(self.n, dtype=self.states.m.dtype, device=self.flat.device)
        z.zero_mean_grad(self.hp, self.grads, mean, stream=stream)
        return mean

    # -- memory and checkpoints -------------------------------------------------
    def memory_bytes(self, rank: int = 0, convention: int = 0) -> Dict[str, int]:
        """Rank `rank`'s bytes at this stage: params, grads, optimizer, by the
        closed forms (convention 0) or the emulation's bookkeeping (convention 1,
        fp64/fp32 only), as zero_memory_bytes defines them."""
        d = z.zero_memory_bytes(self.n, self.n_workers, rank, self.stage, self.mode, convention)
        return {k: d[k] for k in ("params", "grads", "optimizer")}

    def state_dict(self) -> Dict:
        """The step count and device copies of the gathered parameters and state."""
        s = self.states
        return {"t": self.t, "param": self.flat.clone(),
                "master": None if s.master is None else s.master.clone(),
                "m": s.m.clone(), "v": None if s.v is None else s.v.clone()}

    def load_state_dict(self, sd: Dict) -> None:
        """Restore a state_dict() of an optimizer of the same shape; checks every
        entry before it copies any."""
        s = self.states
        pairs = [(self.flat, sd["param"], "param")]
        pairs += [(getattr(s, k), sd[k], k) for k in ("master", "m", "v")]
        for dst, src, name in pairs:
            if (dst is None) != (src is None):
                raise ValueError(f"state_dict: {name} does not match this optimizer")
            if dst is not None and (src.dtype != dst.dtype or src.numel() != dst.numel()):
                raise ValueError(f"state_dict: {name} has another dtype or size")
        self.t = int(sd["t"])
        for dst, src, _ in pairs:
            if dst is not None:
                dst.copy_(src)


def state_shards(states: z.States, n_workers: int) -> List:
    """The N per-worker (m_shard, v_shard) pairs of "ZeRO-Sharded Adam Step",
    section "What to implement": worker r's pair is the [a_r, b_r) view of the
    flat m and v (np.array_split bounds), so each stays the size of its shard
    and no memory is copied. v is None for momentum SGD."""
    n = states.m.numel()
    out = []
    for r in range(n_workers):
        a, b = z.zero_shard_bounds(n, n_workers, r)
        out.append((states.m[a:b], None if states.v is None else states.v[a:b]))
    return out


def init_states(n_params: int, n_workers: int, device="cuda", precision: str = "fp32",
                param=None) -> z.States:
    """init_states ("ZeRO-Sharded Adam Step", section "What to implement"): the
    workers' (m, v) shards as flat buffers of zeros (and, in mixed precision,
    the fp32 master copied from `param`)."""
    import torch
    mode, _, sdt = _MODE_DTYPE[precision]
    sdt = getattr(torch, sdt)
    mixed = mode in (z.ZERO_MODE_MIXED_BF16, z.ZERO_MODE_MIXED_F16)
    if mixed and param is None:
        raise ValueError("mixed precision: pass param to set the master copy")
    st = z.States(torch.empty(n_params, dtype=sdt, device=device) if mixed else None,
                  torch.empty(n_params, dtype=sdt, device=device),
                  torch.empty(n_params, dtype=sdt, device=device))
    hp = z.HParams(n=n_params, n_workers=n_workers, mode=mode, lr=0.0, beta1=0.9, beta2=0.999,
                   eps=1e-8)
    z.zero_init_states(hp, param, st)
    return st


def zero_step(param, grads: Sequence, states: z.States, t: int, lr: float = 1e-2,
              betas=(0.9, 0.999), eps: float = 1e-8, weight_decay: float = 0.0,
              precision: str = "fp32"):
    """zero_step ("ZeRO-Sharded Adam Step", section "What to implement"), the
    functional form: returns (new_param, new_states) and leaves its inputs as
    they were. lr defaults to the page's 1e-2."""
    new_param = param.clone()
    new_states = z.States(None if states.master is None else states.master.clone(),
                          states.m.clone(), states.v.clone())
    mode = _MODE_DTYPE[precision][0]
    hp = z.HParams(n=param.numel(), n_workers=len(grads), mode=mode, lr=lr, beta1=betas[0],
                   beta2=betas[1], eps=eps, weight_decay=weight_decay)
    z.zero_step(hp, new_param, list(grads), new_states, t)
    return new_param, new_states
