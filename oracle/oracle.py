"""ctypes front end of the CPU oracle (test infrastructure only).

Arrays are numpy arrays. Modes: MODE_F64 (fp64 parameters, gradients and
moments; the parameter is its own master), MODE_F32 (the same in fp32),
MODE_MIXED (bf16 parameters and gradients as uint16 bit patterns, fp32 master,
m and v) and MODE_MIXED_F16 (the same with fp16 bit patterns). Every step
function is functional: it returns new arrays and leaves
its inputs untouched, as the problem statement's zero_step returns
(new_param, new_states).
"""
import ctypes as C
import os

import numpy as np

from . import build_oracle

MODE_F64, MODE_F32, MODE_MIXED, MODE_MIXED_F16 = 0, 1, 2, 3
MIXED_MODES = (MODE_MIXED, MODE_MIXED_F16)
_PARAM_DT = {MODE_F64: np.float64, MODE_F32: np.float32, MODE_MIXED: np.uint16,
             MODE_MIXED_F16: np.uint16}
_STATE_DT = {MODE_F64: np.float64, MODE_F32: np.float32, MODE_MIXED: np.float32,
             MODE_MIXED_F16: np.float32}

_i64, _i32, _dbl, _vp = C.c_int64, C.c_int, C.c_double, C.c_void_p


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _ptr_array(arrs):
    return (C.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])


class Oracle:
    def __init__(self, path=None, mutant=0):
        if path is None:
            path = build_oracle.lib_path(mutant)
            if not os.path.exists(path):
                path = build_oracle.build(mutant)
        self.path = path
        lib = C.CDLL(path)
        self.lib = lib
        lib.orc_mutant.restype = _i32
        lib.orc_split_bounds.argtypes = [_i64, _i64, _i64, C.POINTER(_i64), C.POINTER(_i64)]
        lib.orc_owner.argtypes = [_i64, _i64, _i64]
        lib.orc_owner.restype = _i64
        lib.orc_bf16_round.argtypes = [_vp, _vp, _i64]
        lib.orc_fp16_round.argtypes = [_vp, _vp, _i64]
        lib.orc_fp16_widen.argtypes = [_vp, _vp, _i64]
        lib.orc_init_states.argtypes = [_i32, _i64, _vp, _vp, _vp, _vp]
        step_args = [_i32, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                     _i64, _dbl, _dbl, _dbl, _dbl, _dbl, _vp]
        for name in ("orc_zero_step", "orc_full_step"):
            f = getattr(lib, name)
            f.argtypes = step_args
            f.restype = _i32
        lib.orc_rank_step.argtypes = [_i32, _i64, _i64, _i64] + step_args[3:]
        lib.orc_rank_step.restype = _i32
        lib.orc_mean_grad.argtypes = [_i32, _i64, _i64, _i64, _vp, _vp, C.POINTER(_dbl)]
        lib.orc_mean_grad.restype = _i32
        lib.orc_step_mean.argtypes = [_i32, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _vp, _vp, _i64, _dbl, _dbl, _dbl, _dbl, _dbl, _vp,
                                      C.POINTER(_dbl), _dbl]
        lib.orc_step_mean.restype = _i32
        lib.orc_clip_factor.argtypes = [_dbl, _dbl]
        lib.orc_clip_factor.restype = _dbl
        lib.orc_sgd_step.argtypes = [_i32, _i32, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp,
                                     _vp, _i64, _dbl, _dbl, _dbl, _dbl, _i32, _vp]
        lib.orc_sgd_step.restype = _i32
        lib.orc_memory_bytes.argtypes = [_i64, _i64, _i64, _i32, _i64, _i64, _i64, _i32,
                                         C.POINTER(_i64)]
        lib.orc_memory_bytes.restype = _i32
        lib.orc_min_stage.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64, _i64]
        lib.orc_min_stage.restype = _i32

    @property
    def mutant(self):
        return self.lib.orc_mutant()

    # -- shards ---------------------------------------------------------------
    def split_bounds(self, n, N, r):
        a, b = _i64(), _i64()
        self.lib.orc_split_bounds(n, N, r, C.byref(a), C.byref(b))
        return a.value, b.value

    def owner(self, n, N, i):
        return self.lib.orc_owner(n, N, i)

    # -- bf16 -----------------------------------------------------------------
    def bf16_round(self, x):
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, dtype=np.uint16)
        self.lib.orc_bf16_round(_ptr(x), _ptr(out), x.size)
        return out

    def fp16_round(self, x):
        """IEEE binary16 bit patterns of float32 values, rounded to nearest even."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, dtype=np.uint16)
        self.lib.orc_fp16_round(_ptr(x), _ptr(out), x.size)
        return out

    def fp16_widen(self, h):
        """float32 values of fp16 bit patterns (exact)."""
        h = np.ascontiguousarray(h, dtype=np.uint16)
        out = np.empty(h.shape, dtype=np.float32)
        self.lib.orc_fp16_widen(_ptr(h), _ptr(out), h.size)
        return out

    # -- states ---------------------------------------------------------------
    def init_states(self, mode, param):
        param = np.ascontiguousarray(param, dtype=_PARAM_DT[mode])
        n = param.size
        sdt = _STATE_DT[mode]
        m = np.empty(n, sdt)
        v = np.empty(n, sdt)
        master = np.empty(n, np.float32) if mode in MIXED_MODES else None
        self.lib.orc_init_states(mode, n, _ptr(param), _ptr(master), _ptr(m), _ptr(v))
        return master, m, v

    # -- steps ----------------------------------------------------------------
    def _prep(self, mode, param, grads, master, m, v):
        param = np.ascontiguousarray(param, dtype=_PARAM_DT[mode])
        grads = [np.ascontiguousarray(g, dtype=_PARAM_DT[mode]) for g in grads]
        sdt = _STATE_DT[mode]
        m = np.ascontiguousarray(m, dtype=sdt)
        v = np.ascontiguousarray(v, dtype=sdt)
        if master is not None:
            master = np.ascontiguousarray(master, dtype=np.float32 if mode in MIXED_MODES else sdt)
        return param, grads, master, m, v

    def _call_full(self, fn, mode, param, grads, master, m, v, t, lr, b1, b2, eps, wd, decay):
        param, grads, master, m, v = self._prep(mode, param, grads, master, m, v)
        n, N = param.size, len(grads)
        for g in grads:
            assert g.size == n
        p_out = np.empty_like(param)
        mst_out = np.empty(n, np.float32) if mode in MIXED_MODES else None
        m_out, v_out = np.empty_like(m), np.empty_like(v)
        dec = None if decay is None else np.ascontiguousarray(decay, dtype=np.uint8)
        rc = fn(mode, n, N, _ptr(param), _ptr_array(grads), _ptr(master), _ptr(m), _ptr(v),
                _ptr(p_out), _ptr(mst_out), _ptr(m_out), _ptr(v_out), int(t), float(lr),
                float(b1), float(b2), float(eps), float(wd), _ptr(dec))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return p_out, mst_out, m_out, v_out

    def zero_step(self, mode, param, grads, master, m, v, t, lr, b1=0.9, b2=0.999,
                  eps=1e-8, wd=0.0, decay=None):
        """The sharded step over all N workers. Returns (param, master, m, v)."""
        return self._call_full(self.lib.orc_zero_step, mode, param, grads, master, m, v,
                               t, lr, b1, b2, eps, wd, decay)

    def full_step(self, mode, param, grads, master, m, v, t, lr, b1=0.9, b2=0.999,
                  eps=1e-8, wd=0.0, decay=None):
        """Shard-free Adam over the whole vector driven by the averaged gradient."""
        return self._call_full(self.lib.orc_full_step, mode, param, grads, master, m, v,
                               t, lr, b1, b2, eps, wd, decay)

    def rank_step(self, mode, N, r, param, chunk_grads, master, m, v, t, lr, b1=0.9,
                  b2=0.999, eps=1e-8, wd=0.0, decay=None):
        """Worker r's share: chunk gradients and shard-local master/m/v.

        Returns (full gathered param, master chunk, m chunk, v chunk)."""
        param, chunk_grads, master, m, v = self._prep(mode, param, chunk_grads, master, m, v)
        n = param.size
        a, b = self.split_bounds(n, N, r)
        c = b - a
        assert len(chunk_grads) == N
        for g in chunk_grads:
            assert g.size == c
        assert master is not None and master.size == c and m.size == c and v.size == c
        p_out = np.empty_like(param)
        mst_out, m_out, v_out = np.empty_like(master), np.empty_like(m), np.empty_like(v)
        dec = None if decay is None else np.ascontiguousarray(decay, dtype=np.uint8)
        rc = self.lib.orc_rank_step(mode, n, N, r, _ptr(param), _ptr_array(chunk_grads),
                                    _ptr(master), _ptr(m), _ptr(v), _ptr(p_out), _ptr(mst_out),
                                    _ptr(m_out), _ptr(v_out), int(t), float(lr), float(b1),
                                    float(b2), float(eps), float(wd), _ptr(dec))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return p_out, mst_out, m_out, v_out

    # -- momentum SGD -----------------------------------------------------------
    def sgd_step(self, mode, param, grads, master, buf, t, lr, wd=0.0, momentum=0.0,
                 dampening=0.0, nesterov=False, decay=None, form="sharded", N=None, rank=-1):
        """Momentum SGD. form: 'sharded' (all workers), 'full' (shard-free) or 'rank'
        (worker `rank`'s share: chunk gradients, shard-local master and buffer).
        Returns (param, master, buf)."""
        f = {"sharded": 0, "full": 1, "rank": 2}[form]
        param = np.ascontiguousarray(param, dtype=_PARAM_DT[mode])
        grads = [np.ascontiguousarray(g, dtype=_PARAM_DT[mode]) for g in grads]
        sdt = _STATE_DT[mode]
        buf = np.ascontiguousarray(buf, dtype=sdt)
        n = param.size
        N = len(grads) if N is None else N
        if master is not None:
            master = np.ascontiguousarray(master, dtype=np.float32 if mode in MIXED_MODES else sdt)
        p_out = np.empty_like(param)
        if f == 2:
            mst_out = np.empty_like(master)
        else:
            mst_out = np.empty(n, np.float32) if mode in MIXED_MODES else None
        b_out = np.empty_like(buf)
        dec = None if decay is None else np.ascontiguousarray(decay, dtype=np.uint8)
        rc = self.lib.orc_sgd_step(f, mode, n, N, rank, _ptr(param), _ptr_array(grads),
                                   _ptr(master), _ptr(buf), _ptr(p_out), _ptr(mst_out),
                                   _ptr(b_out), int(t), float(lr), float(wd), float(momentum),
                                   float(dampening), int(bool(nesterov)), _ptr(dec))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return p_out, mst_out, b_out

    # -- materialised mean gradient and clipping --------------------------------
    def mean_grad(self, mode, n, N, grads, rank=-1):
        """The reduce-scatter mean, materialised, and the squared norm.

        Full mode (rank < 0): grads are N full-length arrays; returns (mean of
        length n, sum over shards of the shard squared norms). Rank mode: grads are
        worker `rank`'s N chunks; returns (its c_r means, its shard's squared norm)."""
        grads = [np.ascontiguousarray(g, dtype=_PARAM_DT[mode]) for g in grads]
        assert len(grads) == N
        if rank < 0:
            length = n
        else:
            a, b = self.split_bounds(n, N, rank)
            length = b - a
        for g in grads:
            assert g.size == length
        out = np.empty(length, _STATE_DT[mode])
        ss = _dbl()
        rc = self.lib.orc_mean_grad(mode, n, N, rank, _ptr_array(grads), _ptr(out), C.byref(ss))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return out, ss.value

    def step_mean(self, mode, N, param, mean, master, m, v, t, lr, b1=0.9, b2=0.999, eps=1e-8,
                  wd=0.0, decay=None, clip_sumsq=None, max_norm=0.0, rank=-1):
        """Adam from a materialised mean gradient, optionally clipped by the global
        squared norm clip_sumsq. Returns (param, master, m, v); in rank mode master,
        m, v are the shard's."""
        param = np.ascontiguousarray(param, dtype=_PARAM_DT[mode])
        sdt = _STATE_DT[mode]
        mean = np.ascontiguousarray(mean, dtype=sdt)
        m = np.ascontiguousarray(m, dtype=sdt)
        v = np.ascontiguousarray(v, dtype=sdt)
        n = param.size
        if master is not None:
            master = np.ascontiguousarray(master, dtype=np.float32 if mode in MIXED_MODES else sdt)
        p_out = np.empty_like(param)
        if rank >= 0:
            mst_out = np.empty_like(master)
        else:
            mst_out = np.empty(n, np.float32) if mode in MIXED_MODES else None
        m_out, v_out = np.empty_like(m), np.empty_like(v)
        dec = None if decay is None else np.ascontiguousarray(decay, dtype=np.uint8)
        cs = None if clip_sumsq is None else C.byref(_dbl(float(clip_sumsq)))
        rc = self.lib.orc_step_mean(mode, n, N, rank, _ptr(param), _ptr(mean), _ptr(master),
                                    _ptr(m), _ptr(v), _ptr(p_out), _ptr(mst_out), _ptr(m_out),
                                    _ptr(v_out), int(t), float(lr), float(b1), float(b2),
                                    float(eps), float(wd), _ptr(dec), cs, float(max_norm))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return p_out, mst_out, m_out, v_out

    def clip_factor(self, sumsq, max_norm):
        return self.lib.orc_clip_factor(float(sumsq), float(max_norm))

    # -- memory ---------------------------------------------------------------
    def min_stage(self, n, N, P, G, K, activation_bytes, available_bytes):
        """The smallest ZeRO stage whose memory need fits, or -1."""
        return self.lib.orc_min_stage(n, N, P, G, K, activation_bytes, available_bytes)

    def memory_bytes(self, n, N, r, stage, P, G, K, convention=0):
        out = (_i64 * 3)()
        rc = self.lib.orc_memory_bytes(n, N, r, stage, P, G, K, convention, out)
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return {"params": out[0], "grads": out[1], "optimizer": out[2],
                "total": out[0] + out[1] + out[2]}
