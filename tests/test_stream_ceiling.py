"""The streaming-ceiling kernels that bench.py measures the memory system with
(libzceil.so). They are measurement tools, not part of the optimizer; these
tests check that they do the work whose bytes bench.py counts: every input
byte read, the XOR of the inputs written to every output, nothing written past
the end."""
import ctypes
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "zero_sharded_optimizer_amd", "libzceil.so")


def _lib():
    if not os.path.exists(LIB):
        pytest.skip("libzceil.so not built")
    lib = ctypes.CDLL(LIB)
    P = ctypes.POINTER
    lib.zceil_streams.restype = ctypes.c_int
    lib.zceil_streams.argtypes = [P(ctypes.c_void_p), P(ctypes.c_int32), ctypes.c_int32,
                                  P(ctypes.c_void_p), P(ctypes.c_int32), ctypes.c_int32,
                                  ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p]
    return lib


def _call(lib, ins, win, outs, wout, ngroups, shape=0):
    pin = (ctypes.c_void_p * max(1, len(ins)))(*ins)
    pout = (ctypes.c_void_p * max(1, len(outs)))(*outs)
    a = (ctypes.c_int32 * max(1, len(win)))(*win)
    b = (ctypes.c_int32 * max(1, len(wout)))(*wout)
    return lib.zceil_streams(pin, a, len(ins), pout, b, len(outs), ngroups, shape, None)


def test_exports_and_rejects_bad_arguments_before_any_launch():
    """Argument checks return -1 before any HIP call, so they run without a GPU."""
    lib = _lib()
    fake = [1 << 32, (1 << 32) + (1 << 24)]
    assert _call(lib, [], [], fake[:1], [16], 10) == -1                 # no inputs
    assert _call(lib, fake[:1], [16], [], [], 10) == -1                 # no outputs
    assert _call(lib, fake[:1] * 129, [16] * 129, fake[1:], [16], 10) == -1  # 129 inputs
    assert _call(lib, fake[:1], [12], fake[1:], [16], 10) == -1         # width not 8 or 16
    assert _call(lib, [fake[0] + 8], [16], fake[1:], [16], 10) == -1    # misaligned
    assert _call(lib, [0], [16], fake[1:], [16], 10) == -1              # NULL stream pointer
    assert _call(lib, fake[:1], [16], fake[1:], [16], -1) == -1         # negative size
    assert _call(lib, fake[:1], [16], fake[1:], [16], 10, shape=7) == -1  # no such shape
    assert _call(lib, fake[:1], [16], fake[1:], [16], 0) == 0           # empty: nothing to do


@pytest.mark.gpu
@pytest.mark.parametrize("shape", [0, 1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("nin", [5, 21, 40])
@pytest.mark.parametrize("ngroups", [1, 1023, 1024 * 3 + 517])
def test_xor_of_the_inputs_reaches_every_output(ngroups, nin, shape):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    print(f"[case] zceil_streams ngroups={ngroups} nin={nin} shape={shape}", flush=True)
    lib = _lib()
    rng = np.random.default_rng(ngroups)
    win, wout = ([16, 8, 16, 8, 16] * 8)[:nin], [16, 8, 16]
    tail = 64  # guard bytes after each output
    ins_h = [rng.integers(0, 256, ngroups * w, dtype=np.uint8) for w in win]
    ins = [torch.from_numpy(x).cuda() for x in ins_h]
    outs = [torch.full((ngroups * w + tail,), 0xA5, dtype=torch.uint8, device="cuda")
            for w in wout]
    assert _call(lib, [t.data_ptr() for t in ins], win, [t.data_ptr() for t in outs], wout,
                 ngroups, shape) == 0
    torch.cuda.synchronize()
    acc = np.zeros((ngroups, 16), np.uint8)
    for x, w in zip(ins_h, win):
        acc[:, :w] ^= x.reshape(ngroups, w)
    for t, w in zip(outs, wout):
        got = t.cpu().numpy()
        assert np.array_equal(got[: ngroups * w].reshape(ngroups, w), acc[:, :w])
        assert np.all(got[ngroups * w:] == 0xA5)
