"""ZeroOptimizer's configuration checks, which run before any device work
('Data parallelism and ZeRO stages 1 to 3', openlearn L11.3, section 'What the
tests check': stage 0 or 4, or no parameters, is rejected early)."""
import pytest

from zero_sharded_optimizer_amd.optimizer import ZeroOptimizer, init_states


@pytest.mark.parametrize("stage", [0, 4, -1])
def test_zero_rejects_bad_stage(stage):
    with pytest.raises(ValueError, match="stage must be 1, 2 or 3"):
        ZeroOptimizer([object()], 2, stage)


def test_zero_rejects_no_parameters():
    with pytest.raises(ValueError, match="no parameters"):
        ZeroOptimizer([], 2, 1)
    with pytest.raises(ValueError, match="no parameters"):
        ZeroOptimizer(iter(()), 2, 3)


@pytest.mark.parametrize("kw,msg", [
    (dict(n_workers=0), "n_workers"),
    (dict(n_workers=10**6), "n_workers"),
    (dict(precision="fp8"), "precision"),
    (dict(optimizer="lamb"), "optimizer"),
    (dict(decay=[True, False]), "one flag per parameter"),
])
def test_zero_rejects_bad_configuration(kw, msg):
    args = dict(params=[object()], n_workers=2, stage=1)
    args.update(kw)
    with pytest.raises(ValueError, match=msg):
        ZeroOptimizer(**args)


def test_parameters_must_be_device_tensors_of_the_mode():
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError, match="expected a GPU tensor of torch.float32"):
        ZeroOptimizer([torch.zeros(3)], 2, 1, precision="fp32")


def test_mixed_init_states_needs_the_parameters():
    with pytest.raises(ValueError, match="pass param"):
        init_states(10, 2, device="cpu", precision="bf16")


def test_zero_rejects_a_repeated_parameter():
    """A tensor listed twice would get two slices of the gathered buffer and be
    stepped twice per step."""
    torch = pytest.importorskip("torch")
    t = torch.zeros(4)
    with pytest.raises(ValueError, match="more than once"):
        ZeroOptimizer([t, torch.zeros(2), t], 2, 1)


def test_zero_rejects_parameters_that_share_memory():
    """Two views of one storage would each become a slice of their own, so the
    tie between them would silently break."""
    torch = pytest.importorskip("torch")
    base = torch.zeros(16)
    with pytest.raises(ValueError, match="share memory"):
        ZeroOptimizer([base[:10], torch.zeros(3), base[8:]], 2, 1)
