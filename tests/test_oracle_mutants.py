"""Each planted mistake in the oracle must be caught by at least one pin.

The mistakes follow the pitfall list of 'Data parallelism and ZeRO stages 1 to 3'
(openlearn L11.3, section '5. Pitfalls': summing instead of averaging, a rank
beginning at another rank's chunk, no all-gather after the update, stage 2 keeping the
full gradients, dropped hyperparameters) plus plausible slips in the Adam formula
itself (exchanged betas, a dropped bias correction, eps inside the square root,
coupled instead of decoupled decay, a wrong sign, an off-by-one step count, an
inverted decay mask, truncating instead of rounding to bf16 or fp16, an unclamped or
wrongly normed clipping factor, a NaN norm clamped away). The mistakes are
planted in the oracle on the CPU only.
"""
import pytest

from oracle import Oracle
from oracle import build_oracle
from oracle_pins import ALL_PINS

MUTANTS = {
    1: "sum instead of mean",
    2: "wrong chunk start",
    3: "no all-gather",
    4: "betas exchanged",
    5: "v bias correction dropped",
    6: "eps inside sqrt",
    7: "coupled weight decay",
    8: "wrong sign",
    10: "default lr instead of caller's",
    11: "bf16 truncation",
    12: "decay mask inverted",
    13: "stage 2 counts full grads",
    14: "off-by-one step in bias correction",
    15: "clipping factor not clamped at 1",
    16: "1-norm instead of squared norm",
    17: "SGD momentum buffer starting at zero",
    18: "SGD with decoupled instead of coupled decay",
    19: "fp16 truncation",
    20: "NaN clipping factor clamped to 1",
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=[MUTANTS[k] for k in sorted(MUTANTS)])
def test_planted_mistake_is_caught(tmp_path, mutant):
    lib = build_oracle.build(mutant, outdir=str(tmp_path))
    O = Oracle(path=lib)
    assert O.mutant == mutant
    caught = []
    for pin in ALL_PINS:
        try:
            pin(O)
        except AssertionError:
            caught.append(pin.__name__)
        except (ValueError, ZeroDivisionError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {mutant} ({MUTANTS[mutant]})"
