"""Pin strength: every planted mistake in the oracle must fail at least one pin.

Each mutant is a build of oracle/lora_oracle.c with ORC_MUTANT=k (CPU only):
 1 rsLoRA divides by r instead of sqrt(r)      7 negative real slots not mapped to active
 2 alpha 0 gives scale 1, not adapter_scale    8 x row stride ignored
 3 shrink drops the last input column          9 scale table tail filled with 1, not 0
 4 B read transposed                           10 MoE pair index e*max_loras + a
 5 delta subtracted                            11 segment end treated as inclusive
 6 padding rows take the active slot           12 base drops the first input column
13 grouped expert range end treated as inclusive
14 grouped row slot read relative to its expert's first row
15 a stack applies its first adapter only
16 the embedding gather reads B transposed
17 the embedding pair copied without its transpose
18 a listed row's x read at its list position    19 a listed row's slot read at its list position
20 a listed segmented row's x at its position    21 a listed gather row's token at its position
22 a listed grouped row's expert at its position 23 a listed stack row's level slot at its position
24 a listed embedding row's slot at its position
"""
import shutil

import pytest

import oracle
import oracle_pins
from oracle import build as obuild

MUTANTS = list(range(1, 25))


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    return tmp_path_factory.mktemp("mutants")


@pytest.mark.parametrize("k", MUTANTS)
def test_mutant_is_caught(mutant_dir, k):
    lib = obuild.build(mutant_dir / f"liblora_oracle_m{k}.so", mutant=k)
    o = oracle.Oracle(lib)
    assert o.mutant == k
    caught = []
    for p in oracle_pins.PINS:
        try:
            p(o)
        except AssertionError:
            caught.append(p.__name__)
    assert caught, f"mutant {k} passed every pin"
