"""Planted mistakes in the oracle must be caught by at least one pin.

Each mutant is a build of oracle/oracle.c with ORACLE_MUTANT=k, which swaps
in one plausible mistake (off-by-one slot, ignored stride, reversed length
rule, unclamped log2, wrong GQA map, transposed key packing, unnormalised
output, merge without the partition sums, partition dropping a token, value
rows read token-major; for the decode metadata: inclusive prefix sum, delta
dropped, column not scaled to a token position, SWA map applied to the page
instead of the slot, pool row index ignored; for the speculative page
table: draft row used as the request row, draft column not shifted; fp8
exponent bias 8, k_scale applied to values, ALiBi bias sign flipped).
Mistakes are planted in the oracle only, on the CPU.
"""
import pytest

import oracle
import pins

N_MUTANTS = oracle.get().lib.orc_num_mutants()


@pytest.mark.parametrize("mutant", range(1, N_MUTANTS + 1))
def test_mutant_is_caught(mutant):
    o = oracle.Oracle(mutant=mutant)
    assert o.mutant == mutant
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(o)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {mutant} passed every pin"
