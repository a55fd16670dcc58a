"""Plant plausible mistakes in a copy of the KV-append oracle (oracle/kv_cache.py)
and require that at least one pin of test_oracle_kv_cache.py catches each.

The oracle file is never modified: each mutant is a text substitution applied
to its source, executed as a fresh module and swapped in for the pins.
"""
import types
from pathlib import Path

import pytest

import test_oracle_kv_cache as pins
from oracle import kv_cache

SRC = Path(kv_cache.__file__).read_text()

# (name, exact text in kv_cache.py, replacement)
MUTANTS = [
    ("pop_from_front", "return [self.free.pop() for _ in range(count)]",
     "return [self.free.pop(0) for _ in range(count)]"),
    ("floor_block_count", "return -(-int(num_tokens) // int(block_size))", "return int(num_tokens) // int(block_size)"),
    ("slot_off_by_one", "pool[pb, 0, :, t % bs, :] = k_new[row + i]", "pool[pb, 0, :, (t + 1) % bs, :] = k_new[row + i]"),
    ("v_written_to_k", "pool[pb, 1, :, t % bs, :] = v_new[row + i]", "pool[pb, 0, :, t % bs, :] = v_new[row + i]"),
    ("rows_not_advanced", "        row += new[r]\n    return", "    return"),
    ("append_from_zero", "t = ctx[r] + i", "t = i"),
    ("release_prepends", "self.free.extend(int(b) for b in blocks)", "self.free[:0] = [int(b) for b in blocks]"),
    ("not_all_or_nothing", "if total > len(alloc.free):", "if False:"),
    ("requests_in_reverse", "for r in range(num_seqs):\n        block_table[r, have[r]:want[r]]",
     "for r in reversed(range(num_seqs)):\n        block_table[r, have[r]:want[r]]"),
    ("table_check_loose", "if want[r] > max_blocks:", "if want[r] > max_blocks + 1:"),
]

PINS = ([pins.test_allocator_worked_example, pins.test_batch_allocation_equals_per_request_allocation,
         pins.test_partial_block_filled_before_a_new_one]
        + [lambda s=s: pins.test_append_extends_every_logical_sequence(s) for s in range(6)]
        + [lambda c=c: pins.test_failed_append_changes_nothing(c) for c in ("exhausted", "table_full")])


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_kv_mutant_is_caught(name, old, new):
    assert SRC.count(old) == 1, "mutation anchor for %s not unique/present" % name
    mod = types.ModuleType("kv_cache_mutant")
    exec(compile(SRC.replace(old, new), "kv_cache_mutant.py", "exec"), mod.__dict__)
    saved = pins.kc
    pins.kc = mod
    caught = 0
    try:
        for pin in PINS:
            try:
                pin()
            except Exception:   # a pin fired (assertion, or the mutant broke a shape)
                caught += 1
    finally:
        pins.kc = saved
    assert caught, "mutant %s survived every pin" % name


def test_unmutated_oracle_passes_every_pin():
    for pin in PINS:
        pin()
