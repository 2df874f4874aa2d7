"""Plant plausible mistakes in a copy of the oracle and check a pin catches each.

CPU only. Each mutant is the oracle's own source with one edit (a wrong mask
comparison, a dropped scale, the modulo head mapping, log2 for ln, a missing
normalisation, an unweighted combine, a reversed page table walk). The edited
copy is loaded in place of the real functions for the duration of one pin,
which must then fail.
"""

import os
import types

import pytest

import oracle
import oracle.attention as oatt
import oracle.paged as opaged
from tests import test_oracle_pins as pins

HERE = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _mutant(relpath, old, new):
    path = os.path.join(HERE, "oracle", relpath)
    with open(path) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor not unique in {relpath}: {old!r}"
    mod = types.ModuleType("oracle._mutant")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), path, "exec"), mod.__dict__)
    return mod


def _install(monkeypatch, mod, names, targets):
    for name in names:
        for tgt in targets:
            monkeypatch.setattr(tgt, name, getattr(mod, name))


ATT = ("attention_rows", "prefill_attention", "decode_attention", "combine_partials")

MUTANTS = [
    ("mask includes the diagonal's neighbour",
     "attention.py", "hidden = np.arange(n)[None, :] > pos[r0:r1, None]",
     "hidden = np.arange(n)[None, :] >= pos[r0:r1, None]",
     lambda: pins.test_closed_form_zero_query_pins_mask_offset(3)),
    ("scale dropped",
     "attention.py", "S = scale * (q[r0:r1] @ k.T)", "S = (q[r0:r1] @ k.T)",
     pins.test_closed_form_single_key),
    ("modulo head mapping",
     "attention.py", "g = hq // G\n        o, l = attention_rows(q[b, hq][idx]",
     "g = hq % Hkv\n        o, l = attention_rows(q[b, hq][idx]",
     pins.test_gqa_equals_mha_on_repeat_interleaved_kv),
    ("log2 instead of natural log",
     "attention.py", "m + np.log(np.where(seen, lsum, 1.0))",
     "m + np.log2(np.where(seen, lsum, 1.0))",
     lambda: pins.test_matches_torch_sdpa_fp64_with_explicit_mask(9, 9, True)),
    ("probabilities not normalised",
     "attention.py", "out[r0:r1] = P @ v", "out[r0:r1] = E @ v",
     lambda: pins.test_probability_rows(True, 5)),
    ("transposed value operand",
     "attention.py", "out[r0:r1] = P @ v", "out[r0:r1] = (P @ v[:, ::-1])",
     lambda: pins.test_matches_torch_sdpa_fp64_with_explicit_mask(3, 11, True)),
    ("combine without normalised weights",
     "attention.py", "coef[:, seen] = w[:, seen] / tot[None, seen]", "coef[:, seen] = w[:, seen]",
     pins.test_split_combine_equals_unsplit),
]


@pytest.mark.parametrize("label,relpath,old,new,pin", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pin_catches_attention_mutant(monkeypatch, label, relpath, old, new, pin):
    mod = _mutant(relpath, old, new)
    _install(monkeypatch, mod, ATT, (oracle, oatt))
    with pytest.raises(AssertionError):
        pin()


def test_pin_catches_reversed_table_walk(monkeypatch):
    mod = _mutant("paged.py", "blk = _table_entry(table_row, i)",
                  "blk = _table_entry(table_row, nblk - 1 - i)")
    _install(monkeypatch, mod, ("gather_paged",), (oracle, opaged))
    with pytest.raises(AssertionError):
        pins.test_paged_gather_is_bit_exact()


def test_pin_catches_wrong_append_slot(monkeypatch):
    mod = _mutant("paged.py", "out[blk, t % block_size] = new_rows[b, r]",
                  "out[blk, (t + 1) % block_size] = new_rows[b, r]")
    _install(monkeypatch, mod, ("kv_append_ref",), (oracle, opaged))
    with pytest.raises(AssertionError):
        pins.test_kv_append_round_trip_and_untouched_bytes()


import oracle.fp8 as ofp8  # noqa: E402
from tests import test_oracle_fp8 as fp8pins  # noqa: E402

FP8 = ("e4m3_decode", "e4m3_encode", "quantize", "dequantize")

FP8_MUTANTS = [
    ("exponent bias 8 (the FNUZ variant)",
     "return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)",
     "return sign * (1.0 + m / 8.0) * 2.0 ** (e - 8)",
     fp8pins.test_decode_matches_torch_for_every_code),
    ("ties away from zero",
     "pick = np.where(tie & (_POS_CODES[best] % 2 == 1), nxt, best)",
     "pick = np.where(tie, nxt, best)",
     fp8pins.test_closed_forms),
    ("no saturation beyond 448",
     "mag = np.minimum(np.abs(np.where(nan, 0.0, v)), E4M3_MAX)",
     "mag = np.abs(np.where(nan, 0.0, v))",
     fp8pins.test_closed_forms),
    ("scale multiplied instead of divided",
     "y = (xf / s).astype(np.float32)",
     "y = (xf * s).astype(np.float32)",
     fp8pins.test_quantisation_error_bound),
]


@pytest.mark.parametrize("label,old,new,pin", FP8_MUTANTS, ids=[m[0] for m in FP8_MUTANTS])
def test_pin_catches_fp8_mutant(monkeypatch, label, old, new, pin):
    mod = _mutant("fp8.py", old, new)
    _install(monkeypatch, mod, FP8, (oracle, ofp8))
    with pytest.raises((AssertionError, ValueError)):
        pin()
