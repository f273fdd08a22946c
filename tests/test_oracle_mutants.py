"""The oracle's pins catch planted mistakes (CPU only).

Each case copies oracle.c with one plausible mistake planted (a dropped scale,
an off-by-one visibility rule, a wrong head map, swapped merge weights, a
wrong sign, a transposed operand ...), builds it with gcc into a temporary
directory, swaps it in, and checks that at least one pin of test_oracle.py
fails.  The committed oracle is never modified.
"""
import ctypes
import inspect
import os
import subprocess

import pytest

import oracle.oracle as orc
import tests.test_oracle as pins

MUTANTS = {
    "dropped_scale": ("s[t] = sigma * dot;", "s[t] = dot;"),
    "visibility_off_by_one": ("return (j - i) <= delta;", "return (j - i) < delta;"),
    "gqa_modulo_map": ("return (h * hkv) / hq;", "return h % hkv;"),
    "lse_missing_max": ("*lse = m + log(l);", "*lse = log(l);"),
    "merge_swapped_weights": ("o[c] = (wa * oa[c] + wb * ob[c]) / tot;",
                              "o[c] = (wb * oa[c] + wa * ob[c]) / tot;"),
    "ds_wrong_sign": ("const double ds = p * (dp - D);",
                      "const double ds = p * (dp + D);"),
    "dk_dropped_scale": ("dk[c] += sigma * ds * (double)qrow[c];",
                         "dk[c] += ds * (double)qrow[c];"),
    "dq_transposed_operand": ("dq[c] += sigma * ds * (double)krow[c];",
                              "dq[c] += sigma * ds * (double)vrow[c];"),
    "dv_uses_ds": ("dv[c] += p * (double)dorow[c];",
                   "dv[c] += ds * (double)dorow[c];"),
    "dilation_not_segment_relative": ("(p - seg0 - s) % r != 0", "(p - s) % r != 0"),
    "head_shift_keys_unshifted": ("for (int64_t t = seg0 + s;", "for (int64_t t = seg0;"),
    "head_shift_by_kv_head": ("const int64_t off = head_shift ? h % r[b] : 0;",
                              "const int64_t off = head_shift ? g % r[b] : 0;"),
    "dilated_causal_strict": ("if (!causal || t <= p)", "if (!causal || t < p)"),
    "dilated_merge_drops_branch": ("merge_row(acc, lacc, ob, lb, d, tmp, &lnew);",
                                   "merge_row(ob, lb, ob, lb, d, tmp, &lnew);"),
    "dilated_bwd_dk_misses_scale": ("dk[c] += sigma * ds * (double)qrow[c];\n                        }\n                    }\n                }\n            }\n        }\n        free(keys);",
                                    "dk[c] += ds * (double)qrow[c];\n                        }\n                    }\n                }\n            }\n        }\n        free(keys);"),
    "dilated_bwd_uses_local_lse": ("const double P = exp(sigma * dot - lse[row]);\n                    const double ds = P * (dp - D[row]);\n                    for (int64_t c = 0; c < d; ++c)\n                        dq[c] += sigma * ds * (double)krow[c];\n                }",
                                   "const double P = exp(sigma * dot - lse[row] + 0.1);\n                    const double ds = P * (dp - D[row]);\n                    for (int64_t c = 0; c < d; ++c)\n                        dq[c] += sigma * ds * (double)krow[c];\n                }"),
}


def _pin_calls():
    """Every (name, zero-arg callable) of the pin module, parameters expanded."""
    calls = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if not params:
            calls.append((name, fn))
            continue
        argnames, values = params[0].args
        argnames = [a.strip() for a in argnames.split(",")]
        for vals in values:
            vals = vals if len(argnames) > 1 else (vals,)
            kw = dict(zip(argnames, vals))
            calls.append((f"{name}{vals}", lambda fn=fn, kw=kw: fn(**kw)))
    return calls


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistake_is_caught(mutant, tmp_path, monkeypatch):
    old, new = MUTANTS[mutant]
    src = open(orc.SRC).read()
    assert src.count(old) >= 1, f"mutation site for {mutant} not found"
    mutated = src.replace(old, new)
    csrc = tmp_path / "oracle_mut.c"
    csrc.write_text(mutated)
    so = tmp_path / "liboracle_mut.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                           "-o", str(so), str(csrc), "-lm"])
    monkeypatch.setattr(orc, "LIB", str(so))
    monkeypatch.setattr(orc, "_lib", None)
    caught = []
    for name, call in _pin_calls():
        try:
            call()
        except AssertionError:
            caught.append(name)
            break
    monkeypatch.setattr(orc, "_lib", None)
    assert caught, f"no pin caught the planted mistake {mutant}"
    os.remove(so)
