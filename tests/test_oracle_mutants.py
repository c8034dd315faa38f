"""Planted mistakes in the oracle (on the CPU only): each mutant below is a
plausible slip in one step of E1-E6 or the fp8 codec -- a dropped term, a
wrong sign or index, a swapped operand -- and must make at least one of the
pins in test_oracle.py fail. A control run first checks that every pin
passes on the unmodified oracle, so a failure can only come from the mutant.

Mutants are made from the oracle's own source text by one substring
replacement and executed in the same module namespace, then bound in place
of the original everywhere the oracle modules and the pins module refer to
it (the pytest monkeypatch fixture restores them)."""
import inspect
import sys
import textwrap

import numpy as np
import pytest

import oracle
import oracle.core
import oracle.fp8
import test_oracle as pins

PIN_TESTS = sorted(n for n in dir(pins) if n.startswith("test_"))


def param_sets(fn):
    """The argument combinations of a pin's parametrize marks."""
    combos = [dict()]
    for m in getattr(fn, "pytestmark", []):
        if m.name != "parametrize":
            continue
        names = [n.strip() for n in m.args[0].split(",")]
        grown = []
        for c in combos:
            for vals in m.args[1]:
                vals = vals if len(names) > 1 else (vals,)
                d = dict(c)
                d.update(zip(names, vals))
                grown.append(d)
        combos = grown
    return combos


def failing_pins():
    """Names of the pins that fail (any exception) for some parameter set."""
    out = []
    for name in PIN_TESTS:
        fn = getattr(pins, name)
        for params in param_sets(fn):
            try:
                fn(**params)
            except Exception:
                out.append(name)
                break
    return out


def mutate(fn, old, new):
    src = textwrap.dedent(inspect.getsource(fn))
    assert src.count(old) == 1, f"{fn.__name__}: {old!r} found {src.count(old)} times"
    ns = dict(fn.__globals__)
    exec(compile(src.replace(old, new), f"<mutant of {fn.__name__}>", "exec"), ns)
    return ns[fn.__name__]


def bind(monkeypatch, orig, replacement):
    """Replace every module-level binding of `orig` in the oracle modules and
    the pins module."""
    n = 0
    for mod in list(sys.modules.values()):
        name = getattr(mod, "__name__", "")
        if not (name == "oracle" or name.startswith("oracle.") or name == pins.__name__):
            continue
        for attr, val in list(vars(mod).items()):
            if val is orig:
                monkeypatch.setattr(mod, attr, replacement)
                n += 1
    assert n > 0


# (function, text in its source, replacement, what the slip is)
MUTANTS = [
    ("pool_keys", ".mean(axis=0)", ".sum(axis=0)", "E1: block sum instead of mean"),
    ("pool_keys", "k[j * B:min((j + 1) * B, L)]", "k[j * B:min((j + 1) * B, L) - 1]",
     "E1: last token of each key block dropped"),
    ("pool_queries", "lo, hi = max(i * B, P), min((i + 1) * B, L)", "lo, hi = i * B, min((i + 1) * B, L)",
     "E1: cached prefix rows counted in the first query block"),
    ("block_scores", "full = c * (qbar[h] @ kbar[g].T)", "full = qbar[h] @ kbar[g].T",
     "E2: softmax scale dropped"),
    ("block_scores", "g = h // G", "g = h % Hkv", "E2: wrong query-head to KV-head mapping"),
    ("select", "R[g, il, :i + 1] = diff.max(axis=0)", "R[g, il, :i + 1] = diff.min(axis=0)",
     "E4: intersection instead of union over the group's heads"),
    ("select", ">= -tau", ">= tau", "E5: sign of the threshold"),
    ("select", "keep[g, il, 0] = True", "pass", "E5: sink block not forced"),
    ("select", "keep[g, il, i] = True", "pass", "E5: diagonal block not forced"),
    ("select", "M = S.max(axis=2)", "M = S[:, :, :1].max(axis=2)", "E3: row maximum over the sink only"),
    ("attend", "zp = c * (Q @ Kp.T) + bias[None, :]", "zp = c * (Q @ Kp.T)",
     "E6: ln|J| multiplicity of the pseudo-tokens dropped"),
    ("attend", "block_scores[h, il, pruned_j][None, :] + bias[None, :]", "block_scores[h, il, pruned_j][None, :]",
     "block-score variant: ln|J| multiplicity dropped"),
    ("attend", "block_scores[h, il, pruned_j]", "block_scores[h, max(il - 1, 0), pruned_j]",
     "block-score variant: the previous query block's scores"),
    ("select", "return select(S, 1, tau, i0)", "return select(S, 2, tau, i0)",
     "per-head variant: lists shared by pairs of heads"),
    ("attend", "future = tok[None, :] > t[:, None]", "future = tok[None, :] >= t[:, None]",
     "E6: causal mask excludes the query's own position"),
    ("attend", "Kp = kbar[g, pruned_j, :]", "Kp = vbar[g, pruned_j, :]", "E6: pooled keys and values swapped"),
    ("attend", "lse[h, lo - P:hi - P] = m + np.log(l)", "lse[h, lo - P:hi - P] = np.log(l)",
     "E6: maximum not added back into lse"),
    ("attend", "Q = q[lo - P:hi - P, h, :]", "Q = q[lo:hi, h, :]", "E6: query rows not offset by the prefix"),
    ("attend", "(w @ Vx + wp @ Vp)", "(w @ Vx)", "E6: correction values dropped from the numerator"),
    ("attend", "l = w.sum(axis=1) + wp.sum(axis=1)", "l = w.sum(axis=1)",
     "E6: correction mass dropped from the denominator"),
    ("attend", "kept_j = [j for j in range(i + 1) if keep[g, il, j]]",
     "kept_j = [j for j in range(i) if keep[g, il, j]]", "E6: exact tokens of the diagonal block dropped"),
    ("pool_update", "j = (start + t) // B", "j = t // B",
     "E1 cache: new tokens placed by their offset in the chunk, not their position"),
    ("pool_update", "C[:counts.shape[0]] = counts", "pass", "E1 cache: earlier chunks' token counts dropped"),
    ("pool_means", "sums[:, :nb] / counts[:nb, None]", "sums[:, :nb] / B", "E1 cache: partial block divided by B"),
]


def test_control_all_pins_pass():
    assert failing_pins() == []


@pytest.mark.parametrize("fname,old,new,what", MUTANTS, ids=[m[3] for m in MUTANTS])
def test_core_mutant_is_caught(monkeypatch, fname, old, new, what):
    orig = getattr(oracle.core, fname)
    bind(monkeypatch, orig, mutate(orig, old, new))
    caught = failing_pins()
    assert caught, f"no pin catches: {what}"


def test_fp8_decode_mutant_is_caught(monkeypatch):
    """Subnormal E4M3 codes decoded with the normal exponent bias."""
    bad = mutate(oracle.fp8._decode_one, "2.0 ** (1 - 7)", "2.0 ** (0 - 7)")
    monkeypatch.setattr(oracle.fp8, "_TABLE", np.array([bad(c) for c in range(256)], dtype=np.float64))
    assert failing_pins()
