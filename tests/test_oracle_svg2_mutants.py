"""The semantic-permutation pins are strong enough: each plausible mistake
planted in a copy of oracle/svg2.py fails at least one of them (CPU only).

A mutant is a textual edit of the module's source (a flipped comparison, a
dropped weight, a wrong order); the copy is loaded as a module of its own and
every pin in test_oracle_svg2 is run against it.  The unmutated copy must
pass them all."""
import importlib.util
import inspect
import os

import pytest

import test_oracle_svg2 as P
from oracle import svg2

SRC = inspect.getsource(svg2)

# (name, text in oracle/svg2.py, replacement)
MUTANTS = [
    ("farthest_centroid", "assign = d.argmin(axis=1)",
     "assign = d.argmax(axis=1)"),
    ("no_centroid_update", "cent[c] = members.mean(axis=0)", "pass"),
    ("tie_to_higher_index", "assign = d.argmin(axis=1)",
     "assign = d.shape[1] - 1 - d[:, ::-1].argmin(axis=1)"),
    ("init_from_first_tokens", "x[[c * n // C for c in range(C)]]", "x[list(range(C))]"),
    ("unstable_sort", 'np.argsort(assign, kind="stable")', "np.argsort(-np.asarray(assign))[::-1]"),
    ("shares_without_sizes", "w[live] = counts[live] * np.exp", "w[live] = np.exp"),
    ("shares_without_scale", "z[live] = scale * (", "z[live] = ("),
    ("ascending_shares", "key=lambda j: (-w[j], j)", "key=lambda j: (w[j], j)"),
    ("stop_one_late", "        if cum >= p:\n            break", "        if cum > p + 0.3:\n            break"),
    ("cluster_id_uses_wrong_slot", "_, perm, off, base = key_slots[j // Ck]",
     "_, perm, off, base = key_slots[j % len(key_slots)]"),
    ("missing_slot_base", "parts.append(base + np.asarray", "parts.append(0 + np.asarray"),
    ("no_max_subtraction_in_lse", "lse[rows] = (m + np.log(l))[:, 0]", "lse[rows] = np.log(l)[:, 0]"),
]

PINS = [getattr(P, n) for n in dir(P) if n.startswith("test_")]


def _load(text, name):
    path = os.path.join(os.environ.get("TMPDIR", "/tmp"), f"svg2_mutant_{name}_{os.getpid()}.py")
    with open(path, "w") as f:
        f.write(text)
    spec = importlib.util.spec_from_file_location(f"svg2_mutant_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    os.remove(path)
    return mod


def _run_pins(mod, monkeypatch):
    monkeypatch.setattr(P, "svg2", mod)
    failed = []
    for pin in PINS:
        params = inspect.signature(pin).parameters
        args = [0] if "seed" in params else []
        try:
            pin(*args)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(pin.__name__)
    return failed


def test_unmutated_copy_passes_every_pin(monkeypatch):
    assert _run_pins(_load(SRC, "none"), monkeypatch) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_fails_a_pin(monkeypatch, name, old, new):
    assert SRC.count(old) == 1, name
    failed = _run_pins(_load(SRC.replace(old, new), name), monkeypatch)
    assert failed, f"mutant {name} passes every pin"
