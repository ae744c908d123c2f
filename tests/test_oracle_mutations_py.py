"""Plant plausible mistakes in the functions the oracle writes in Python
(``oracle/__init__.py``: the sparse branch's key blocks, Gini coefficient,
block selection, pooled map and composition; the merge of two attentions)
and check that the pins catch each one.

Each mutation is a textual edit of a copy of the module, loaded under another
name over the same compiled library; every pin of ``test_oracle_pins`` runs
against it and at least one must fail.
"""
import importlib.util
import os

import pytest

import oracle
from tests import test_oracle_pins as pins
from tests.test_oracle_mutations import _pin_calls

SRC = os.path.join(os.path.dirname(oracle.__file__), "__init__.py")

MUTATIONS = {
    "gini halves the denominator": ("/ (2.0 * p.size * p.sum())", "/ (p.size * p.sum())"),
    "selection takes the smallest masses first": ("key=lambda j: (-float(mass[j]), j)",
                                                  "key=lambda j: (float(mass[j]), j)"),
    "selection ties go to the higher index": ("key=lambda j: (-float(mass[j]), j)",
                                              "key=lambda j: (-float(mass[j]), -j)"),
    "selection returned in mass order": ("    return sorted(chosen)\n", "    return chosen\n"),
    "selection stops one block early": ("        chosen.append(j)\n        total += float(mass[j])\n"
                                        "        if total >= tau:\n            break",
                                        "        total += float(mass[j])\n"
                                        "        if total >= tau:\n            break\n"
                                        "        chosen.append(j)"),
    "own keys cut into context-size blocks": (
        "for s in range(0, n_own, b_intra)]", "for s in range(0, n_own, b_inter)]"),
    "pooled map drops the scale": ('s = np.einsum("hd,jhd->hj", qbar, kbar) * scale',
                                   's = np.einsum("hd,jhd->hj", qbar, kbar)'),
    "pooled map uses block sums, not means": ("kbar = np.stack([k[a:b].mean(axis=0)",
                                              "kbar = np.stack([k[a:b].sum(axis=0)"),
    "every head uses head 0's threshold": ("chosen = select_blocks(pmap[h], float(tau[h]))",
                                           "chosen = select_blocks(pmap[h], float(tau[0]))"),
    "every head uses head 0's map": ("chosen = select_blocks(pmap[h], float(tau[h]))",
                                     "chosen = select_blocks(pmap[0], float(tau[h]))"),
    "merge weights the parts the wrong way round": (
        "out = (wa / tot).T[:, :, None] * oa + (wb / tot).T[:, :, None] * ob",
        "out = (wb / tot).T[:, :, None] * oa + (wa / tot).T[:, :, None] * ob"),
    "merge forgets to normalise the weights": (
        "out = (wa / tot).T[:, :, None] * oa + (wb / tot).T[:, :, None] * ob",
        "out = wa.T[:, :, None] * oa + wb.T[:, :, None] * ob"),
    "merge lse drops the max": ("    return out, m + np.log(tot)", "    return out, np.log(tot)"),
}


def _failing_pins(text, tmp_path):
    path = tmp_path / "oracle_mut.py"
    path.write_text(text)
    spec = importlib.util.spec_from_file_location("oracle_mut", str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod._lib = oracle._load()          # the same compiled arithmetic
    caught = []
    for name, fn, kwargs in _pin_calls():
        try:
            fn(oracle_lib=mod, **kwargs)
        except Exception:              # an assertion, or a shape/index error
            caught.append(name)
    return caught


def test_unmutated_copy_passes_every_pin(tmp_path):
    """The copy-and-load route itself breaks nothing."""
    assert _failing_pins(open(SRC).read(), tmp_path) == []


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_pins_catch_planted_mistake_in_python_part(mutation, tmp_path):
    old, new = MUTATIONS[mutation]
    text = open(SRC).read()
    assert text.count(old) == 1, "mutation anchor not found once: %r" % old
    caught = _failing_pins(text.replace(old, new), tmp_path)
    assert caught, "no pin failed for the planted mistake: %s" % mutation
