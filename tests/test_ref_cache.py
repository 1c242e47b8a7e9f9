"""The stored oracle references of tests/golden/refcache (written by tests/golden/make_ref_cache.py, the oracle alone):
every planned call has its entry, and entries recomputed by the oracle here match what is stored bit for bit."""
import importlib.util
import os

import numpy as np
import pytest

import parity

_GEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "make_ref_cache.py")


@pytest.fixture(scope="module")
def gen():
    spec = importlib.util.spec_from_file_location("make_ref_cache", _GEN)
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_every_planned_reference_is_stored(gen):
    missing = [fn.__name__ for fn, a, kw in gen.plan() if parity.load_ref(gen.key_of(fn, a, kw)) is None]
    assert not missing, f"{len(missing)} references not stored: run tests/golden/make_ref_cache.py"


def test_stored_references_recompute(gen, oracle_mod):
    """A few small entries of each kind, recomputed from the oracle, equal the stored ones."""
    picked = {}
    for fn, a, kw in gen.plan():
        L = a[3] if fn is parity.soft_reference else a[4]
        w = a[0]
        if L <= 6 and w.shape[0] * w.shape[1] <= 200 and len(picked.get(fn.__name__, [])) < 2:
            picked.setdefault(fn.__name__, []).append((fn, a, kw))
    assert len(picked) == 4
    for entries in picked.values():
        for fn, a, kw in entries:
            stored = parity.load_ref(gen.key_of(fn, a, kw))
            assert stored is not None
            assert gen._same(fn.uncached(oracle_mod, *a, **kw), stored), fn.__name__


def test_key_covers_every_input(gen):
    """Changing any input array or scalar changes the digest."""
    w = np.zeros((2, 3), np.float32)
    c = np.zeros(16, np.float32)
    base = parity.ref_key("soft_reference", {"w": w, "c": c, "L": 4, "k": 2, "T": 0.1, "sigma": None})
    w2 = w.copy()
    w2[1, 2] = np.float32(1e-30)
    assert parity.ref_key("soft_reference", {"w": w2, "c": c, "L": 4, "k": 2, "T": 0.1, "sigma": None}) != base
    assert parity.ref_key("soft_reference", {"w": w, "c": c, "L": 4, "k": 2, "T": 0.2, "sigma": None}) != base
    assert parity.ref_key("soft_reference", {"w": w, "c": c, "L": 4, "k": 2, "T": 0.1,
                                             "sigma": np.zeros(2, np.int32)}) != base
    assert parity.ref_key("grad_reference", {"w": w, "c": c, "L": 4, "k": 2, "T": 0.1, "sigma": None}) != base
