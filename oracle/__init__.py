"""Oracle for the bounded-decay KDA (delta-rule) chunked forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import anything from this package.  It
shares no code with the GPU library and never imports it.

* ``native.recurrent``     -- the definition: plain C float64 token recurrence (OpenMP)
* ``reference.*``          -- NumPy float64 twins and the self-check forms
                              (brute force, quadratic form, chunked WY/UT form)
* ``overflow.*``           -- CPU prediction of bf16 overflow of Gamma-scaled
                              operands (the ablation with the unbounded gate)

Every function is pinned by ``tests/test_oracle_pins.py`` against values fixed
by the pages and by mathematics (hand-derived golden cases, closed forms,
special cases, brute force); nothing is pinned only against itself.
"""
from . import native, overflow, reference  # noqa: F401
