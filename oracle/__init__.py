"""Plain fp64 CPU oracle for the edge-conditioned Clebsch-Gordan tensor-product
convolution ("Sobek: streaming equivariant tensor-product convolution", abstract).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call, link
or execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP library (no tables, helpers, headers or generators); the only common module
is the seeded input generator, which holds none of the method's arithmetic.

The oracle follows the *conventional* schedule the abstract describes: it
materialises per-edge weights, messages and adjoints (in bounded edge chunks)
and scatter-adds them.  The streaming library must reach the same numbers.

Modules
-------
cg       complex CG by the Racah formula, real-basis CG tables, irreps, paths
sh       real spherical harmonics (component normalised) and their Jacobian
radial   Bessel radial basis with the p=6 polynomial envelope, and R'(d)
tpconv   forward / backward / double backward, materialising schedule

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
library routines (sympy CG, scipy spherical harmonics, scipy quadrature),
invariants (rotation, inversion, translation, permutation) and finite
differences.  Conventions that nothing on the pages fixes (the sign of odd-sum
paths, the Bessel prefactor) are "parity unpinned": they hold by choice and are
checked only against the library's exported tables.
"""
