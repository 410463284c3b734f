"""CPU float64 oracle for the edge-conditioned O(3) tensor-product convolution.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (the HIP library and its Python binding) never imports, links or
executes it, and shares no code with it.

What it computes follows the Sobek paper ("Sobek: Streaming Equivariant Tensor
Product Convolutions"), Sec. 2, in the conventional *materialized* schedule the
paper contrasts the streaming one with: per-edge radial weights W = phi A
(Eq. 12-13), per-edge messages (Eq. 6, 7, 11) and a receiver sum.  First and
second derivatives come from torch-CPU float64 autograd of that definition,
chunked over edges (valid because every loss used is a sum over edges).

Modules:
  irreps  -- irreps bookkeeping and Clebsch-Gordan selection rules (Eq. 3-5, 9-10)
  sh      -- real spherical harmonics l <= 3 (the convention fixed for this library)
  wigner  -- real-basis Wigner-D matrices by least squares on the harmonics
  cg      -- real-basis coupling tensors as the null space of the equivariance constraint
  radial  -- Gaussian and Bessel-with-polynomial-envelope radial bases
  conv    -- forward / backward / double backward, materialized
  csr     -- receiver and sender CSR views (stable)
  radius  -- radius graph of a point set by brute force (graph preparation)
  layout  -- mul_ir <-> ir_mul feature layouts at the boundary

Parity status: every function above is pinned by tests against something other
than itself (closed forms, scipy/sympy routines, invariants, finite differences,
brute force); see the test files named in each module docstring.
"""
