"""CPU oracle for the fused Clebsch-Gordan tensor-product (CGTP) convolution.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
definition that the HIP path is checked against.  Only the test-suite, the
smoke check of ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py``
may import, call, link or execute anything in here.  The product path
(``clebsch_gordan_tensor_cgtp_amd``) never imports it and shares no code,
tables or constant generators with it.

What it computes follows "An Efficient Sparse Kernel Generator for
O(3)-Equivariant Deep Networks" (sciencestack.ai page): the Abstract (a
block-sparse CG tensor contracted with two dense vectors, then a structured
weight) and Figures 1 and 4 (the batched use case A and the graph-convolution
use case B).  Conventions the pages leave open (real basis, normalisation,
sign, layouts, path/slot rule) are fixed readings, each stated in the module
that implements it.

Modules
-------
irreps   irreps grammar, path enumeration and output-slot rule
cg       exact Racah CG -> real basis -> Frobenius 1 -> sign rule -> nonzeros
sh       real spherical harmonics (component normalisation)
wigner   real Wigner D by least squares (for equivariance checks)
ref      numpy definitions: batched TP (uvu, uvw) and its backward, conv forward,
         backward and double backward (uvu and uvw), the uvw conv forward and backward,
         the radial-projection conv forward and backward (W = rho Theta; uvu, and uvw
         with each edge's own W_p blocks)
loops    ctypes front-end to ``cpu_loops.c`` (explicit fp64 loops, OpenMP), and
         the double backward, the uvw conv and the radial conv on sampled rows
         composed from those loops

Parity status: every function here is pinned by the ``-m "not gpu"`` tests
(closed forms, orthogonality, a library CG/SH, brute force, equivariance,
the trilinear identity and finite differences; the double backward (uvu and
uvw) against torch autograd applied twice to a dense einsum, finite
differences of the first-order oracle, and its four Euler identities; the uvw and radial
backwards against torch autograd through a dense einsum, one-hot and adjoint
identities).  No function is "parity unpinned".
"""
