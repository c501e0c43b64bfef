"""fp64 CPU oracle of the Looped Latent Attention decode path.

TEST INFRASTRUCTURE ONLY: only tests/, __graft_entry__.smoke() and the benchmark's CPU-baseline
leg may import this package.  It shares no code with the HIP library and never imports it.
`oracle.oracle` wraps the plain C implementation (lla_oracle.c); `oracle.brute` is an
independent NumPy brute force for tiny inputs.
"""
from . import brute, oracle  # noqa: F401
