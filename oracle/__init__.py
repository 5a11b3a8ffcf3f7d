"""Plain CPU oracle of the sparse MoE block forward.

Test infrastructure only: the test-suite, the package smoke check and the
benchmark's CPU-baseline leg may import it; the product path never does.
It shares no code with the HIP path (see ``oracle.oracle`` for the method).
"""
from .oracle import forward, route  # noqa: F401
