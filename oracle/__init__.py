"""fp64 CPU oracle for one EAGLE-2 draft round.

Test infrastructure only: the tests, the smoke check and the bench's CPU
baseline leg may import it; the product path never does.
"""
from .eagle_oracle import *  # noqa: F401,F403
