"""CPU oracle for the ConvRot-quantized linear.  Test infrastructure only:
imported by the tests, the smoke check and the benchmark's CPU-baseline leg,
never by the GPU library."""
from .convrot_oracle import *  # noqa: F401,F403
from . import convrot_oracle  # noqa: F401
