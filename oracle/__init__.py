"""CPU fp64 oracle of the Video Swin window-attention block.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke entry point and the
benchmark's CPU-baseline leg, never by the product path.
"""
from .vswin import *  # noqa: F401,F403
from . import vswin  # noqa: F401
