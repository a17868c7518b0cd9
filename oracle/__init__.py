"""CPU oracle for the LIME inference hot path.

Test infrastructure only: imported by the tests, the smoke check and the
bench's CPU-baseline leg, never by the product path.
"""
from .lime_oracle import *  # noqa: F401,F403
