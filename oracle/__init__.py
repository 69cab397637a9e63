"""CPU oracle for the OmniMoE routed atomic-expert layer.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by
the benchmark's CPU-baseline leg, never by the library or its binding.
It shares no code with the GPU path.  See omni_oracle.py for the passages
each function follows and the readings taken where the pages are silent.
"""
from .omni_oracle import *  # noqa: F401,F403
