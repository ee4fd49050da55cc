"""Seeded synthetic inputs shared by the GPU tests, the bench and the oracle.

Holds random draws and storage layout only, none of the path's arithmetic.
"""
from .synth import *  # noqa: F401,F403
