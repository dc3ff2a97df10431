"""Seeded synthetic input generator (shared by the oracle tests and the GPU path)."""
from .synth import *  # noqa: F401,F403
from .synth import build, lib  # noqa: F401
