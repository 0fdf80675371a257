"""Seeded synthetic inputs shared by the tests, the smoke check and the
benchmark.  Holds no arithmetic of the method: only shapes, seeds, value
distributions and random draws."""
from .synthetic import *  # noqa: F401,F403
