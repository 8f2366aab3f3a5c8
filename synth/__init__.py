"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark."""
from .inputs import *  # noqa: F401,F403
