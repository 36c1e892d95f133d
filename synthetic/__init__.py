"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This package holds random-number generation, storage-format casts of the
generated values and the workload shapes only. It computes no step of the
method: anything derived from the predictor, the projection or the scores
(for example a planting direction) is computed by the caller and passed in.
"""
from .gen import *  # noqa: F401,F403
from .configs import CONFIGS, Config  # noqa: F401
