"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

Holds no conv-backward arithmetic (see ``gen`` for the generator's definition and ``workloads`` for
the five workloads). Both the GPU library's callers and the CPU oracle's callers draw from here.
"""
from . import gen, workloads  # noqa: F401
from .workloads import HEADLINE, WORKLOADS, Workload, custom  # noqa: F401
