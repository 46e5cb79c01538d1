"""MI355X-native tensor-parallel MLP shard: a HIP (gfx950) library behind a C ABI.

The compute lives in ``libmlptp.so`` (built from ``csrc/``); ``binding`` marshals arguments to
it through ctypes. ``workloads`` and ``synth`` describe and draw the seeded synthetic inputs.
"""
from .workloads import ALL, BY_NAME, Workload  # noqa: F401
