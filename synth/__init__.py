"""Seeded synthetic inputs shared by the CPU oracle's tests and the HIP path's tests/bench.

Holds workload parameters and random-input construction only; no part of the method.
"""
from .configs import CHUNK2, CHUNK7, LONGLIVE, SWEEP, TINY, WORKLOADS, Sweep, Workload
from .gen import Inputs, make, make_denoise_steps, make_on_device, make_sweep_layer

__all__ = ["CHUNK2", "CHUNK7", "LONGLIVE", "SWEEP", "TINY", "WORKLOADS", "Sweep", "Workload",
           "Inputs", "make", "make_denoise_steps", "make_on_device", "make_sweep_layer"]
