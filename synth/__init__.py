"""Seeded synthetic inputs, shared by the oracle's tests and the HIP path's tests and bench.

This package draws random numbers and rounds them to the storage formats
(bf16, OCP E4M3FN). It holds none of the method's arithmetic: no products,
sums, normalisation or permutation of the method appear here.
"""
from .gen import (stream_key, uniform, normal, encode_bf16, encode_e4m3,
                  uniform_bf16, normal_bf16, normal_e4m3)
from . import workloads

__all__ = ["stream_key", "uniform", "normal", "encode_bf16", "encode_e4m3",
           "uniform_bf16", "normal_bf16", "normal_e4m3", "workloads"]
