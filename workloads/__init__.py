"""Seeded synthetic workloads shared by the tests, the benchmark and the smoke check.

This package holds no step of the attention method: it only names the
problem shapes and draws random inputs.  Both the HIP path and the CPU oracle
consume what it returns.
"""
from .configs import (CONFIGS, FLASHTPA_BATCHES, FLASHTPA_HEADS, FLASHTPA_RQ, FLASHTPA_SEQS, SWEEP_SHAPES, Config,
                      flashtpa_config, headsplit_config)
from .gen import Inputs, make_inputs, make_query_factors

__all__ = ["CONFIGS", "Config", "SWEEP_SHAPES", "FLASHTPA_HEADS", "FLASHTPA_RQ", "FLASHTPA_SEQS", "FLASHTPA_BATCHES",
           "flashtpa_config", "headsplit_config", "Inputs", "make_inputs", "make_query_factors"]
