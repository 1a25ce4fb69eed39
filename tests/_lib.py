"""Shared test helpers: load (building if needed) the HIP library binding."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "learned_token_pruning_amd", "libtokengate.so")


def binding():
    if not os.path.exists(LIB):
        from learned_token_pruning_amd import build as _b
        _b.build()
    from learned_token_pruning_amd import tokengate
    return tokengate


def gpu_available():
    import torch
    return torch.cuda.is_available()
