"""Guard for tests that start another program (a compiler, a helper)."""

import sys

import pytest


def skip_if_gpu_initialised():
    """Skip in a process that has already initialised the GPU: such a process
    starts no other program."""
    torch = sys.modules.get("torch")
    if torch is not None and torch.cuda.is_initialized():
        pytest.skip("this process has initialised the GPU and starts no other program")
