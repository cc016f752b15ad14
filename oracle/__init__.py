"""CPU oracle of the W4.4A8 mixed-precision linear layer.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py``; never by the product package.
"""
from .mixllm_oracle import *  # noqa: F401,F403
from . import mixllm_oracle as core  # noqa: F401
