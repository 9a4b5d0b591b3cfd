"""CPU oracle for the MoE layer.  TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  It shares no code with the HIP library
(token_routing_shuffle_amd) and imports nothing from it.

Parity status of each function (what pins it is in tests/test_oracle_*.py):
  logits, select, route, sigmoid_keys, oracle_expf, ffn, expert_ffn,
  shared_ffn, moe_output, shuffle, gather, combine, build_lut: pinned.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import lib  # noqa: F401
