"""Float64 CPU oracle of the Qwen3-style decoder layer.

Test infrastructure only: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the HIP path.
"""
from .qwen3_oracle import *  # noqa: F401,F403
