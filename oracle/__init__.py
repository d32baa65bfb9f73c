"""fp64 CPU oracle for the decode path.  Test infrastructure only: imported by
tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg, never by the
product path."""
from .oracle import (Oracle, KVCache, rmsnorm, rope_angles, apply_rope, silu,  # noqa: F401
                     softmax, attend, greedy, lane_partials)
