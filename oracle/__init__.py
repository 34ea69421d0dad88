"""CPU oracle of the sparse MoE FFN layer (float64).  Test infrastructure only: imported
solely by tests/, __graft_entry__.smoke() and the CPU-baseline leg of bench.py."""
from . import moe_ref  # noqa: F401
