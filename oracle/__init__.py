"""CPU oracle for the sparse MoE block. Test infrastructure only: imported by tests/, by the
package's smoke check and by the benchmark's CPU-baseline leg, never by the product path."""
from .moe_oracle import *  # noqa: F401,F403
