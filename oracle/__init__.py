"""CPU oracle (fp64) for the log-linear Mamba-2 forward pass.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this package. It shares no code with the HIP
library and never imports it.
"""

from .loglinear import (  # noqa: F401
    as_f64, bit_length, bruteforce, bruteforce_rows, level, level_matrix,
    num_levels, recurrent,
)
from .deltanet import gdn_attention, gdn_bruteforce, gdn_recurrent, gdn_recurrent_step  # noqa: F401
