"""CPU oracle (test infrastructure only; never imported by the library)."""
from .dspark_oracle import (draft, draft_workload, schedule, verify, widen,  # noqa: F401
                            philox4x32_10, gumbel_uniform_bits, gumbel_noise)
