"""fp64 CPU oracle (test infrastructure only; see linattn_oracle's header)."""
from .linattn_oracle import (bounded_gate, chunked_fwd, decode_step,  # noqa: F401
                             recurrent_fwd, recurrent_fwd_heads, sigmoid)
