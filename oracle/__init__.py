"""fp64 CPU oracle of Forgetting Attention — test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this package.
It shares no code with the HIP library and imports nothing from it.
"""
from .fox_oracle import (  # noqa: F401
    log_sigmoid, gate_logf, gate_logf_bwd, rms_norm, rms_norm_bwd, fixed_gate_logf, cumsum_logf,
    reverse_cumsum,
    decay_bias_bruteforce, attn_probs_bruteforce, attn_fwd_bruteforce, attn_bwd_bruteforce,
    attn_fwd, attn_fwd_rows, attn_bwd, attn_bwd_tail, skip_bounds, skip_plan, shift_gate, shift_gate_bwd, kv_shift, kv_shift_bwd,
    out_norm_gate, out_norm_gate_bwd,
)
