"""CPU oracle for the JSSA sparse decode step.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the
benchmark's cpu_baseline leg may import, call or execute anything in this
package. It shares no code with the HIP path (token_level_sparse_kv_amd), and
the HIP path never imports it.
"""
from . import calib, jssa, numerics  # noqa: F401
