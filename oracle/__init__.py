"""fp64 CPU oracle for the VLA scan and its gradients: test infrastructure only (see vla_oracle)."""
from .vla_oracle import oracle_project_u, oracle_scan  # noqa: F401
from .vla_oracle_grad import oracle_scan_grad  # noqa: F401
