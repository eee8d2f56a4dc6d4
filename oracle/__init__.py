"""fp64 CPU oracle for the VLA scan: test infrastructure only (see vla_oracle)."""
from .vla_oracle import oracle_project_u, oracle_scan  # noqa: F401
