"""fp64 CPU oracle for RMSNorm -- test infrastructure only (see oracle.py)."""
