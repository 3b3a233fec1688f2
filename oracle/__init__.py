"""Float64 CPU oracle (test infrastructure only; see oracle.c)."""
