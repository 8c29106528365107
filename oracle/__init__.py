"""fp64 CPU oracle for the PRR decode step: test infrastructure only (tests, smoke check, CPU-baseline timing)."""
