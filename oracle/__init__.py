"""CPU oracle for the HiLS attention hot path (test infrastructure only)."""
