"""fp64 CPU oracle for the SageSLA attention forward (test infrastructure only)."""
