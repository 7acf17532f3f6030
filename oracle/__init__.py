"""CPU oracle for the ReplaySSM step and flush -- test infrastructure only.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The GPU library never does, and the two share no code."""
