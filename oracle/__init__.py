"""fp64 CPU oracle for cascade verify attention.  Test infrastructure only:
imported by tests, the smoke check and the bench's CPU-baseline leg, never by
the product path."""
