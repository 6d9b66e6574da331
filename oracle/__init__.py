"""CPU parity oracle for vocab-row selection -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The GPU product path never calls it and shares no code with it.
"""
