"""CPU oracle of the MoE-layer forward (test infrastructure only).

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product library never links or calls it.
"""
