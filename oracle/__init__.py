"""CPU oracle of the HiSparse decode-step swap-in resolver.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.
"""
