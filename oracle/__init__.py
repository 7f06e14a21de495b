"""CPU oracle for exact attention (fp64) and a model of the online recurrence.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import anything from here.
"""
