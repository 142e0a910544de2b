"""The oracle: a plain fp64 CPU implementation of the registration step.

Test infrastructure only: the test suite, the smoke check and the CPU-baseline
leg of ``bench.py`` may import it. The product path (the HIP library and its
binding) never does.
"""
