"""CPU oracle of the importance-aware KV decode step.

TEST INFRASTRUCTURE ONLY: only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this package.
"""
