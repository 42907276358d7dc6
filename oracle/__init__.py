"""CPU oracle for the block-based fixed-length BF16 codec.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT: only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import anything from here.
"""
