"""CPU oracle for batched draft verification -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the CPU-baseline leg of the benchmark may import
this package.  The product path (``draft_verification_softmax_amd``) never does, and the
two share no code.
"""
