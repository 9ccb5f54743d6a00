"""CPU oracle of the OasisKV decode hot path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product library never does, and it shares no code
with the HIP path.
"""
