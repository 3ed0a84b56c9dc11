"""CPU oracle for block-scaled FP4 quantisation -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product library (block_scaled_fp4_amax_amd) never
imports it and shares no code with it.

`oracle.ref` binds the plain C oracle (fp4_oracle.c); `oracle.exact` is an
independent exact-rational model used to pin the C oracle on small inputs.
"""
