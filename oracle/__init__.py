"""Plain, slow fp64 CPU oracle of TurboQuant-style online vector quantization.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.  Only the test suite
(tests/), the smoke check in __graft_entry__.py and the CPU-baseline leg of
bench.py may import it.  The HIP library never calls it, and it shares no code,
table or constant generator with the library: both implement the same written
definitions independently.

Modules:
  philox      Philox4x32-10 counter RNG, Box-Muller, bf16 rounding, plan randomness
  codebook    Lloyd-Max codebook for the rotated-coordinate Beta law
  rotation    randomized Hadamard rotation as dense fp64 matrices
  turboquant  encode / query preparation / estimate / top-k; TurboQuant-MSE encode and
              dequantization
  layout      packed byte layout of the codes
  policy      outlier channels by variance; appending encoded tokens to a cache

Parity status of each function is listed in the module docstrings.  Every
function has an external pin (tests/test_oracle_pins.py); the Philox bit stream
is pinned by the generator's published known-answer vectors.
"""
