"""CPU oracle for the expert-parallel MoE layer (test infrastructure only).

Plain, slow, float64 NumPy code that states what the layer computes, written
from the pages' description of the method (route to the top-k experts,
dispatch each token to the owners of its experts, run each expert's gate/up/down
FFN, combine the results weighted by the route weights).  It shares no code
with the HIP path and neither imports the other.  Only the test suite, the
package smoke check and the benchmark's CPU-baseline leg may import it; the
product path never calls it.

Modules:
* ``moe``   routing, local filtering with the logical-to-physical replica map,
            stable expert-contiguous permutation, SwiGLU experts, combine, the
            shared expert, and a dense brute-force evaluation;
* ``fp8``   OCP E4M3 decode/encode and the block / per-token quantisers;
* ``eplb``  redundant-expert map for skewed routing and the load-balancing
            placement policy with its load simulation;
* ``arith`` the pages' byte and parameter arithmetic.

Parity pins live in ``tests/test_oracle_*.py``.  Parity unpinned: the exact bits
of float outputs (they depend on summation order; covered by tolerance), and E4M3
codes of the intermediate activation where two implementations' float32 values
straddle a rounding boundary.
"""
