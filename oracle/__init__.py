"""fp64 CPU oracle for block-sparse attention with mean-pooled block selection.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import this package.  The HIP library
never calls it, links it or shares code with it, and it never imports the
HIP library.

Every function is the plain definition of one step, in float64, read from the
pages it cites:

* "Efficient Long-Context Modeling in Diffusion Language Models via Block
  Approximate Sparse Attention" (BA-Att): mean pooling and block logits
  (section 3.1, Eq. 2), top-kappa block mask (section 3.1 and Algorithm 1),
  attention restricted to kept block pairs (section 2, Eq. 1 and the
  "Block-Sparse Attention" paragraph).
* "Log-linear sparse attention in plain MLX" (README of loglinear-sparse-dit):
  repeated pooling, coarse-to-fine per-token top-k, KV enrichment with a
  level logit bias.
* The LoSA blog post (Locality-aware Sparse Attention, "LoSA method"
  section): active tokens by query MSE, cached prefix (O, LSE) reuse, and the
  prefix/suffix online-softmax merge.

Nothing here is blocked, fused or reordered beyond what those definitions
state.  Library primitives used as steps: numpy matmul, sort, exp, log.

basa_oracle_ref.cpp is a second, independent fp64 reference of the BA-Att
steps (pooling, block logits, top-k, block-sparse and merged attention) in
plain C++ loops, compiled with g++ into liboracle_ref.so and reached through
oracle.cref.  Both references are pinned to the same independent facts and
checked against each other.
"""
from .basa_oracle import *  # noqa: F401,F403
from .basa_oracle import __all__  # noqa: F401
