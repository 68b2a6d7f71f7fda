"""CPU oracle for one GPU's share of an expert-parallel MoE FFN layer.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or execute this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it. It shares no code with the GPU library (no kernels, headers, helpers,
tables or pre/post-processing); its inputs come from ``moe_workloads`` like the GPU side's.

Source of the method: "X-Stage: An Overlooked Pipeline Stage for Communication-Computation
Overlap in DiT Inference" (arXiv 2607.23264), Introduction, the MoE-layer paragraph: a router
picks one or more experts per token, Dispatch sends each token to its experts, each expert runs
Linear-1 (hidden -> intermediate), a SwiGLU activation and Linear-2 (intermediate -> hidden),
and Combine aggregates the top-k expert outputs with the router weights. The expert-wave
paragraph that follows it says waves group experts for locality and execution order only, so
the oracle has no schedule: every order of tiles computes the same layer.

Modules:
  moe_ref     the plain definition, float64 with explicit bfloat16 rounding points
  brute       scalar pure-Python loops (exact rationals where possible) for micro shapes
  invariants  special-case builders (identical experts, one expert, exact-integer case)
  burst_gap   the Burst-Gap model of Section 3 (issue time, period, capacity, design test)
  attention_ref  the attention forward of Section 4.3 (full, non-causal softmax(QK^T/sqrt(d))V)

Pins: every function here is checked by ``tests/test_oracle_*.py`` against something other
than itself (hand-worked golden cases, closed forms, library routines, brute force,
invariants). No function is "parity unpinned".
"""
