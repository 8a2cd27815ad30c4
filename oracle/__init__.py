"""CPU oracle for the sparse mixture-of-experts feed-forward layer (forward and
backward passes).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table
or helper with the HIP library; it reads only inputs produced by the seeded
generators.

Sources (cited by title and section throughout):

* [LLM-T11]  "Mixture of Experts", chapter 11 of the LLM tutorial
  (llm-tutorial.darvinyi.com/ch11-moe).
* [ITM-14]   "Mixture of experts -- more parameters, same compute per token",
  chapter 14 of the Inside the Model guide.
* [LM-33]    "Chapter 33 -- Mixture of Experts (MoE)", language-modelling notes
  (karam-nus.github.io).
* [NNV-15]   "Mixture-of-Experts", chapter 15 of Neural Networks, Visually.
* [TA]       "Mixture of experts (MoE)", Tech Atlas glossary entry.

Modules:

* ``moe_oracle`` -- numpy float64 definition of the forward pass, step by step
  (router scores, ordered top-k, gates, capacity, permutation, experts,
  gate-weighted sum, shared experts), and of the routing statistics a batch
  yields (load fractions, mean router probabilities, balance loss, drop rate,
  loss-free bias update).
* ``moe_backward`` -- numpy float64 backward pass of the same layer with the
  routing held fixed: expert-output and gate gradients, the chain rule through
  each expert, the gate Jacobians, the balance-loss gradient and the router.
* ``brute``      -- pure-Python loops over tiny inputs: a second, independent
  spelling of the same definition that also counts multiplies.
* ``accounting`` -- parameter and multiply counts the pages print.

Parity status: every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_pins.py`` (brute force, closed forms, special cases that
reduce to library routines, invariants, and the numbers the pages print) or,
for the backward pass, ``tests/test_backward_pins.py`` (finite differences of
the forward, torch.autograd of an independent spelling, closed forms).
"""

from . import accounting, brute, moe_backward, moe_oracle  # noqa: F401
