"""Plain, slow float64 CPU oracle for the chunked test-time-training memory.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.  It
shares no code with the HIP library (no kernels, headers, helpers, constants or
pre/post-processing) and it never imports that library.

What it computes, in the pages' own order (a per-token loop, float64):

* ``linear_forward`` -- the linear memory ``z = M q`` trained by gradient steps
  on ``l = 1/2 ||M k - v||^2`` with gradients taken at the chunk-start state,
  Titans momentum and forgetting.  Pinned by the pages' worked examples and by
  closed forms (delta rule, linear attention, batch gradient descent, one-step
  loss contraction, decay unrolling, constant-gate momentum expansion).
* ``linear_backward`` -- the outer gradient of ``linear_forward`` with respect
  to every input and the initial state, by reverse mode through the same
  per-token loop.  Pinned by central finite differences of the pinned forward,
  the pages' scalar outer-gradient examples, and the closed-form gradients of
  weighted linear attention.
* ``linear_forward_chunk_gates`` / ``linear_backward_chunk_gates`` -- the same
  iteration with gates shared by the tokens of a chunk.  Pinned by the closed
  form that the shared gates allow (a geometric decay sum inside a chunk) and
  by finite differences of the chunk gates.
* ``mlp_forward`` -- the same schedule for a 2-layer MLP memory
  ``f(u) = u + SiLU(u W1) W2`` with gradients by explicit backprop.  Pinned by
  torch.autograd (a library routine), finite differences, and by agreement of
  an autograd-driven generic loop whose linear instance is pinned by the
  worked examples.
* ``deep_forward`` -- the same schedule for a deep memory of any depth
  L >= 2, ``f(u) = u + SiLU(...SiLU(u W_1)...) W_L``, with its own explicit
  backprop (``deep_chunk_grads``).  Pinned by torch.autograd and finite
  differences at depths 2-4, by the generic autograd loop at depths 2-4, by
  agreement with ``mlp_forward`` at depth 2, and by the plain read (no
  update) at theta = eta = alpha = 0.

Every function here is pinned by tests in ``tests/test_oracle_*.py``; none is
"parity unpinned".
"""

from .memory import (deep_chunk_grads, deep_forward, linear_backward, linear_backward_chunk_gates, linear_forward,
                     linear_forward_chunk_gates, mlp_chunk_grads, mlp_forward, silu, silu_grad)

__all__ = ["linear_forward", "linear_backward", "linear_forward_chunk_gates", "linear_backward_chunk_gates",
           "mlp_forward", "silu", "silu_grad", "mlp_chunk_grads", "deep_forward", "deep_chunk_grads"]
