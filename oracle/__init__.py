"""CPU oracle for the token-choice MoE layer — TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 implementation of what the layer computes, used to check
the GPU library.  Only the test suite, the smoke check and the benchmark's CPU
baseline may import it; the GPU product path never does, and this package
imports nothing from it.

Sources (titles of the pages the method is taken from):

* "专家组合 (MoE)" lesson, AI Engineering from Scratch (phase 7, lesson 11):
  sections Concept (the replaced FFN and the gated sum), Load balancing
  (item 2 expert capacity + token dropping, item 3 auxiliary-loss-free
  bias), Shared experts, Fine-grained experts, Build it
  step 1 (the router function) and step 2 (the +-gamma bias controller),
  Exercises items 2 (hash router) and 3 (routing replay), Key terms.
* AREX article on The Ultimate MoE Training Handbook: the paragraph on router
  precision (fp32 router; softmax, sigmoid or sqrt(softplus) scoring) and the
  paragraph on the 64-expert top-8 teaching model (parameter counts).

Parity pins: every public function here is checked by ``tests/test_oracle_*``
against closed forms, library routines, brute force, finite differences or
numbers the pages print; ``oracle.pure`` codes the forward a second time in
plain Python loops, and the two are checked against each other.

PARITY UNPINNED: ``aux_loss`` / ``aux_grad_logits`` (the auxiliary
load-balancing loss): the pages name the loss but give no formula; the
Switch/GShard form is taken, and only its internal consistency (closed
forms, finite differences, autograd) is checked.
"""
from .moe import (  # noqa: F401
    SCORE_FNS,
    bf16_round,
    bf16_from_bits,
    score,
    route,
    splitmix_key,
    hash_route,
    aux_probs,
    aux_loss,
    aux_grad_logits,
    permute,
    expert_ffn,
    grouped_ffn,
    combine,
    bias_update,
    forward,
    backward,
    expert_backward_rows,
    gate_backward,
    router_backward,
    moe_ffn_params,
    dense_ffn_params,
)
