"""CPU oracle for the vocab-side draft-and-verify step of MTP speculative decoding.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls, links or
executes this package. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it. It shares no code, constant table or helper with the HIP
library; the two meet only through the seeded synthetic inputs (the `synth`
package, which holds no arithmetic of the method).

Everything here is plain, slow and written to be checked by eye against the
pages it follows:

* "The Tiny Draft Model Hidden Inside Qwen" (divagr.com), sections "One step
  deeper than the main model" and "What vLLM and SGLang do with the weights":
  the MTP drafter projects through the same vocabulary head as the main model.
* same page, section "How the draft becomes real output": the verifier runs one
  pass over every draft position, produces a distribution at each, keeps the
  longest agreeing prefix, replaces the first rejected slot with a draw from a
  corrected distribution; greedy verification returns exactly what ordinary
  greedy decoding returns.
* "Speculative Decoding and MTP: Why Guessing Is Free" (DEV Community), sections
  "Speculative decoding: draft, then verify" (k correct guesses give k+1 tokens)
  and "It's exact, not approximate" (the output law equals the target's).
* "Faster Rollouts with MTP Speculative Decoding" (SkyRL docs), section
  "Monitoring acceptance" (the acceptance metrics) and "Results" (a worked
  example that fixes their definitions).

The pages state the properties of the acceptance test but print no formula. The
rule used here is the standard speculative-sampling rule (Leviathan, Kalman &
Matias 2023; Chen et al. 2023): accept draft d with probability min(1, p(d)/q(d)),
else draw from normalize(max(0, p - q)); after k acceptances draw a bonus token
from the last target distribution. Random numbers come from Philox4x32-10
(Salmon, Moraes, Dror & Shaw, SC'11), written here from its published definition.

Layers:
  numerics  (fp64)        : decode_bf16, lm_head_logits, softmax
  decision rule           : greedy_verify, stochastic_verify, inverse_cdf,
                            residual_weights, sample_drafts,
                            greedy_verify_ragged, stochastic_verify_ragged
  random numbers          : philox.philox4x32_10, philox.verify_uniforms
  metrics                 : metrics.acceptance_metrics
  MTP input fusion        : mtp_input.rms_norm, fused_input, mtp_input_fuse
  top-k soft-CE draft loss: draft_loss.topk_teacher, soft_targets, draft_loss,
                            draft_loss_grad

Every function is pinned by a `-m "not gpu"` test against something other than
itself (exact rational enumeration, closed forms, library routines, an
independent Philox source, the pages' worked example). No function is parity
unpinned.
"""

from .verify import (
    decode_bf16,
    lm_head_logits,
    softmax,
    greedy_verify,
    residual_weights,
    inverse_cdf,
    stochastic_verify,
    sample_drafts,
    verify_greedy_from_hidden,
    verify_sample_from_hidden,
    draft_from_hidden,
    greedy_verify_ragged,
    stochastic_verify_ragged,
    verify_greedy_ragged_from_hidden,
    verify_sample_ragged_from_hidden,
)
from .mtp_input import rms_norm, fused_input, mtp_input_fuse
from .draft_loss import topk_teacher, soft_targets, draft_loss, draft_loss_grad, draft_loss_row
from .philox import philox4x32_10, uniform24, verify_uniforms
from .metrics import acceptance_metrics

__all__ = [
    "decode_bf16", "lm_head_logits", "softmax", "greedy_verify",
    "residual_weights", "inverse_cdf", "stochastic_verify", "sample_drafts",
    "verify_greedy_from_hidden", "verify_sample_from_hidden", "draft_from_hidden",
    "greedy_verify_ragged", "stochastic_verify_ragged", "verify_greedy_ragged_from_hidden",
    "verify_sample_ragged_from_hidden",
    "rms_norm", "fused_input", "mtp_input_fuse",
    "topk_teacher", "soft_targets", "draft_loss", "draft_loss_grad", "draft_loss_row",
    "philox4x32_10", "uniform24", "verify_uniforms", "acceptance_metrics",
]
