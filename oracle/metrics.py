"""Acceptance metrics of speculative decoding (test infrastructure only).

"Faster Rollouts with MTP Speculative Decoding" (SkyRL docs), section
"Monitoring acceptance", names the counters: acceptance rate = accepted / drafted
tokens; mean acceptance length = tokens produced per target forward pass (1.0 means
no gain, k+1 is the ceiling); a per-depth breakdown pos_1..pos_k; raw counts of
drafted and accepted tokens. The same page's "Results" section prints a worked
example (per-depth 88.6 / 77.0 / 66.3 %, rate 77.3 %, mean length 3.32) whose
arithmetic fixes the definitions used here: pos_d is cumulative, P(a >= d), the
mean length is 1 + sum_d pos_d and the rate is the mean of pos_d, i.e. E[a] / k.
"""

import numpy as np


def acceptance_metrics(accepted_len, k):
    """Metrics over a batch of verify outcomes; accepted_len holds a in [0, k] per request-step."""
    a = np.asarray(accepted_len, dtype=np.int64).ravel()
    n = a.size
    drafted = n * k
    accepted = int(a.sum())
    pos = [float(np.mean(a >= d)) if n else 0.0 for d in range(1, k + 1)]
    return {
        "num_draft_tokens": drafted,
        "num_accepted_tokens": accepted,
        "acceptance_rate": accepted / drafted if drafted else 0.0,
        "mean_acceptance_length": 1.0 + (accepted / n if n else 0.0),
        "pos": pos,
        "histogram": np.bincount(a, minlength=k + 1)[: k + 1].tolist(),
        "emitted_tokens": accepted + n,
    }
