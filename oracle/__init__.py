"""Float64 CPU oracle for one training step of the small decoder-only GPT.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
GPU library never calls it, and it shares no code with the GPU library: it is
plain numpy in float64, slow and written to be checked by eye against the
pages that define the model.

Sources (cited by page title and section; the pages are the nanochat web
pages this project was built from):

* "nanochat explainer" (cloudtoid LLM book), section "Modern architecture
  choices": RoPE, RMSNorm, ReLU-squared, QK-norm, untied embeddings.
* same page, "Architecture Choices" -> "RoPE Intuition": q and k are rotated by
  angles proportional to position so that q.k depends on relative distance.
* same page, "Architecture Choices" -> "ReLU² Sparsity": zero the negatives,
  square the positives.
* same page, "The 'One Dial' Design" -> "How dimensions are derived":
  d_model = 64 * depth, heads = d_model / 128, head_dim = 128, FFN = 4 * d_model.
* same page, "The Full Pipeline" -> "Pretraining": causal next-token
  prediction with a cross-entropy loss; the optimizer step (Muon for the
  matrices, AdamW for the embedding and unembedding, cosine schedule with
  warmup, clipping at 1.0, weight decay 0.1) is in ``optim.py``.

Readings where the pages are silent:
parameter-free RMSNorm with eps = 1e-6 inside the square root; pre-norm
residual blocks plus one final norm before the LM head; QK-norm then RoPE
(the order is immaterial because the rotation is orthogonal); split-half RoPE
pairs (i, i + hd/2) rotated by +t*theta_i with theta_i = base^(-2i/hd);
attention scale 1/sqrt(head_dim); causal mask including the diagonal; no
biases, no dropout, no logit cap; loss = mean over all B*T positions in nats.

Pin status of every public function is stated in its docstring; all are
pinned by the CPU tests in ``tests/test_oracle_*.py`` (finite differences,
closed forms, invariants, an independent torch float64 autograd model, and the
page-printed depth-dial figures under ``tests/golden/``).
"""

from .model import (  # noqa: F401
    Config,
    derive_config,
    param_shapes,
    param_count,
    forward,
    forward_backward,
    forward_logits,
)
from . import ops  # noqa: F401
from . import optim  # noqa: F401
