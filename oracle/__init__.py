"""CPU oracle for the GPT-2 training step -- TEST INFRASTRUCTURE ONLY.

Plain, slow NumPy implementation of what one training step computes
(forward, backward, global-norm clip, AdamW, learning-rate schedule, seeded
init).  Only the test suite, the package's smoke entry and the benchmark's
cpu_baseline leg may import it; the product path never does.  It shares no
code with the HIP library or its Python binding and imports neither.

Sources (cited by page title and section):
  PDS = "Pretraining and adapting a language model on a dependency-free stack"
        (model text around Fig. 1; §4 recipe paragraphs: optimisation,
        precision, batch (§4.4); the four-level checks).
  GLM = "Was ein Sprachmodell vorhersagt" (grow a language model course
        outline; activity table rows 4-12: embeddings, scaled dot-product
        attention Q.K^T/sqrt(d) with causal mask, block, cross-entropy,
        AdamW, schedule, global-norm clipping).

Every function is pinned by tests/test_oracle_*.py against closed forms,
printed values, invariants, brute force or finite differences; nothing here
is "parity unpinned".
"""
from .model import (Config, CONFIGS, tensor_specs, n_params, layout, init_params,
                    flatten, unflatten, forward, backward, loss_and_grads)
from .optim import lr_at, global_norm, clip_adamw
from . import ops, rng

__all__ = ["Config", "CONFIGS", "tensor_specs", "n_params", "layout", "init_params",
           "flatten", "unflatten", "forward", "backward", "loss_and_grads",
           "lr_at", "global_norm", "clip_adamw", "ops", "rng"]
