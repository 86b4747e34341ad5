"""CPU oracle of the GSQ relaxed-quantization step.

TEST INFRASTRUCTURE, not part of the product. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import, call or execute anything in this package. It is a plain, slow, fp64
NumPy implementation written from the GSQ paper pages; it shares no code,
table or constant generator with the GPU library in
``post_weight_quantization_philox_amd`` and neither imports the other.

Every function is pinned by ``tests/test_oracle_*.py`` against facts that do
not come from the oracle itself (an independent Philox implementation, closed
forms, finite differences, brute force, the numbers the pages print).
"""

from .philox import (philox4x32_10, noise_words, uniform_from_word, gumbel,
                     logistic)
from .gsq import (GRID_INT2, GRID_TERNARY, GRID_INT3_LOCAL, GRID_INT3, N_LOGITS, Q_MAX,
                  CODE_BITS, LOCAL_OFFSETS, level_value, grid_levels,
                  candidate_codes, init_rtn, gptq_hessian, gptq, noise, relax_probs, ternary_terms,
                  relax_fwd, relax_bwd, recon_loss_grad,
                  recon_loss_grad_grouped, recon_loss_grad_offset, gram, recon_loss_grad_gram,
                  hard_loss, lion, harden, pack_codes,
                  unpack_codes, scales_to_f16_bits, harden_pack, tau_schedule,
                  round_bf16, step, quantize_layer)
