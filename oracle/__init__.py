"""Float64 CPU oracle of the REINFORCE Zero learner hot path.

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and
the benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP kernels.  See reinforce_zero.py (learner path) and
rollout_sampler.py (rollout-side draw), run_diagnostics.py (run-level
diagnostics), mx_head.py (the MX-format head), lora_head.py (a LoRA
adapter on the head) and score_centering.py (the score-centering update)
for the definitions and sources.
"""
from .reinforce_zero import *  # noqa: F401,F403
from .rollout_sampler import *  # noqa: F401,F403
from .run_diagnostics import *  # noqa: F401,F403
from .mx_head import *  # noqa: F401,F403
from .lora_head import *  # noqa: F401,F403
from .score_centering import *  # noqa: F401,F403
from .reinforce_zero import __all__ as _rz_all
from .rollout_sampler import __all__ as _rs_all
from .run_diagnostics import __all__ as _rd_all
from .mx_head import __all__ as _mx_all
from .lora_head import __all__ as _lo_all
from .score_centering import __all__ as _sc_all

__all__ = (list(_rz_all) + list(_rs_all) + list(_rd_all) + list(_mx_all)
           + list(_lo_all) + list(_sc_all))
