"""CPU oracle of the TokenMixer-Large block-stack forward (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package. The product path (``token_moe_amd``) never does.
"""
from .tmx_oracle import *  # noqa: F401,F403
