"""CPU oracle of the mixture-of-experts FFN forward -- TEST INFRASTRUCTURE.

Only tests/, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg
may import this package.  The GPU library never does.

The arithmetic lives in ``moe_oracle.c`` (plain C, fp64); this module compiles
it with gcc and wraps it with ctypes.  Parity status of each function is listed
in ``moe_oracle.h``.
"""
from .oracle import (build, load, params_of, route, permute, forward,  # noqa: F401
                     router_logits, mxfp4_value, activation, activation1, OrcParams)
