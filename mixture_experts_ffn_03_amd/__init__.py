"""MI355X-native mixture-of-experts FFN forward (HIP kernels behind a C ABI).

``MoE`` (layer.py) is the Python surface; ``_lib`` is the ctypes binding of
``libmoe_mi355x.so`` (include/moe_mi355x.h); ``synth`` draws seeded inputs.
Importing this package does not load the library; the first call that needs
it does, and fails loudly if it has not been built.
"""
from .layer import MoE, from_config  # noqa: F401
