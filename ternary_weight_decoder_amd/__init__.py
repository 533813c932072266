"""MI355X (gfx950) ternary-weight x int8-activation projections.

The product is the C-ABI library ``libbitnet_tm.so`` (header
``include/bitnet_tm.h``) built from ``csrc/``; ``binding`` is a thin torch-facing
wrapper with the same entry-point names.  ``synth`` holds seeded input
generators.  Importing this package does not load torch or the library; the
binding names below are resolved on first use.
"""

_BINDING_NAMES = {
    "bitnet_ternarize_pack", "bitnet_quant_act", "bitnet_ternary_matmul",
    "bitnet_ternary_matmul_q8", "bitnet_ternary_matmul_grouped", "GroupedPlan",
    "BitnetError", "bitnet_packed_bytes", "bitnet_matmul_workspace_bytes",
    "bitnet_ternarize_workspace_bytes", "bitnet_grouped_workspace_bytes",
}


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
