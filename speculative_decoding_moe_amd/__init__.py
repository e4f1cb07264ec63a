"""MoE verify-block hot path for MI355X (gfx950).

The library is libmoeverify.so (C ABI: include/moe_verify.h); ``binding`` wraps it with the same
names. Importing ``binding`` requires the built library and fails loudly without it.
"""


def __getattr__(name):
    if name in ("binding",):
        import importlib
        return importlib.import_module(f"{__name__}.binding")
    raise AttributeError(name)
