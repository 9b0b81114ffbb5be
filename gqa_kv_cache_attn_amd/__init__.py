"""MI355X-native single-token grouped-query decode attention over a KV cache.

The compute path is ``libgqa_decode.so`` (hand-written HIP for gfx950 behind a
C ABI declared in ``include/gqa_decode.h``). ``binding`` is a thin ctypes
layer with the same entry-point names; it only marshals pointers, sizes and
the stream. It is imported lazily so that ``inputs`` (the seeded workload
generator) can be used on machines without the built library.
"""

__all__ = [
    "gqa_decode",
    "prepare_gqa_decode",
    "launch_gqa_decode_prepared",
    "gqa_validate_args",
    "gqa_plan",
    "GqaError",
]


def __getattr__(name):
    if name in __all__ or name in ("binding", "GqaPrepared", "library_path"):
        import importlib

        binding = importlib.import_module(__name__ + ".binding")
        if name == "binding":
            return binding
        return getattr(binding, name)
    raise AttributeError(name)
