"""MI355X-native DSA indexer -> top-2,048 -> sparse MLA read (gfx950 HIP kernels behind a C ABI).

The compute entry points live in ``sparse_attention_12_amd.binding`` (loaded
on first use; it raises if the HIP library is missing).  ``workloads`` draws
seeded synthetic inputs and ``costmodel`` holds the cache/work arithmetic.
"""
__all__ = ["binding", "workloads", "costmodel"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
