"""Device-wide prefix scan, stream compaction and count-scan-emit packing for
AMD Instinct MI355X (gfx950), as hand-written HIP kernels behind a C ABI
(include/scan_wave64.h).  This package holds the kernels (csrc/), their
build (build.py), the ctypes binding (binding.py) and the seeded synthetic
input generators (inputs.py).

The binding is imported lazily so that `inputs` can be used without torch's
GPU stack; any binding call raises if the HIP library is missing.
"""

_BINDING_NAMES = {
    "scan_inclusive", "scan_inclusive_noalloc", "scan_exclusive", "scan_dim", "scan_segmented", "compact_if", "partition_if", "pack_offsets",
    "pack_emit_neighbors", "scan_copy", "scan_workspace_init", "scan_workspace_bytes", "scan_workspace_error",
    "plan", "version", "load_library", "workspaces", "ScanError", "Tuning",
}


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
