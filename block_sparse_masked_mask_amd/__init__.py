"""Block-sparse masked attention for MI355X (gfx950).

The compute lives in libbsm.so (HIP kernels behind the C ABI in include/bsm.h);
`block_sparse_masked_mask_amd.bsm` is its ctypes binding and `.synth` holds the
seeded input generators. Submodules load lazily so that importing the package
does not require the built library.
"""

_BINDING = ("resolve_dflash_is_causal", "block_mask_shape", "build_block_mask",
            "dynamic_topk_mask", "dflash_dense_mask", "masked_attn_fwd", "create_mask",
            "DFlash", "BlockMask", "Geometry", "geometry_of", "lib")


def __getattr__(name):
    if name in _BINDING:
        from . import bsm
        return getattr(bsm, name)
    raise AttributeError(name)
