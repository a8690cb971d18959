"""SVG2 semantic-aware-permutation sparse attention for AMD MI355X (gfx950).

The five steps of the method run in HIP kernels behind the C ABI of
include/svg2.h; this package is the thin Python binding over it
(``binding``), a layer driver that chains the calls (``pipeline``), the
seeded synthetic-input generators (``synth``) and the build script
(``build``).
"""
from .binding import (Svg2Error, kmeans, lib, library_path, permute, select_topp, unpermute,  # noqa: F401
                      varblock_attn, version)

__all__ = ["Svg2Error", "kmeans", "lib", "library_path", "permute", "select_topp", "unpermute",
           "varblock_attn", "version"]
