"""Fingerprint of kernel sources: ties measured counter data to the exact
kernels it was taken on.  kernel_source_hash() covers every device source;
kernel_family_hash(family) only the files one kernel family is built from,
so a change to another family's file leaves its measurements valid."""
import glob
import hashlib
import os

_CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")

# device sources shared by every kernel
_COMMON = ("mx_args.hpp", "mx_device.hpp", "mx_pipe.hpp")
# the files each kernel family's launches are compiled from
FAMILY_FILES = {
    "tile": _COMMON + ("mx_tile.hip", "mx_tile_deep.hip"),
    "skinny": _COMMON + ("mx_skinny.hip", "mx_quantize.hpp"),
    "gemv": _COMMON + ("mx_gemv.hip",),
    "rows": _COMMON + ("mx_skinny_rows.hip",),
    "quant": _COMMON + ("mx_quant.hip", "mx_quantize.hpp"),
    "stream": _COMMON + ("mx_stream.hip",),
}


def _hash(files) -> str:
    h = hashlib.sha256()
    for f in sorted(files):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def kernel_source_hash() -> str:
    return _hash(glob.glob(os.path.join(_CSRC, "*.hip")) + glob.glob(os.path.join(_CSRC, "*.hpp")))


def kernel_family_hash(family: str) -> str:
    return _hash([os.path.join(_CSRC, f) for f in FAMILY_FILES[family]])
