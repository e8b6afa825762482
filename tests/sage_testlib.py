"""Helpers shared by the GPU tests: device upload of seeded fields, fp16 comparisons."""
from __future__ import annotations

import sys

import numpy as np

import bit_vector_quantized_amd as sage


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def field(c, name):
    return c[name] if isinstance(c, dict) else getattr(c, name)


def log2k(c) -> int:
    return int(field(c, "K")).bit_length() - 1


def upload(c, device="cuda"):
    import torch

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    return dict(
        signs=t(field(c, "signs")), idx=t(field(c, "idx")), rcode=t(field(c, "rcode")),
        mu=t(np.asarray(field(c, "mu"), np.uint16).view(np.float16)),
        delta=t(np.asarray(field(c, "delta"), np.uint16).view(np.float16)),
        codebook=t(np.asarray(field(c, "codebook"), np.uint16).view(np.float16)),
        pi=t(np.asarray(field(c, "pi"), np.int32)),
    )


def upload_pack(c, device="cuda", identity_pi=False) -> sage.Packed:
    d = upload(c, device)
    L = log2k(c)
    V = int(field(c, "V"))
    return sage.pack(d["signs"], d["idx"], d["rcode"], d["mu"], d["delta"], d["codebook"],
                     None if identity_pi else d["pi"], L, V)


def fp16_ordered(bits: np.ndarray) -> np.ndarray:
    """Map fp16 bit patterns to integers ordered like the values (+0 and -0 both map to 0)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    return np.abs(fp16_ordered(a_bits) - fp16_ordered(b_bits))
