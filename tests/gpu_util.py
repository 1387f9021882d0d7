"""Helpers shared by the GPU parity tests (marshalling and comparisons only)."""
from __future__ import annotations

import numpy as np

BF16_MAX_ABS = 2e-2  # max |O_gpu - O_oracle| for bf16 outputs
BF16_REL_L2 = 5e-3  # ||O_gpu - O_oracle||_2 / ||O_oracle||_2
FP8_REL_L2 = 5e-2  # 8-bit paths in general: the kernels quantise P against a running max
# 8-bit paths when the kernel's quantisation reference equals the oracle's row
# max (the row max sits in the first tile the kernel reads and the request is
# not split): the E4M3 codes of P are then the oracle's (the extend's are a
# power of two apart, exact while they stay normal), so what is left is the
# bf16 rounding of O, at most 2^-8 relative per element (bf16 keeps 8
# significant bits), plus fp32 sums and products, far below that
FP8_REL_L2_SAME_MAX = 4e-3
LSE_ABS = 2e-3  # lse is fp32, scores from bf16 inputs and fp32 accumulation


def torch_mod():
    import torch
    return torch


def dev_bf16(x):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda").to(torch.bfloat16)


def dev_i32(x):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to("cuda")


def dev_u8(x):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).to("cuda")


def dev_i8(x):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int8)).to("cuda")


def dev_qk8(x, spec):
    """Q or K codes of an 8-bit batch: int8 for the INT8 Sage dtype, else E4M3 bytes."""
    return dev_i8(x) if spec.dtype == "int8" else dev_u8(x)


def kv_dtype_of(pkv, spec):
    return pkv.PKV_SAGE_INT8 if spec.dtype == "int8" else pkv.PKV_FP8_E4M3


def qk_codes_of(spec):
    """How the oracle reads the batch's Q and K bytes."""
    return "int8" if spec.dtype == "int8" else "e4m3"


def dev_f32(x):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")


def host(t) -> np.ndarray:
    torch = torch_mod()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy().astype(np.float64)


def rel_l2(got, ref) -> float:
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(np.asarray(got, np.float64) - ref) / (den if den > 0 else 1.0))


def assert_bf16_close(got, ref, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = float(np.abs(got - ref).max()) if got.size else 0.0
    rel = rel_l2(got, ref)
    assert err <= BF16_MAX_ABS and rel <= BF16_REL_L2, f"{what}: max abs {err:.3e}, rel L2 {rel:.3e}"
    return err, rel


def assert_lse_close(got, ref, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    inf = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), inf), f"{what}: -inf pattern differs"
    if (~inf).any():
        err = float(np.abs(got[~inf] - ref[~inf]).max())
        assert err <= LSE_ABS, f"{what}: lse max abs {err:.3e}"


def check_rel_l2(got, ref, what="", bound=FP8_REL_L2):
    """rel L2 of an 8-bit result against the oracle, printed and checked."""
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    rel = rel_l2(got, ref)
    print(f"{what}: rel L2 {rel:.3e} (bound {bound:.1e})", flush=True)
    assert rel <= bound, f"{what}: rel L2 {rel:.3e} > {bound:.1e}"
    return rel
