"""GPU parity of the gated output norm (gdn_gated_rmsnorm) against the oracle's fp64 version on the
same (already rounded) inputs.  Tolerance: fp32 output max|err| <= 1e-5 * rms(y_ref); bf16 output
|err| <= (2^-8 + 1e-5) |y_ref| element by element: one round-to-nearest bf16 rounding of the result
is half an ulp, up to 2^-8 of the value just above a power of two, and the fp32 arithmetic before it
adds a few 1e-7."""
import numpy as np
import pytest
import torch

from gated_deltanet_delta_amd import gdn_gated_rmsnorm
from helpers import assert_close
from oracle import oracle as O

pytestmark = pytest.mark.gpu

BF16_REL = 2.0 ** -8 + 1e-5


def inputs(rows, d, z_dtype, seed):
    rng = np.random.default_rng(seed)
    x = (0.3 * rng.standard_normal((rows, d))).astype(np.float32)
    x[3] = 0.0                                   # an all-zero row: output zero
    x[5] *= 1e6                                  # large rows: scale-free up to eps
    x[7] *= 1e-4                                 # tiny rows: eps damps them
    z = torch.from_numpy(rng.standard_normal((rows, d)).astype(np.float32)).to(z_dtype)
    z[9] = 40.0                                  # silu saturates to z
    z[11] = -40.0                                # silu nearly closes
    w = rng.uniform(0.5, 1.5, d).astype(np.float32)
    return torch.from_numpy(x), z, torch.from_numpy(w)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("z_dtype,out_dtype", [(torch.bfloat16, torch.bfloat16), (torch.bfloat16, torch.float32),
                                               (torch.float32, torch.float32), (torch.float32, torch.bfloat16)])
def test_gated_rmsnorm_matches_oracle(d, z_dtype, out_dtype):
    rows = 1000 + d // 64                         # not a multiple of the rows per workgroup
    x, z, w = inputs(rows, d, z_dtype, seed=d)
    y = gdn_gated_rmsnorm(x.cuda(), z.cuda(), w.cuda(), 1e-6, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref = O.gated_rmsnorm(x.double().numpy(), z.double().numpy(), w.double().numpy(), 1e-6)
    got = y.double().cpu().numpy()
    assert np.all(got[3] == 0.0)
    if out_dtype == torch.float32:
        assert_close(f"gated rmsnorm d={d} z {z_dtype} out fp32", y, ref, 1e-5)
    else:
        err = np.abs(got - ref)
        worst = float(np.max(err / (np.abs(ref) + 1e-30)))
        print(f"  gated rmsnorm d={d} z {z_dtype} out bf16: max rel err {worst:.3e} (tol {BF16_REL:.3e})", flush=True)
        assert np.all(err <= BF16_REL * np.abs(ref) + 1e-30)


def test_gated_rmsnorm_on_prefill_output_shape():
    """On o of a Qwen3-Next-shaped prefill ([B, T, Hv, dv] viewed as rows of dv): fp32 in, bf16 out."""
    rng = np.random.default_rng(7)
    x = torch.from_numpy((0.5 * rng.standard_normal((1, 256, 32, 128))).astype(np.float32))
    z = torch.from_numpy(rng.standard_normal((1, 256, 32, 128)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy(rng.uniform(0.5, 1.5, 128).astype(np.float32))
    y = gdn_gated_rmsnorm(x.cuda(), z.cuda(), w.cuda(), 1e-6)
    torch.cuda.synchronize()
    assert y.shape == x.shape and y.dtype == torch.bfloat16
    ref = O.gated_rmsnorm(x.double().numpy(), z.double().numpy(), w.double().numpy(), 1e-6)
    got = y.double().cpu().numpy()
    assert np.all(np.abs(got - ref) <= BF16_REL * np.abs(ref) + 1e-30)
