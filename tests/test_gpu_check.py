"""dspark_check_inputs against a NumPy count of the same values: anchors and
tokens outside [0, V), NaN / +inf logits (-inf is a mask and allowed),
non-finite weights, confidences outside [0, 1].  Bad values are planted at
seeded positions, including the unaligned ends of a tensor that starts off a
16-byte boundary."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from draft_sampling_verification_w1_amd import dspark
    dspark.lib()
    return torch.device("cuda:0")


BF16_NAN, BF16_NNAN, BF16_PINF, BF16_NINF = 0x7FC0, 0xFFC1, 0x7F80, 0xFF80


def _plant_bf16(rng, a, n_nan, n_pinf, n_ninf):
    flat = a.reshape(-1)
    idx = rng.choice(flat.size, n_nan + n_pinf + n_ninf, replace=False)
    # always hit both ends (the unaligned head and tail of the device buffer)
    idx[0], idx[-1] = 0, flat.size - 1
    vals = [BF16_NAN if i % 2 == 0 else BF16_NNAN for i in range(n_nan)] + \
           [BF16_PINF] * n_pinf + [BF16_NINF] * n_ninf
    flat[idx] = np.array(vals, np.uint16)


def _plant_f32(rng, a, n_nan, n_pinf, n_ninf):
    flat = a.reshape(-1)
    idx = rng.choice(flat.size, n_nan + n_pinf + n_ninf, replace=False)
    idx[0], idx[-1] = 0, flat.size - 1
    flat[idx] = np.array([np.nan] * n_nan + [np.inf] * n_pinf + [-np.inf] * n_ninf, np.float32)


def _to_dev_offset(a, dev, dtype, offset):
    """Copy `a` to the GPU as a contiguous tensor that starts `offset`
    elements into its allocation (off a 16-byte boundary when offset > 0)."""
    if dtype == torch.bfloat16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    buf = torch.empty(t.numel() + offset, dtype=t.dtype, device=dev)
    view = buf[offset:].view(t.shape)
    view.copy_(t.to(dev))
    return view


def _reference(arrs, bf16, V):
    from draft_sampling_verification_w1_amd import synth

    def f32(x):
        return synth.bf16_bits_to_f32(x) if bf16 else x

    U, T, W1, W2, A, X, c = arrs
    nanpinf = lambda x: int(np.count_nonzero(np.isnan(f32(x)) | np.isposinf(f32(x))))
    return {
        "anchors": int(np.count_nonzero((A < 0) | (A >= V))),
        "tokens": int(np.count_nonzero((X < 0) | (X >= V))),
        "U": nanpinf(U),
        "T": nanpinf(T),
        "W": int(np.count_nonzero(~np.isfinite(f32(W1)))) + int(np.count_nonzero(~np.isfinite(f32(W2)))),
        "c": int(np.count_nonzero(~((c >= 0) & (c <= 1)))),
    }


@pytest.mark.parametrize("bf16,R,gamma,V,offset", [(True, 5, 3, 1003, 3), (False, 5, 3, 1003, 1),
                                                   (True, 64, 4, 100003, 0), (True, 1, 1, 7, 5)])
def test_check_inputs_counts(dev, bf16, R, gamma, V, offset):
    from draft_sampling_verification_w1_amd import dspark, synth
    rng = np.random.default_rng(R * 1000 + V)
    dt = torch.bfloat16 if bf16 else torch.float32
    f = (lambda x: synth.f32_to_bf16_bits(x)) if bf16 else (lambda x: x)
    U = f(rng.standard_normal((R, gamma, V), dtype=np.float32) * 4)
    T = f(rng.standard_normal((R, gamma + 1, V), dtype=np.float32) * 4)
    W1 = f(rng.standard_normal((V, 256), dtype=np.float32) * 0.02)
    W2 = f(rng.standard_normal((256, V), dtype=np.float32) * 0.02)
    A = rng.integers(0, V, R).astype(np.int32)
    X = rng.integers(0, V, (R, gamma)).astype(np.int32)
    c = rng.random((R, gamma), dtype=np.float32)
    c.reshape(-1)[0] = 0.0
    c.reshape(-1)[-1] = 1.0

    def run(arrs):
        U_, T_, W1_, W2_, A_, X_, c_ = arrs
        d = [_to_dev_offset(U_, dev, dt, offset), _to_dev_offset(T_, dev, dt, offset),
             _to_dev_offset(W1_, dev, dt, offset), _to_dev_offset(W2_, dev, dt, offset),
             _to_dev_offset(A_, dev, torch.int32, offset), _to_dev_offset(X_, dev, torch.int32, offset),
             _to_dev_offset(c_, dev, torch.float32, offset)]
        got = dspark.check_inputs(R, gamma, V, dt, *d)
        torch.cuda.synchronize()
        return got

    clean = (U, T, W1, W2, A, X, c)
    got = run(clean)
    assert got == {k: 0 for k in dspark.CHECK_FIELDS}, got

    plant = _plant_bf16 if bf16 else _plant_f32
    n = U.size
    plant(rng, U, min(5, n), min(3, max(n - 5, 0)), min(4, max(n - 8, 0)))
    plant(rng, T, 2, 1, 3)
    plant(rng, W1, 1, 1, 1)
    plant(rng, W2, 2, 0, 1)
    A[0] = -1
    A[-1] = V
    X.reshape(-1)[0] = V + 5
    X.reshape(-1)[-1] = -7
    c.reshape(-1)[0] = 1.5
    c.reshape(-1)[-1] = np.nan
    if c.size > 2:
        c.reshape(-1)[1] = -0.25
        c.reshape(-1)[2] = -0.0  # allowed
    bad = (U, T, W1, W2, A, X, c)
    ref = _reference(bad, bf16, V)
    assert ref["U"] > 0 and ref["W"] > 0 and ref["anchors"] > 0
    got = run(bad)
    assert got == ref, (got, ref)

    # tensors left out are not counted
    d = dspark.check_inputs(R, gamma, V, dt, U=None, T=_to_dev_offset(T, dev, dt, offset))
    torch.cuda.synchronize()
    assert d == {**{k: 0 for k in dspark.CHECK_FIELDS}, "T": ref["T"]}
