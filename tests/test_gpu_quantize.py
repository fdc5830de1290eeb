"""GPU parity of the per-row symmetric quantiser (moe_quantize_rows, the step
before the path) against the CPU oracle: codes and scales bit-exact.

Inputs are seeded and synthetic: rows N(0, s^2) with a per-row s, all-zero
rows, and rows of exact half-way points (ties), in f32 and bf16.  The
full-size case is the GLM-class layer's routed gate and up weights in bf16
(256 experts x 2 x 2048 rows of 6144), generated on the device by torch's
seeded generator; sampled rows are compared with the oracle and every row's
scale and code range are checked.
"""
import numpy as np
import pytest

import int4_routed_expert_02_amd as moe
import oracle
from gpu_util import say

pytestmark = pytest.mark.gpu

QMAX = {4: 7, 8: 127}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load()


def host_rows(seed, rows, cols, bits):
    rng = np.random.default_rng(seed)
    src = (rng.standard_normal((rows, cols)) * rng.uniform(0.005, 2.0, (rows, 1))).astype(np.float32)
    src[::17] = 0.0
    # exact half-way points with a power-of-two scale: ties must go to even
    qm = QMAX[bits]
    ties = np.resize(np.concatenate([[qm], np.arange(-qm, qm) + 0.5]), cols) * 0.25
    ties[0] = qm * 0.25
    src[3] = ties.astype(np.float32)
    return src


def to_bf16_bits(a):
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def gpu_quantize(src_np, bits):
    import torch
    if src_np.dtype == np.uint16:
        t = torch.from_numpy(src_np.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        t = torch.from_numpy(src_np).cuda()
    q, qs = moe.moe_quantize_rows(t, bits)
    torch.cuda.synchronize()
    return q.cpu().numpy(), qs.cpu().numpy()


def same(tag, got, want):
    (gq, gs), (wq, ws) = got, want
    nq = int(np.sum(gq.view(np.uint8) != wq.view(np.uint8)))
    ns = int(np.sum(gs.view(np.uint32) != ws.view(np.uint32)))
    say(f"{tag}: {gq.shape[0]} rows, {nq} code bytes and {ns} scales differ")
    assert nq == 0 and ns == 0


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("fmt", ["f32", "bf16"])
@pytest.mark.parametrize("rows,cols", [(257, 1024), (40, 6144), (9, 8)])
def test_quantize_matches_oracle(bits, fmt, rows, cols):
    src = host_rows(100 + rows + cols + bits, rows, cols, bits)
    if fmt == "bf16":
        src = to_bf16_bits(src)
    same(f"{fmt} int{bits} {rows}x{cols}", gpu_quantize(src, bits), oracle.quantize_rows(src, bits))


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("fmt", ["f32", "bf16"])
@pytest.mark.parametrize("cols", [1024, 130])
def test_quantize_tiny_rows(bits, fmt, cols):
    """Rows whose scale max|w| / qmax is subnormal (max|w| around 1e-38 for
    int4, 1e-37 for int8, and smaller still, down to a row of denormals), where
    1 / scale overflows or loses precision: codes and scales still equal the
    oracle's plain f32 division, zeros stay 0."""
    rng = np.random.default_rng(31 + bits + cols)
    rows = 24
    amax = np.float32(1e-38 if bits == 4 else 1e-37) * np.logspace(0, -4, rows).astype(np.float32)
    src = (rng.uniform(-1.0, 1.0, (rows, cols)) * amax[:, None]).astype(np.float32)
    src[:, 0] = amax                # the row maximum itself
    src[:, 1] = amax / 2            # a half of it
    src[:, 2] = 0.0                 # zeros must stay 0
    src[:, 3] = -amax
    src[-1] = 0.0
    src[-1, 5] = np.float32(1e-40)   # a row of denormals
    src[-1, 6] = np.float32(-3e-41)
    if fmt == "bf16":
        src = to_bf16_bits(src)
    got = gpu_quantize(src, bits)
    want = oracle.quantize_rows(src, bits)
    same(f"tiny {fmt} int{bits} {rows}x{cols}", got, want)
    assert np.all(want[1] < np.float32(2.0 ** -126))


@pytest.mark.parametrize("bits,cols", [(4, 130), (8, 131), (4, 2), (8, 1)])
def test_quantize_ragged_widths(bits, cols):
    src = host_rows(7 + cols, 33, cols, bits)
    same(f"ragged int{bits} 33x{cols}", gpu_quantize(src, bits), oracle.quantize_rows(src, bits))


@pytest.mark.parametrize("bits", [4, 8])
def test_quantize_unaligned_source(bits):
    # a source starting 4 bytes past a 16-byte boundary takes the value-by-value path
    import torch
    rows, cols = 21, 64
    src = host_rows(55, rows, cols, bits)
    flat = torch.zeros(rows * cols + 4, dtype=torch.float32, device="cuda")
    flat[1:1 + rows * cols] = torch.from_numpy(src.reshape(-1)).cuda()
    q = torch.empty((rows, cols // 2) if bits == 4 else (rows, cols), dtype=torch.uint8, device="cuda")
    qs = torch.empty(rows, dtype=torch.float32, device="cuda")
    st = moe.load().moe_quantize_rows(flat.data_ptr() + 4, moe.MOE_SRC_F32, rows, cols, bits, q.data_ptr(),
                                      qs.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == moe.MOE_OK
    torch.cuda.synchronize()
    wq, ws = oracle.quantize_rows(src, bits)
    same(f"unaligned int{bits}", (q.cpu().numpy(), qs.cpu().numpy()), (wq.view(np.uint8), ws))


def glm_gateup_bf16(seed=1300):
    """The GLM-class layer's routed gate and up weights in bf16: 256 experts x
    2 x 2048 rows of 6144, N(0, s^2) with s ~ U(0.005, 0.05) per row."""
    import torch
    rows, cols = 256 * 2 * 2048, 6144
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    src = torch.empty(rows, cols, dtype=torch.bfloat16, device="cuda")
    step = 65536
    for r0 in range(0, rows, step):
        s = torch.empty(step, 1, device="cuda").uniform_(0.005, 0.05, generator=g)
        src[r0:r0 + step] = (torch.randn(step, cols, device="cuda", generator=g) * s).to(torch.bfloat16)
    return src


def test_quantize_full_size_glm_gateup():
    import torch
    src = glm_gateup_bf16()
    rows, cols = src.shape
    q, qs = moe.moe_quantize_rows(src, 4)
    torch.cuda.synchronize()
    # every row's scale: max|w| (exact on any device) over 7, one f32 division on the host
    amax = torch.cat([src[r:r + 65536].float().abs().amax(dim=1) for r in range(0, rows, 65536)]).cpu().numpy()
    want_s = amax.astype(np.float32) / np.float32(7.0)
    bad_s = int(np.sum(qs.cpu().numpy().view(np.uint32) != want_s.view(np.uint32)))
    # every row's codes lie in [-7, 7] and reach +-7
    lo_bad, top_bad = 0, 0
    for r in range(0, rows, 65536):
        b = q[r:r + 65536].to(torch.int16)
        nib = torch.cat([b & 15, b >> 4], dim=1)
        val = torch.where(nib >= 8, nib - 16, nib)
        lo_bad += int((val < -7).sum())
        top_bad += int((val.abs().amax(dim=1) != 7).sum())
    # sampled rows against the oracle, code bytes and scale bits
    pick = np.random.default_rng(3).choice(rows, 48, replace=False)
    idx = torch.from_numpy(pick).cuda()
    src_rows = src[idx].view(torch.int16).cpu().numpy().view(np.uint16)
    wq, ws = oracle.quantize_rows(src_rows, 4)
    say(f"GLM gate/up family {rows}x{cols} bf16: {bad_s} scales off, {lo_bad} codes below -7, "
        f"{top_bad} rows not reaching +-7")
    assert bad_s == 0 and lo_bad == 0 and top_bad == 0
    same("GLM gate/up sampled rows", (q[idx].cpu().numpy(), qs[idx].cpu().numpy()), (wq, ws))
