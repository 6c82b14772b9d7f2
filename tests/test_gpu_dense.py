"""GPU parity of the small-batch dense NVFP4 GEMV (through the C ABI) against
the fp64 oracle, every output compared.

Shapes: the attention projections of a Flint-shaped model (hidden 2048, 32
query and 4 KV heads of 64: fused QKV [2560, 2048], O [2048, 2048]), and
ragged ones that exercise several rows per wave step, padded rows and the
smallest matrix.  Inputs are seeded: every e2m1 code (both zeros included),
e4m3 block scales in [0.5, 2], tensor scale 0.37, x ~ N(0, 1) in bf16.

Bar, from the arithmetic: the kernel sums exact products in fp32 (error
~K * 2^-24 relative to sum |w x|) and rounds once to bf16 (at most half an
ulp, 2^-9 relative); so |y - ref| <= 2^-8 |ref| + 2^-16 * sum_k |W x|.
"""

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _note(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_expert_gemv_amd import binding  # noqa: F401  (raises if the library is not built)
    yield
    torch.cuda.synchronize()


def _bf16_bits(x):
    f = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((f + 0x7FFF + ((f >> 16) & 1)) >> 16).astype(np.uint16)


def _case(rows, cols, batch, seed):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(0x30, 0x41, size=(rows, cols // 16), dtype=np.uint8)   # e4m3 0.5 .. 2.0
    x_bits = _bf16_bits(rng.standard_normal((batch, cols)))
    return codes, scales, x_bits


def _run(codes, scales, ts, x_bits):
    from quantized_expert_gemv_amd import binding as B
    rows, cols = codes.shape[0], 2 * codes.shape[1]
    batch = x_bits.shape[0]
    cr, sr = B.moe_pack_dense(codes, scales, ts)
    dev = torch.device("cuda")
    cr_d = torch.from_numpy(cr).to(dev)
    sr_d = torch.from_numpy(sr).to(dev)
    x = torch.from_numpy(x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    y = torch.full((batch, rows), float("nan"), dtype=torch.bfloat16, device=dev)
    B.moe_dense_gemv(rows, cols, cr_d, sr_d, x, y, batch)
    torch.cuda.synchronize()
    return y.float().cpu().numpy()


def _check(name, rows, cols, batch, seed):
    import oracle
    codes, scales, x_bits = _case(rows, cols, batch, seed)
    ts = 0.37
    _note(f"[dense] {name}: rows={rows} cols={cols} batch={batch}")
    y = _run(codes, scales, ts, x_bits)
    ref = oracle.dense_gemv(codes, scales, ts, x_bits)
    w_abs = np.abs(oracle.dequant_nvfp4(codes, scales, ts))
    mag = np.abs(oracle.bf16_bits_to_f64(x_bits)) @ w_abs.T
    err = np.abs(y - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -16 * mag
    worst = float(np.max(err - bound))
    _note(f"[dense] {name}: max|err|={err.max():.3e} max|ref|={np.abs(ref).max():.3e} worst margin={worst:.3e}")
    assert np.all(np.isfinite(y))
    assert np.all(err <= bound)


@pytest.mark.parametrize("batch", [1, 8])
def test_dense_qkv_projection(batch):
    _check("qkv", 2560, 2048, batch, 10 + batch)


@pytest.mark.parametrize("batch", [2, 4])
def test_dense_o_projection(batch):
    _check("o", 2048, 2048, batch, 20 + batch)


@pytest.mark.parametrize("rows,cols,batch", [(1, 32, 1), (7, 96, 3), (100, 96, 5), (333, 512, 8),
                                             (4097, 1024, 2), (64, 2048, 7)])
def test_dense_ragged_shapes(rows, cols, batch):
    _check("ragged", rows, cols, batch, rows + cols + batch)


def test_dense_writes_only_its_rows_and_repeats_bitwise():
    from quantized_expert_gemv_amd import binding as B
    rows, cols, batch = 100, 96, 3
    codes, scales, x_bits = _case(rows, cols, batch, 5)
    cr, sr = B.moe_pack_dense(codes, scales, 1.0)
    dev = torch.device("cuda")
    cr_d, sr_d = torch.from_numpy(cr).to(dev), torch.from_numpy(sr).to(dev)
    x = torch.from_numpy(x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    # y inside a larger buffer: the words after batch * rows must stay untouched
    buf = torch.full((batch * rows + 64,), 7.0, dtype=torch.bfloat16, device=dev)
    B.moe_dense_gemv(rows, cols, cr_d, sr_d, x, buf, batch)
    first = buf.clone()
    B.moe_dense_gemv(rows, cols, cr_d, sr_d, x, buf, batch)
    torch.cuda.synchronize()
    assert torch.all(buf[batch * rows:] == 7.0)
    assert torch.equal(first.view(torch.int16), buf.view(torch.int16))
