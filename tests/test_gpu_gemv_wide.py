"""Decode GEMV on a 70B-class weight stream with 5-16 tokens: the launch
streams 235M weights.  The gate/up shape stages m_tok x 8192 activation
bytes (up to 128 KB) in LDS with LDS-direct loads; the down shape's token
rows (28672 wide: up to 458 KB) do not fit, and every wave reads its k-blocks
of them from memory.

The packed weights are random valid codes written straight in the packed
formats (this test is about the product alone); the oracle unpacks every
row from the panel-major storage, in row blocks on a thread pool, and
contracts them exactly: every int32 acc must match bit for bit (y within the
usual 1e-6 relative)."""

import numpy as np
import pytest

from gpu_util import FMT_DENSE2, FMT_NM, check_y, par_map, say, to_dev, to_np
from oracle import sbl_oracle as O

pytestmark = pytest.mark.gpu



def _random_fields(rng, nbytes):
    """Bytes of four 2-bit fields, each a valid u in {0, 1, 2}."""
    u = rng.integers(0, 3, (nbytes, 4), dtype=np.uint8)
    return (u[:, 0] | (u[:, 1] << 2) | (u[:, 2] << 4) | (u[:, 3] << 6)).astype(np.uint8)


def _random_bitmap(rng, nbytes):
    """Bitmap bytes with exactly 6 of 8 bits set (6:8)."""
    pats = np.array([b for b in range(256) if bin(b).count("1") == 6], np.uint8)
    return pats[rng.integers(0, len(pats), nbytes)]


@pytest.mark.parametrize("N_OUT,K,m_tok", [(28672, 8192, 16), (28672, 8192, 9),
                                            (8192, 28672, 16), (8192, 28672, 9), (8192, 28672, 5)])
@pytest.mark.parametrize("fmt", [FMT_DENSE2, FMT_NM])
def test_wide_gemv_every_row(fmt, N_OUT, K, m_tok):
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    rng = np.random.default_rng([41, fmt, m_tok, K])
    n, m = 6, 8
    if fmt == FMT_DENSE2:
        packed = _random_fields(rng, N_OUT * K // 4)
        meta = None
    else:
        packed = _random_fields(rng, N_OUT * K * 6 // 32)
        meta = _random_bitmap(rng, N_OUT * K // 8)
    q = rng.integers(-127, 128, (m_tok, K), dtype=np.int8)
    gamma = rng.uniform(0.5, 4.0, m_tok).astype(np.float32)
    beta = np.float32(0.0137)
    say(f"wide GEMV {N_OUT}x{K} fmt={fmt} m_tok={m_tok}")
    y, acc = sbl.linear(to_dev(packed), to_dev(meta) if meta is not None else None, fmt, n, m,
                        torch.tensor([beta], device="cuda"), to_dev(q), to_dev(gamma), N_OUT, want_acc=True)
    torch.cuda.synchronize()
    acc, y = to_np(acc), to_np(y)

    def block(r0):
        rows = np.arange(r0, min(r0 + 1024, N_OUT))
        if fmt == FMT_DENSE2:
            codes = O.unpack_dense2(O.from_panels(packed, N_OUT, K // 4, 16, rows=rows), K)
        else:
            codes = O.unpack_nm(O.from_panels(packed, N_OUT, K * 6 // 32, 12, rows=rows),
                                O.from_panels(meta, N_OUT, K // 8, 8, rows=rows), n, m, K)
        return O.contract(codes, q)                      # [m_tok][len(rows)]

    acc_ref = np.concatenate(par_map(block, range(0, N_OUT, 1024)), axis=1)
    assert np.array_equal(acc, acc_ref)
    check_y(y, O.rescale(acc_ref, beta, gamma), acc_ref)
