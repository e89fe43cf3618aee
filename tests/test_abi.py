"""CPU checks of the C ABI: the library loads, exports every symbol the header
declares, sizes its buffers correctly and rejects bad arguments on the host
(before any HIP call) with the documented status codes."""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sbl.h")
LIB = os.path.join(ROOT, "sparse_linear_layers_absmean_amd", "libsbl.so")

# Validation calls below pass fake (never dereferenced) device addresses.  They
# must be rejected on the host; as a belt-and-braces guard they are not run
# on a machine that has a GPU, where a validation bug could reach a kernel.
HAS_GPU_NODE = os.path.exists("/dev/kfd")


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sbl_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libsbl.so is not built (run __graft_entry__.build())")
    import torch  # noqa: F401  (same HIP runtime as the tests that use the GPU)
    from sparse_linear_layers_absmean_amd import sbl
    return sbl.load()


def test_header_declares_the_four_calls():
    fns = _header_functions()
    for f in ["sbl_quant_weights", "sbl_pack", "sbl_quant_acts", "sbl_linear"]:
        assert f in fns


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (sbl_[a-z0-9_]+)", out))
    for f in _header_functions():
        assert f in exported, f
        assert hasattr(lib, f)


def test_abi_version_and_strings(lib):
    assert lib.sbl_abi_version() == 11
    for st in range(7):
        assert len(lib.sbl_status_string(st)) > 0
    assert lib.sbl_last_hip_error() == 0


@pytest.mark.parametrize("n_out,k", [(1, 64), (256, 256), (1536, 4096), (8640, 3200), (3, 131072)])
def test_packed_and_meta_bytes(lib, n_out, k):
    assert lib.sbl_packed_bytes(n_out, k, 6, 8, 0) == n_out * k // 4
    assert lib.sbl_packed_bytes(n_out, k, 6, 8, 1) == n_out * k * 6 // 32
    assert lib.sbl_packed_bytes(n_out, k, 2, 4, 1) == n_out * k * 2 // 16
    assert lib.sbl_packed_bytes(n_out, k, 5, 8, 1) == n_out * k * 5 // 32
    assert lib.sbl_meta_bytes(n_out, k, 0) == 0
    assert lib.sbl_meta_bytes(n_out, k, 1) == n_out * k // 8
    ws = lib.sbl_workspace_bytes(n_out, k)
    assert ws % 4096 == 0 and 4096 <= ws <= 57344


def test_packed_bytes_closed_form_bits_per_weight(lib):
    # DENSE2 holds 2 bits/weight; N:M 6:8 holds 2.5 (codes 1.5 + bitmap 1); 2:4 holds 2 (1 + 1)
    n_out, k = 1024, 4096
    w = n_out * k
    assert lib.sbl_packed_bytes(n_out, k, 6, 8, 0) * 8 == 2 * w
    assert (lib.sbl_packed_bytes(n_out, k, 6, 8, 1) + lib.sbl_meta_bytes(n_out, k, 1)) * 8 == 2.5 * w
    assert (lib.sbl_packed_bytes(n_out, k, 2, 4, 1) + lib.sbl_meta_bytes(n_out, k, 1)) * 8 == 2 * w


@pytest.mark.parametrize("args", [(0, 64, 6, 8, 0), (4, 0, 6, 8, 0), (4, 96, 6, 8, 0),
                                  (4, 262144, 6, 8, 0), (4, 64, 0, 8, 1), (4, 64, 9, 8, 1),
                                  (4, 64, 2, 3, 1), (4, 64, 6, 8, 7)])
def test_packed_bytes_rejects(lib, args):
    assert lib.sbl_packed_bytes(*args) == -1


A = 1 << 20          # a 16-byte aligned fake address (never dereferenced)
S = ctypes.c_void_p


@pytest.mark.skipif(HAS_GPU_NODE, reason="fake-pointer validation runs only on GPU-less hosts")
def test_quant_weights_validation(lib):
    f = lib.sbl_quant_weights
    ws = lib.sbl_workspace_bytes(4, 64)
    MK, CD, PK, MT = A + (1 << 16), A + (2 << 16), A + (3 << 16), A + (4 << 16)   # disjoint outputs
    ok = dict(w=A, n_out=4, k=64, n=6, m=8, beta=A, mask=MK, codes=CD, fmt=0, packed=PK, meta=MT,
              ws=A, wsb=ws, s=None)

    def call(**kw):
        a = {**ok, **kw}
        return f(a["w"], a["n_out"], a["k"], a["n"], a["m"], a["beta"], a["mask"], a["codes"],
                 a["fmt"], a["packed"], a["meta"], a["ws"], a["wsb"], a["s"])

    assert call(w=None) == 1
    assert call(beta=None) == 1
    assert call(fmt=1, meta=None) == 1
    assert call(ws=None) == 6
    assert call(wsb=ws - 1) == 6
    assert call(n_out=0) == 2
    assert call(k=96) == 2
    assert call(k=0) == 2
    assert call(k=262144) == 2
    assert call(n_out=1 << 30, k=131072) == 2
    assert call(n=7, m=6) == 4
    assert call(n=0) == 4
    assert call(n=9) == 4
    assert call(fmt=3) == 4
    assert call(fmt=1, meta=MK + 16) == 2           # N:M metadata overlapping the mask output
    assert call(packed=MK + 16) == 2                # DENSE2 slots overlapping the mask
    assert call(codes=PK - 64) == 2                 # codes running into the packed stream
    assert call(fmt=1, meta=PK + 16) == 2           # metadata inside the N:M codes
    assert call(w=A + 2) == 3
    assert call(beta=A + 2) == 3
    assert call(packed=PK + 8) == 3
    assert call(mask=MK + 1) == 3
    assert call(codes=CD + 4) == 3
    assert call(ws=A + 8) == 3


def test_workspace_bytes_cover_one_slot_per_workgroup(lib):
    # per absmean workgroup (256 threads x 8 vectors of 8 values each, up to 1024
    # workgroups, then longer threads; 4096 at 2^34 values): an 8-byte sum and a
    # 48-byte record, the sums padded to 64 bytes, the whole rounded up to 4 KB
    assert lib.sbl_workspace_bytes(1, 64) == 4096
    assert lib.sbl_workspace_bytes(256, 4096) == 4096              # 64 slots: 512 + 3072 bytes
    assert lib.sbl_workspace_bytes(16384, 131072) == 57344        # 2^31 values: 1024 slots
    assert lib.sbl_workspace_bytes(131072, 131072) == 229376      # 2^34 values: 4096 slots
    assert lib.sbl_workspace_bytes(0, 64) == -1
    assert lib.sbl_workspace_bytes(4, 96) == -1


@pytest.mark.skipif(HAS_GPU_NODE, reason="fake-pointer validation runs only on GPU-less hosts")
def test_quant_weights_batch_validation(lib):
    from sparse_linear_layers_absmean_amd.sbl import QuantItem
    f = lib.sbl_quant_weights_batch
    ws = lib.sbl_workspace_bytes(4, 64)

    def item(**kw):
        a = dict(w_bf16=A, n_out=4, k=64, beta=A, mask_bits=A, codes=None, packed=A + (2 << 16), meta=A + (1 << 16),
                 workspace=A, workspace_bytes=ws)
        a.update(kw)
        return QuantItem(**a)

    def call(items, count=None, n=6, m=8, fmt=1):
        arr = (QuantItem * len(items))(*items)
        return f(arr, len(items) if count is None else count, n, m, fmt, None)

    assert f(None, 1, 6, 8, 1, None) == 1
    assert call([item()], count=0) == 2
    assert call([item()], count=257) == 2
    assert call([item(), item(w_bf16=None)]) == 1
    assert call([item(), item(meta=None)]) == 1
    assert call([item(), item(k=96)]) == 2
    assert call([item(), item(workspace_bytes=ws - 8)]) == 6
    assert call([item(), item(workspace=A + ws - 16)]) == 6       # overlaps item 0's workspace
    assert call([item()], n=9) == 4
    assert call([item()], fmt=2) == 4
    assert call([item(), item(w_bf16=A + 2, workspace=A + 2 * ws)]) == 3

    # the variant entry point: flags are checked first, then the same item checks
    fx = lib.sbl_quant_weights_batch_ex

    def call_ex(items, flags, n=6, m=8, fmt=1):
        arr = (QuantItem * len(items))(*items)
        return fx(arr, len(items), n, m, fmt, flags, None)

    assert call_ex([item()], 16) == 4                              # unknown bit
    assert call_ex([item()], -1) == 4
    assert call_ex([item()], 3) == 4                               # the two variants exclude each other
    assert call_ex([item()], 3 | 4) == 4
    assert fx(None, 1, 6, 8, 1, 1, None) == 1
    for flags in (0, 1, 2, 4, 8, 12, 5, 10):
        assert call_ex([item()], flags, n=9) == 4
        assert call_ex([item(), item(k=96)], flags) == 2
        assert call_ex([item(), item(workspace=A + ws - 16)], flags) == 6
        assert call_ex([item(), item(w_bf16=A + 2, workspace=A + 2 * ws)], flags) == 3


@pytest.mark.skipif(HAS_GPU_NODE, reason="fake-pointer validation runs only on GPU-less hosts")
def test_pack_validation(lib):
    f = lib.sbl_pack
    assert f(None, A, 4, 64, 6, 8, 1, A, A, None) == 1
    assert f(A, None, 4, 64, 6, 8, 1, A, A, None) == 1
    assert f(A, A, 4, 64, 6, 8, 0, None, None, None) == 1
    assert f(A, A, 4, 80, 6, 8, 0, A, None, None) == 2
    assert f(A, A, 0, 64, 6, 8, 0, A, None, None) == 2
    assert f(A, A, 4, 64, 6, 8, 2, A, None, None) == 4
    assert f(A, A, 4, 64, 5, 4, 1, A, A, None) == 4
    assert f(A + 4, A, 4, 64, 6, 8, 0, A, None, None) == 3


@pytest.mark.skipif(HAS_GPU_NODE, reason="fake-pointer validation runs only on GPU-less hosts")
def test_quant_acts_validation(lib):
    f = lib.sbl_quant_acts
    assert f(A, 0, 64, A, A, None) == 0                 # empty batch: no-op
    assert f(None, 0, 64, None, None, None) == 0
    assert f(A, -1, 64, A, A, None) == 2
    assert f(A, 1, 63, A, A, None) == 2
    assert f(A, 1, 0, A, A, None) == 2
    assert f(A, (1 << 24) + 1, 64, A, A, None) == 2
    assert f(None, 1, 64, A, A, None) == 1
    assert f(A, 1, 64, None, A, None) == 1
    assert f(A, 1, 64, A, None, None) == 1
    assert f(A + 4, 1, 64, A, A, None) == 3
    assert f(A, 1, 64, A + 2, A, None) == 3
    assert f(A, 1, 64, A, A + 1, None) == 3


@pytest.mark.skipif(HAS_GPU_NODE, reason="fake-pointer validation runs only on GPU-less hosts")
def test_linear_validation(lib):
    f = lib.sbl_linear
    base = [A, A, 0, 6, 8, A, A, A, 4, 16, 64, A, A, None]

    def call(i_val):
        a = list(base)
        for i, v in i_val:
            a[i] = v
        return f(*a)

    assert call([(8, 0)]) == 0                       # m_tok = 0: no-op
    assert call([(9, 0)]) == 0                       # n_out = 0: no-op
    assert call([(8, -1)]) == 2
    assert call([(10, 100)]) == 2
    assert call([(10, 0)]) == 2
    assert call([(2, 5)]) == 4
    assert call([(2, 1), (3, 3), (4, 2)]) == 4       # NM with 3:2
    assert call([(0, None)]) == 1
    assert call([(5, None)]) == 1
    assert call([(6, None)]) == 1
    assert call([(7, None)]) == 1
    assert call([(11, None)]) == 1
    assert call([(2, 1), (1, None)]) == 1            # NM needs meta
    assert call([(0, A + 8)]) == 3
    assert call([(6, A + 4)]) == 3
    assert call([(11, A + 2)]) == 3
    assert call([(12, A + 1)]) == 3


@pytest.mark.skipif(HAS_GPU_NODE, reason="fake-pointer validation runs only on GPU-less hosts")
def test_linear_acts_batch_validation(lib):
    from sparse_linear_layers_absmean_amd.sbl import LinearItem
    f = lib.sbl_linear_acts_batch

    def item(**kw):
        a = dict(packed=A, meta=A, beta=A, xq=None, gamma=None, m_tok=4, n_out=16, k=64, y=A, acc=None)
        a.update(kw)
        return LinearItem(**a)

    def call(items, x=A, m_tok=4, k=64, xq=A, gamma=A, count=None, fmt=1, n=6, m=8):
        arr = (LinearItem * len(items))(*items)
        return f(x, m_tok, k, xq, gamma, arr, len(items) if count is None else count, fmt, n, m, None)

    assert f(A, 4, 64, A, A, None, 1, 1, 6, 8, None) == 1
    assert call([item()], count=0) == 2
    assert call([item()], count=257) == 2
    assert call([item()], k=96) == 2
    assert call([item()], m_tok=-1) == 2
    assert call([item(m_tok=3)]) == 2                 # items must share m_tok and k
    assert call([item(), item(k=128)]) == 2
    assert call([item()], x=None) == 1
    assert call([item()], xq=None) == 1
    assert call([item()], gamma=None) == 1
    assert call([item()], x=A + 4) == 3
    assert call([item()], xq=A + 8) == 3
    assert call([item(), item(meta=None)]) == 1       # NM needs meta
    assert call([item(), item(y=A + 2)]) == 3
    assert call([item()], n=9) == 4
    assert call([item()], fmt=2) == 4
    assert call([item(m_tok=0)], m_tok=0, x=None, xq=None, gamma=None) == 0   # no tokens: no-op


@pytest.mark.skipif(HAS_GPU_NODE, reason="fake-pointer validation runs only on GPU-less hosts")
def test_backward_validation(lib):
    f = lib.sbl_linear_backward
    F = 1 << 40                                             # far apart fake buffers

    def call(dy=A, m_tok=4, n_out=16, k=64, packed=A + F, meta=A + 2 * F, fmt=1, n=6, m=8, beta=A + 3 * F,
             x=A + 4 * F, xq=A + 5 * F, gamma=A + 6 * F, dx=A + 7 * F, dw=A + 8 * F):
        return f(dy, m_tok, n_out, k, packed, meta, fmt, n, m, beta, x, xq, gamma, dx, dw, None)

    assert call(dx=None, dw=None) == 0                     # nothing asked: no-op
    assert call(m_tok=0) == 2
    assert call(n_out=12) == 2                             # n_out % 8
    assert call(k=96) == 2
    assert call(dy=None) == 1
    assert call(gamma=None) == 1
    assert call(packed=None) == 1
    assert call(packed=None, dx=None) != 1                 # dw alone needs no weights
    assert call(xq=None) == 1
    assert call(xq=None, dw=None) != 1                     # dx alone needs no codes
    assert call(meta=None) == 1
    assert call(meta=None, fmt=0) != 1                     # DENSE2 needs no metadata
    assert call(fmt=2) == 4
    assert call(n=9) == 4
    assert call(dy=A + 8) == 3
    assert call(xq=A + 5 * F + 4) == 3
    assert call(dw=A + 7 * F + 64) == 2                    # overlaps dx
    assert call(dx=A + 16) == 2                            # overlaps dy
    assert call(dw=A + 5 * F + 16) == 2                    # overlaps xq


def test_backward_workspace_sizes(lib):
    # codes^T (k x n_out rounded up to 64), dy^T (both rounded up to 64), 3 parts of x_hat^T, 256-byte aligned
    def ws(t, no, k):
        np_, mp = -(-no // 64) * 64, -(-t // 64) * 64
        return sum(-(-b // 256) * 256 for b in (2 * k * np_, 2 * np_ * mp, 6 * k * mp))
    for t, no, k in [(4, 16, 64), (2048, 8640, 3200), (300, 520, 448), (1, 8, 64)]:
        assert lib.sbl_backward_workspace_bytes(t, no, k) == ws(t, no, k)
    assert lib.sbl_backward_workspace_bytes(0, 16, 64) == -1
    assert lib.sbl_backward_workspace_bytes(4, 12, 64) == -1
    assert lib.sbl_backward_workspace_bytes(4, 16, 96) == -1


@pytest.mark.skipif(HAS_GPU_NODE, reason="fake-pointer validation runs only on GPU-less hosts")
def test_backward_ws_validation(lib):
    f = lib.sbl_linear_backward_ws
    F = 1 << 40
    wsb = lib.sbl_backward_workspace_bytes(4, 16, 64)

    def call(dy=A, m_tok=4, n_out=16, k=64, packed=A + F, meta=A + 2 * F, fmt=1, n=6, beta=A + 3 * F,
             x=A + 4 * F, xq=A + 5 * F, gamma=A + 6 * F, dx=A + 7 * F, dw=A + 8 * F, ws=A + 9 * F, nb=wsb):
        return f(dy, m_tok, n_out, k, packed, meta, fmt, n, 8, beta, x, xq, gamma, dx, dw, ws, nb, None)

    assert call(dx=None, dw=None) == 0                     # nothing asked: no-op
    assert call(dx=None, dw=None, ws=None) == 0
    assert call(m_tok=0) == 2
    assert call(n_out=12) == 2
    assert call(dy=None) == 1
    assert call(ws=None) == 1
    assert call(ws=A + 9 * F + 16) == 3                    # 256-byte alignment
    assert call(nb=wsb - 1) == 2                           # too small
    assert call(ws=A + 7 * F) == 2                         # overlaps dx
    assert call(ws=A + 5 * F - 256) == 2                   # overlaps xq
    assert call(ws=A + 8 * F + 256, dx=None) == 2          # overlaps dw
    assert call(fmt=2) == 4
    assert call(dw=A + 7 * F + 64) == 2                    # the plain call's checks hold too


def test_grouped_workspace_sizes(lib):
    # per group: its absmean slots (8 bytes, padded to 64) + 48-byte records, rounded up to 4 KB overall
    assert lib.sbl_workspace_bytes_grouped(4, 64, 1) == 4096              # 4 groups x 14 words
    assert lib.sbl_workspace_bytes_grouped(8640, 3200, 1) == 970752       # one slot per row
    assert lib.sbl_workspace_bytes_grouped(5120, 5120, 5120) == 45056     # one group: 800 slots
    assert lib.sbl_workspace_bytes_grouped(5120, 5120, 99999) == 45056    # a group larger than the matrix
    assert lib.sbl_workspace_bytes_grouped(4, 64, 0) == -1
    assert lib.sbl_workspace_bytes_grouped(4, 96, 1) == -1
    assert lib.sbl_workspace_bytes_grouped(65536, 64, 1) == -1          # more groups than grid rows
    assert lib.sbl_workspace_bytes_grouped(65535, 64, 1) > 0


@pytest.mark.skipif(HAS_GPU_NODE, reason="fake-pointer validation runs only on GPU-less hosts")
def test_grouped_validation(lib):
    fq = lib.sbl_quant_weights_grouped
    F = 1 << 40
    ws = lib.sbl_workspace_bytes_grouped(16, 64, 4)

    def q(rpg=4, beta=A + F, packed=A + 2 * F, meta=A + 3 * F, workspace=A + 4 * F, wsb=ws, fmt=1, n=6):
        return fq(A, 16, 64, n, 8, rpg, beta, None, None, fmt, packed, meta, workspace, wsb, None)

    assert q(rpg=0) == 2
    assert q(wsb=ws - 8) == 6
    assert q(workspace=None) == 6
    assert q(beta=None) == 1
    assert q(n=9) == 4
    assert q(beta=A + 2 * F + 8) == 2                       # beta (4 groups) overlaps packed
    assert q(beta=A + 4 * F + 16) == 2                      # beta overlaps the workspace
    fl = lib.sbl_linear_grouped

    def lin(rpg=4, acc=A + 5 * F, y=A + 6 * F, fmt=1):
        return fl(A + 2 * F, A + 3 * F, fmt, 6, 8, A + F, rpg, A + 7 * F, A + 8 * F, 2, 16, 64, y, acc, None)

    assert lin(rpg=0) == 2
    assert lin(acc=A + 6 * F + 4) == 2                      # acc overlaps y
    assert lin(y=A + F + 8) == 2                            # y overlaps beta (4 groups)
    assert lin(acc=A + F + 12) == 2                         # acc overlaps beta
    assert lin(fmt=3) == 4


@pytest.mark.skipif(HAS_GPU_NODE, reason="fake-pointer validation runs only on GPU-less hosts")
def test_blocked_validation(lib):
    F = 1 << 40
    wsb = lib.sbl_workspace_bytes_blocked
    assert wsb(16, 256, 4, 64) > 0
    assert wsb(16, 256, 4, 96) == -1                        # not a multiple of 64
    assert wsb(16, 256, 4, 192) == -1                       # does not divide k
    assert wsb(16, 256, 0, 64) == -1
    assert wsb(16, 256, 4, 256) == lib.sbl_workspace_bytes_grouped(16, 256, 4)
    ws = wsb(16, 256, 4, 64)
    fq = lib.sbl_quant_weights_blocked

    def q(rpg=4, cpg=64, beta=A + F, workspace=A + 4 * F, wsb_=ws):
        return fq(A, 16, 256, 6, 8, rpg, cpg, beta, None, None, 1, A + 2 * F, A + 3 * F, workspace, wsb_, None)

    assert q(cpg=96) == 2
    assert q(rpg=0) == 2
    assert q(wsb_=ws - 8) == 6
    assert q(beta=None) == 1
    assert q(beta=A + 2 * F + 48) == 2                      # beta (4 x 4 blocks) overlaps packed
    fl = lib.sbl_linear_blocked

    def lin(kg=64, y=A + 6 * F, beta=A + F):
        return fl(A + 2 * F, A + 3 * F, 1, 6, 8, beta, 4, A + 7 * F, A + 8 * F, kg, 2, 16, 256, y, None)

    assert lin(kg=96) == 2
    assert lin(y=A + F + 48) == 2                           # y overlaps beta (4 x 4)


@pytest.mark.skipif(HAS_GPU_NODE, reason="fake-pointer validation runs only on GPU-less hosts")
def test_kgrouped_validation(lib):
    F = 1 << 40
    qa = lib.sbl_quant_acts_kgrouped
    assert qa(A, 2, 256, 96, A + F, A + 2 * F, None) == 2          # kg % 64
    assert qa(A, 2, 256, 192, A + F, A + 2 * F, None) == 2         # kg does not divide k
    assert qa(A, 0, 256, 64, None, None, None) == 0                # no tokens: no-op
    assert qa(None, 2, 256, 64, A + F, A + 2 * F, None) == 1
    assert qa(A + 2, 2, 256, 64, A + F, A + 2 * F, None) == 3
    assert qa(A, 2, 256, 64, A + 16, A + 2 * F, None) == 2         # xq overlaps x
    lk = lib.sbl_linear_kgrouped

    def lin(rpg=4, kg=64, y=A + 6 * F, gamma=A + 8 * F, fmt=1):
        return lk(A + 2 * F, A + 3 * F, fmt, 6, 8, A + F, rpg, A + 7 * F, gamma, kg, 2, 16, 256, y, None)

    assert lin(rpg=0) == 2
    assert lin(kg=100) == 2
    assert lin(kg=512) == 2
    assert lin(fmt=3) == 4
    assert lin(y=A + 8 * F + 4) == 2                                # y overlaps gamma


@pytest.mark.skipif(HAS_GPU_NODE, reason="fake-pointer validation runs only on GPU-less hosts")
def test_quant_weights_batch_noalloc_validation(lib):
    """The allocation-free entry point validates items as the batch call does
    (workspace fields ignored) and rejects batches whose exact-beta scratch
    exceeds the library's fixed array, all before any HIP call."""
    from sparse_linear_layers_absmean_amd.sbl import QuantItem
    f = lib.sbl_quant_weights_batch_noalloc
    limit = 4 << 20

    def item(**kw):
        a = dict(w_bf16=A, n_out=4, k=64, beta=A, mask_bits=A, codes=None, packed=A + (2 << 16), meta=A + (1 << 16),
                 workspace=None, workspace_bytes=0)
        a.update(kw)
        return QuantItem(**a)

    def call(items, count=None, n=6, m=8, fmt=1):
        arr = (QuantItem * len(items))(*items)
        return f(arr, len(items) if count is None else count, n, m, fmt, None)

    assert f(None, 1, 6, 8, 1, None) == 1
    assert call([item()], count=0) == 2
    assert call([item()], count=257) == 2
    assert call([item(), item(w_bf16=None)]) == 1
    assert call([item(), item(meta=None)]) == 1
    assert call([item(), item(k=96)]) == 2
    assert call([item()], n=9) == 4
    assert call([item()], fmt=2) == 4
    assert call([item(), item(w_bf16=A + 2)]) == 3
    # scratch: 2^34-weight items need the largest workspace each; too many of them overflow
    big = lib.sbl_workspace_bytes(1 << 17, 1 << 17)
    fits = limit // (-(-big // 256) * 256)
    assert call([item(n_out=1 << 17, k=1 << 17, mask_bits=None, packed=None, meta=None)] * (fits + 1)) == 6
    small = lib.sbl_workspace_bytes(1 << 15, 1 << 16)            # 2^31 weights
    assert limit // small >= 73


def test_peak_probe_library_exports_its_calls():
    # the benchmark's peak probes live in a library of their own (not the path's ABI)
    probe = os.path.join(ROOT, "sparse_linear_layers_absmean_amd", "libsbl_probe.so")
    if not os.path.exists(probe):
        pytest.fail("libsbl_probe.so is not built (run __graft_entry__.build())")
    out = subprocess.run(["nm", "-D", "--defined-only", probe], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (sbl_[a-z0-9_]+)", out))
    assert exported == {"sbl_probe_stream_read", "sbl_probe_mfma_i8", "sbl_probe_clock_khz"}
