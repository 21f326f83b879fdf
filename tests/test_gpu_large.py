"""Launch slicing at sizes whose grid exceeds one launch: per-token quant of
more than 2^24 short rows, the int8 repack of a weight with more than 2^30
16-byte units, and the online weight quant of more than 2^26 channels. Each
is launched in slices (a launch's workgroups times threads must fit in 32
bits); rows and fragments on both sides of every slice boundary, the first
and the last, and a random sample, are checked against the oracle or the
layout definition.

Inputs are seeded and drawn on the device (torch's generator with a fixed
seed); the rows under test are copied back, so the oracle sees exactly the
values the kernels saw.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from tests.test_gpu_parity import packed_reference

pytestmark = pytest.mark.gpu

DEV = "cuda"
SLICE_BLOCKS = 1 << 22          # workgroups per launch of the sliced launchers


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w8a8_int8_dynamic_amd import ops as _ops
    from w8a8_int8_dynamic_amd import _lib
    assert _ops.device_supported(torch.cuda.current_device()), _lib.last_error()
    return _ops


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def _sample(total: int, edges, rng, n_random: int = 256, width: int = 48) -> np.ndarray:
    idx = set(range(min(width, total)))
    idx.update(range(max(0, total - width), total))
    for e in edges:
        idx.update(range(max(0, e - width), min(total, e + width)))
    idx.update(rng.integers(0, total, n_random).tolist())
    return np.array(sorted(idx), np.int64)


def test_quant_per_token_row_slices(ops, orc):
    """K = 16 bf16 rows take 4 rows per workgroup, so a slice is 2^24 rows;
    M crosses one slice boundary with a ragged remainder."""
    K = 16
    step = SLICE_BLOCKS * 4
    M = step + 4099
    x = (torch.randn((M, K), generator=_gen(7100), device=DEV) *
         torch.exp(torch.randn((M, 1), generator=_gen(7101), device=DEV))).to(torch.bfloat16)
    xq, xs = ops.quant_per_token(x)
    torch.cuda.synchronize()
    rows = _sample(M, [step], np.random.default_rng(7102))
    idx = torch.from_numpy(rows).to(DEV)
    x_rows = x.index_select(0, idx).view(torch.int16).cpu().numpy().view(np.uint16)
    q_ref, s_ref = orc.quant_per_token(x_rows)
    assert np.array_equal(xs.index_select(0, idx).cpu().numpy(), s_ref)
    assert np.array_equal(xq.index_select(0, idx).cpu().numpy(), q_ref)
    del x, xq, xs
    torch.cuda.empty_cache()


def test_prepack_unit_slices(ops):
    """N = 2^20 + 48 channels at K = 16384 is 2^30 + 49,152 16-byte units: the
    repack and its inverse run as two launches each. Fragment rows at the
    boundary (fragment row 2^16) and at both ends match the layout
    definition; the unpacked weight equals the original everywhere."""
    N, K = (1 << 20) + 48, 16384
    kblocks = K // 64
    frag_bytes = kblocks * 1024
    wq = torch.randint(-128, 128, (N, K), generator=_gen(7200), device=DEV, dtype=torch.int8)
    packed = ops.prepack_weight(wq)
    torch.cuda.synchronize()
    boundary_nb = (SLICE_BLOCKS * 256 // 64) // kblocks
    assert boundary_nb == 1 << 16
    nblocks = -(-N // 16)
    for nb in [0, boundary_nb - 1, boundary_nb, boundary_nb + 1, nblocks - 1]:
        rows = wq[nb * 16:(nb + 1) * 16].cpu().numpy()
        got = packed[nb * frag_bytes:(nb + 1) * frag_bytes].cpu().numpy()
        assert np.array_equal(got, packed_reference(rows)), nb
    back = ops.unpack_weight(packed, N, K)
    assert torch.equal(back, wq)
    del wq, packed, back
    torch.cuda.empty_cache()


def test_quant_prepack_fragment_row_slices(ops, orc):
    """N = 2^26 + 37 fp32 channels at K = 16: 2^22 + 3 fragment rows, one
    workgroup each, so two launches. Scales and packed bytes of fragment rows
    on both sides of the boundary, the first and the last (5 channels) match
    the oracle's per-channel codes in the layout."""
    N, K = (1 << 26) + 37, 16
    frag_bytes = 1024                                     # one k-block
    w = torch.randn((N, K), generator=_gen(7300), device=DEV) * 0.02
    packed, ws = ops.quant_prepack_weight(w)
    torch.cuda.synchronize()
    nblocks = -(-N // 16)
    for nb in [0, SLICE_BLOCKS - 1, SLICE_BLOCKS, SLICE_BLOCKS + 1, nblocks - 1]:
        lo, hi = nb * 16, min(N, (nb + 1) * 16)
        w_rows = w[lo:hi].cpu().numpy()
        wq_ref, ws_ref = orc.quant_per_channel(w_rows)
        assert np.array_equal(ws[lo:hi].cpu().numpy(), ws_ref), nb
        got = packed[nb * frag_bytes:(nb + 1) * frag_bytes].cpu().numpy()
        assert np.array_equal(got, packed_reference(wq_ref)), nb
    del w, packed, ws
    torch.cuda.empty_cache()
