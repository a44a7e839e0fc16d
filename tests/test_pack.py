"""mxgemm_pack_b and mxgemm_pack_scales on the GPU against the byte permutations the asm_f4gemm
README prints ("Data layouts": the 16x16 tile-transposed B shuffle and the
scale shuffle), written here with numpy reshapes exactly as stated there,
on padded inputs (N to 16 / 32 rows, K to 128 elements / 8 scale blocks;
pad bytes 0 for B and 0x7F for scales)."""
import numpy as np
import pytest

import block_scaled_precision_mxfp4_amd as mx
from block_scaled_precision_mxfp4_amd import inputs

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
from mxgpu import dev_u8  # noqa: E402


def cdiv(a, b):
    return -(-a // b)


def page_b_shuffle(B, N, K):
    Np, Kp = cdiv(N, 16) * 16, cdiv(K, 128) * 64  # rows, bytes per row
    pad = np.zeros((Np, Kp), dtype=np.uint8)
    pad[:N, : K // 2] = B[:, : K // 2]
    # src.view(N/16, 16, Kp/32, 2, 16).permute(0, 2, 3, 1, 4)
    return pad.reshape(Np // 16, 16, Kp // 32, 2, 16).transpose(0, 2, 3, 1, 4).reshape(-1)


def page_scale_shuffle(S, rows, KB):
    sm, sn = cdiv(rows, 32) * 32, cdiv(KB, 8) * 8
    pad = np.full((sm, sn), 0x7F, dtype=np.uint8)
    pad[:rows, :KB] = S[:, :KB]
    # padded.view(sm/32, 2, 16, sn/8, 2, 4).permute(0, 3, 5, 2, 4, 1)
    return pad.reshape(sm // 32, 2, 16, sn // 8, 2, 4).transpose(0, 3, 5, 2, 4, 1).reshape(-1)


@pytest.mark.parametrize("N,K", [(16, 128), (32, 256), (17, 96), (100, 1056), (8192, 8192), (33, 32)])
def test_pack_matches_page_formula(N, K):
    p = inputs.make_problem(1, N, K, seed=0x9AC + N)
    info = mx.mxgemm_plan(1, N, K, 1, -1, 256)
    Bp = torch.full((info["packed_b_bytes"],), 0xEE, dtype=torch.uint8, device="cuda")
    SBp = torch.full((info["packed_sb_bytes"],), 0xEE, dtype=torch.uint8, device="cuda")
    mx.mxgemm_pack_b(Bp, SBp, dev_u8(p["B"]), dev_u8(p["SB"]), N, K)
    torch.cuda.synchronize()
    assert np.array_equal(Bp.cpu().numpy(), page_b_shuffle(p["B"], N, K))
    assert np.array_equal(SBp.cpu().numpy(), page_scale_shuffle(p["SB"], N, K // 32))


def test_pack_honours_row_strides():
    N, K = 40, 512
    p = inputs.make_problem(1, N, K, seed=0x9AD)
    ldb, ldsb = K + 64, K // 32 + 7
    Bs = np.zeros((N, ldb // 2), dtype=np.uint8)
    Bs[:, : K // 2] = p["B"]
    Ss = np.full((N, ldsb), 0xFF, dtype=np.uint8)
    Ss[:, : K // 32] = p["SB"]
    info = mx.mxgemm_plan(1, N, K, 1, -1, 256)
    Bp = torch.empty((info["packed_b_bytes"],), dtype=torch.uint8, device="cuda")
    SBp = torch.empty((info["packed_sb_bytes"],), dtype=torch.uint8, device="cuda")
    mx.mxgemm_pack_b(Bp, SBp, dev_u8(Bs), dev_u8(Ss), N, K, ldb=ldb, ldsb=ldsb)
    torch.cuda.synchronize()
    assert np.array_equal(Bp.cpu().numpy(), page_b_shuffle(p["B"], N, K))
    assert np.array_equal(SBp.cpu().numpy(), page_scale_shuffle(p["SB"], N, K // 32))


@pytest.mark.parametrize("rows,K,lds_extra", [(1, 32, 0), (64, 4096, 0), (257, 1056, 5), (8192, 8192, 0)])
def test_pack_scales_matches_page_formula(rows, K, lds_extra):
    """mxgemm_pack_scales (A scales for sa_packed = 1) is the same scale
    shuffle, for any row count and row pitch."""
    p = inputs.make_problem(rows, 1, K, seed=0x9AE + rows)
    lds = K // 32 + lds_extra
    Ss = np.full((rows, lds), 0xFF, dtype=np.uint8)
    Ss[:, : K // 32] = p["SA"]
    info = mx.mxgemm_plan(rows, 1, K, 1, -1, 256)
    SAp = torch.full((info["packed_sa_bytes"],), 0xEE, dtype=torch.uint8, device="cuda")
    mx.mxgemm_pack_scales(SAp, dev_u8(Ss), rows, K, lds=lds)
    torch.cuda.synchronize()
    assert np.array_equal(SAp.cpu().numpy(), page_scale_shuffle(p["SA"], rows, K // 32))
