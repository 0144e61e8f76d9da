"""ffnq_pack: the tiled layouts, byte for byte.

The expected bytes are built here in numpy straight from the layout that
include/ffnq.h specifies for FFNQ_FMT_INT8_ROW_TILED and
FFNQ_FMT_INT4_AFFINE_G64_TILED (16-row tiles of 1 KB steps; in a code step
the 16 bytes of row r and lane group g hold the inputs 32d + 8g .. +7 of MFMA
step d; INT4 groups of 8 code blocks, each preceded by its scale/zero step;
INT8 row scales after the tiles).  Pure rearrangement, so the comparison is
exact."""
import numpy as np
import pytest
import torch

import gen
import moe_expert_dequant_amd as fq

pytestmark = pytest.mark.gpu


def ref_pack(mat: dict, n_experts: int) -> np.ndarray:
    fmt, n, k = mat["fmt"], mat["n"], mat["k"]
    T = (n + 15) // 16
    q = np.asarray(mat["q"]).reshape(n_experts, n, -1).view(np.uint8)
    out = []
    for e in range(n_experts):
        qe = np.zeros((T * 16, q.shape[2]), dtype=np.uint8)
        qe[:n] = q[e]
        if fmt == gen.FMT_INT4_AFFINE_G64:
            nbk, gs = k // 128, k // 64
            ng = (nbk + 7) // 8
            s = np.zeros((T * 16, gs), dtype=np.uint16)
            z = np.zeros((T * 16, gs), dtype=np.uint16)
            s[:n] = np.asarray(mat["s"]).reshape(n_experts, n, gs)[e]
            z[:n] = np.asarray(mat["z"]).reshape(n_experts, n, gs)[e]
            tiles = []
            for t in range(T):
                rows = slice(16 * t, 16 * t + 16)
                steps = []
                for j in range(ng):
                    sz = np.zeros((8, 16, 4), dtype=np.uint16)     # block, row, (s0 s1 z0 z1)
                    for bi in range(8):
                        b = 8 * j + bi
                        if b < nbk:
                            sz[bi, :, 0:2] = s[rows, 2 * b:2 * b + 2]
                            sz[bi, :, 2:4] = z[rows, 2 * b:2 * b + 2]
                    steps.append(sz.view(np.uint8).reshape(-1))
                    for bi in range(min(8, nbk - 8 * j)):
                        b = 8 * j + bi
                        # codes of the block's 128 inputs, row-major nibbles: even input low
                        by = qe[rows, 64 * b:64 * b + 64].astype(np.uint32)            # [16][64]
                        codes = np.stack([by & 0xF, by >> 4], axis=-1).reshape(16, 128)
                        words = np.zeros((4, 16, 4), dtype=np.uint32)               # g, row, d
                        for g in range(4):
                            for d in range(4):
                                c8 = codes[:, 32 * d + 8 * g:32 * d + 8 * g + 8]     # [16][8]
                                wv = np.zeros(16, dtype=np.uint32)
                                for v in range(4):
                                    wv |= c8[:, 2 * v] << (4 * v)
                                    wv |= c8[:, 2 * v + 1] << (16 + 4 * v)
                                words[g, :, d] = wv
                        steps.append(words.reshape(-1).view(np.uint8))               # lane = 16 g + row
                tiles.append(np.concatenate(steps))
            out.append(np.concatenate(tiles))
        else:
            nbk = k // 64
            tiles = []
            for t in range(T):
                rows = slice(16 * t, 16 * t + 16)
                for b in range(nbk):
                    blk = qe[rows, 64 * b:64 * b + 64]                               # [16][64] codes
                    lanes = np.zeros((4, 16, 16), dtype=np.uint8)                   # g, row, byte
                    for g in range(4):
                        for d in range(2):
                            for h in range(2):
                                k0 = 32 * d + 8 * g + 4 * h
                                lanes[g, :, 4 * (2 * d + h):4 * (2 * d + h) + 4] = blk[:, k0:k0 + 4]
                    tiles.append(lanes.reshape(-1))
            sc = np.zeros(T * 16, dtype=np.float32)
            sc[:n] = np.asarray(mat["s"]).reshape(n_experts, n)[e]
            sb = sc.view(np.uint8)
            pad = (-len(sb)) % 256
            out.append(np.concatenate(tiles + [sb, np.zeros(pad, dtype=np.uint8)]))
    return np.concatenate(out)


@pytest.mark.parametrize("fmt,n,k,E", [(gen.FMT_INT4_AFFINE_G64, 40, 1152, 1),     # ragged tile, 9 blocks
                                       (gen.FMT_INT4_AFFINE_G64, 32, 768, 3),      # short group, experts
                                       (gen.FMT_INT4_AFFINE_G64, 16, 2048, 1),     # whole groups
                                       (gen.FMT_INT8_ROW, 37, 320, 2),
                                       (gen.FMT_INT8_ROW, 48, 64, 1)])
def test_pack_layout(fmt, n, k, E):
    print("[case] pack", fmt, n, k, E, flush=True)
    mat = gen.qmat(fmt, n, k, gen.tensor_key(9000 + n, k), experts=E if E > 1 else 0, row_scales=True)
    eb = fq.packed_bytes(fmt, n, k)
    want = ref_pack(mat, E)
    assert eb * E == want.size
    got = fq.pack(fq.to_device(mat), E)
    torch.cuda.synchronize()
    assert got["fmt"] == fq.TILED[fmt]
    assert np.array_equal(got["q"].cpu().numpy(), want)
