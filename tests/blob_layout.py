"""The bf16 expert blob, written out in numpy from the layout the C ABI
documents (gate/up matrix P1 then down matrix P2, 16-row tiles of 1 KiB
fragments; P1 row 4q + s of tile t is column 8t + 2q + s/2 of W1 for even s,
of W3 for odd s). Used by tests that need a blob on the host without the GPU
packer; a GPU test checks it byte for byte against moe_pack_expert."""
import numpy as np
import torch


def bf16_bits(t):
    """uint16 bit patterns of a torch bf16 tensor."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def fragments(M):
    """M uint16 [N, K] -> fragment order: tile, K chunk, lane (row + 16 * group), eight values."""
    N, K = M.shape
    return M.reshape(N // 16, 16, K // 32, 4, 8).transpose(0, 2, 3, 1, 4).reshape(-1)


def p1_rows(W1, W3):
    """[2I, H]: the interleaved gate/up rows."""
    H, I = W1.shape
    r = np.arange(2 * I)
    t, rr = r // 16, r % 16
    q, s = rr // 4, rr % 4
    i = 8 * t + 2 * q + s // 2
    return np.where((s % 2 == 0)[:, None], W1.T[i], W3.T[i])


def bf16_blob(W1, W3, W2):
    """uint16 blob of a bf16 expert (W1, W3 [H, I], W2 [I, H] as torch bf16)."""
    w1, w3, w2 = bf16_bits(W1), bf16_bits(W3), bf16_bits(W2)
    return np.ascontiguousarray(np.concatenate([fragments(p1_rows(w1, w3)), fragments(np.ascontiguousarray(w2.T))]))


def _align(v, a):
    return (v + a - 1) // a * a


def _fp4_blocks(C):
    """C uint8 codes [N, K] (rows = output rows) -> bytes in block order: tile, 128-wide K block, lane
    (row + 16 * group of 8), four words of eight nibbles (word j = K 32j + 8 * group + 0..7, nibble p =
    bits 4p..4p+3 = K offset p)."""
    N, K = C.shape
    c = C.reshape(N // 16, 16, K // 128, 4, 4, 8).astype(np.uint32)   # t, r, g, j, grp, p
    c = c.transpose(0, 2, 4, 1, 3, 5)                                 # t, g, grp, r, j, p
    words = (c << (4 * np.arange(8, dtype=np.uint32))).sum(axis=-1, dtype=np.uint32)
    return np.ascontiguousarray(words).view(np.uint8).reshape(-1)


def _fp4_scales(S):
    """S uint8 scales [N, K/32] -> per tile and 128-wide K block, 64 bytes: byte 4r + j = row r, block j."""
    N, KB = S.shape
    s = S.reshape(N // 16, 16, KB // 4, 4).transpose(0, 2, 1, 3)      # t, g, r, j
    return np.ascontiguousarray(s).reshape(-1)


def mxfp4_blob(C1, C3, C2, S1, S3, S2):
    """uint8 blob of an MXFP4 expert from codes C1, C3 [H, I], C2 [I, H] and scales S1, S3 [H/32, I],
    S2 [I/32, H] (numpy uint8): sections P1 codes, P1 scales, P2 codes, P2 scales, each 256-byte aligned."""
    H, I = C1.shape
    p1c = _fp4_blocks(p1_rows(C1, C3))
    p1s = _fp4_scales(p1_rows(S1, S3))
    p2c = _fp4_blocks(np.ascontiguousarray(C2.T))
    p2s = _fp4_scales(np.ascontiguousarray(S2.T))
    o_p1s = _align(len(p1c), 256)
    o_p2 = _align(o_p1s + len(p1s), 256)
    o_p2s = _align(o_p2 + len(p2c), 256)
    total = _align(o_p2s + len(p2s), 256)
    blob = np.zeros(total, np.uint8)
    blob[:len(p1c)] = p1c
    blob[o_p1s:o_p1s + len(p1s)] = p1s
    blob[o_p2:o_p2 + len(p2c)] = p2c
    blob[o_p2s:o_p2s + len(p2s)] = p2s
    return blob


def _int4_blocks(Q):
    """Q int8 codes in [-7, 7], [N, K] (rows = output rows) -> bytes in block order: tile, 128-wide K block,
    lane (row + 16 * group of 8), four words (word j = K 32j + 8 * group + 0..7); nibble p < 4 holds K offset
    2p and nibble p + 4 K offset 2p + 1, each as q + 8."""
    N, K = Q.shape
    c = (Q.astype(np.int32) + 8).astype(np.uint32).reshape(N // 16, 16, K // 128, 4, 4, 8)  # t, r, g, j, grp, k
    c = c.transpose(0, 2, 4, 1, 3, 5)                                  # t, g, grp, r, j, k
    nib = np.concatenate([c[..., 0::2], c[..., 1::2]], axis=-1)        # nibble order k0 k2 k4 k6 k1 k3 k5 k7
    words = (nib << (4 * np.arange(8, dtype=np.uint32))).sum(axis=-1, dtype=np.uint32)
    return np.ascontiguousarray(words).view(np.uint8).reshape(-1)


def _int4_scales(S):
    """S fp16 scales [N, K/128] -> per tile and 128-wide K block, the 16 rows' scales (32 bytes)."""
    N, KG = S.shape
    s = S.reshape(N // 16, 16, KG).transpose(0, 2, 1)                  # t, g, r
    return np.ascontiguousarray(s).view(np.uint8).reshape(-1)


def int4_blob(Q1, Q3, Q2, S1, S3, S2):
    """uint8 blob of an int4 expert from codes Q1, Q3 [H, I], Q2 [I, H] (int8) and fp16 scales S1, S3
    [H/128, I], S2 [I/128, H] (numpy): sections P1 codes, P1 scales, P2 codes, P2 scales, 256-byte aligned."""
    p1c = _int4_blocks(p1_rows(Q1, Q3))
    p1s = _int4_scales(p1_rows(S1, S3))
    p2c = _int4_blocks(np.ascontiguousarray(Q2.T))
    p2s = _int4_scales(np.ascontiguousarray(S2.T))
    o_p1s = _align(len(p1c), 256)
    o_p2 = _align(o_p1s + len(p1s), 256)
    o_p2s = _align(o_p2 + len(p2c), 256)
    total = _align(o_p2s + len(p2s), 256)
    blob = np.zeros(total, np.uint8)
    blob[:len(p1c)] = p1c
    blob[o_p1s:o_p1s + len(p1s)] = p1s
    blob[o_p2:o_p2 + len(p2c)] = p2c
    blob[o_p2s:o_p2s + len(p2s)] = p2s
    return blob
