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
