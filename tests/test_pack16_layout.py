"""CPU check of the index algebra of the packed kernel's 16-row waves (no GPU).

Restated from prefill.hip: the swizzled K/V tile layout (16-byte chunk c of key row r
at byte r * ROWB + ((c ^ key(r)) << 4)); the lane layout of v_mfma_f32_16x16x32_bf16
(lane l: A[l % 16][8 (l / 16) + j], B[8 (l / 16) + j][l % 16], D[4 (l / 16) + i][l % 16]);
the transposed LDS read (in a 16-lane group, lane j points at row key0 + j / 4, dims
d0 + 4 (j % 4); lane i receives dims d0 + i of keys key0 .. key0 + 3); each wave's K and
V addresses (a per-lane base XOR-ed with the k-step or dim block); and the key order
of the P.V contraction (k = 8 q + 4 g + i <-> key 16 g + 4 q + i).  With integer
data, every score and output the lane model produces must equal the dense products.
"""

import numpy as np
import pytest


def swz_key(d, r):
    if d == 128:
        return ((r & 3) << 2) | ((r >> 2) & 3)
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3)


def swz(d, r, c):
    return r * d * 2 + ((c ^ swz_key(d, r)) << 4)


def decode_addr(d, addr):
    """(row, dim) of the bf16 element at byte offset addr of a swizzled tile."""
    rowb = d * 2
    r, off = divmod(addr, rowb)
    chunk = (off >> 4) ^ swz_key(d, r)
    return r, chunk * 8 + (off & 15) // 2


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hoff", [0, 1])
def test_scores_and_pv_follow_the_dense_products(d, hoff):
    rng = np.random.default_rng(d + hoff)
    BN = 64
    K = rng.integers(-4, 5, (BN, d))
    V = rng.integers(-4, 5, (BN, d))
    Q = rng.integers(-4, 5, (16, d))           # the wave's 16 rows
    KS, DB = d // 32, d // 16
    rowb = d * 2
    # --- S^T = K Q^T, per 16-key group g: the lane model ---
    S = np.zeros((32, 16), dtype=np.int64)     # [key within the half][row]
    for g in range(2):
        acc = np.zeros((64, 4), dtype=np.int64)
        for kk in range(KS):
            A = np.zeros((16, 32), dtype=np.int64)
            B = np.zeros((32, 16), dtype=np.int64)
            for l in range(64):
                n16, q4 = l & 15, l >> 4
                kx16 = swz(d, n16, q4)
                addr = 32 * hoff * rowb + 16 * g * rowb + (kx16 ^ (kk << 6))
                r, dim = decode_addr(d, addr)
                assert r == 32 * hoff + 16 * g + n16 and dim == 8 * q4 + 32 * kk
                for j in range(8):
                    A[n16][8 * q4 + j] = K[r][dim + j]
                    B[8 * q4 + j][n16] = Q[n16][8 * q4 + 32 * kk + j]
            Dm = A @ B
            for l in range(64):
                for i in range(4):
                    acc[l][i] += Dm[4 * (l >> 4) + i][l & 15]
        for l in range(64):
            for i in range(4):
                S[16 * g + 4 * (l >> 4) + i][l & 15] = acc[l][i]
    assert np.array_equal(S, K[32 * hoff:32 * hoff + 32] @ Q.T)
    # --- O^T += V^T P^T over the half's 32 keys ---
    P = rng.integers(-3, 4, (16, 32))          # [row][key within the half]
    Ot = np.zeros((d, 16), dtype=np.int64)
    for db in range(DB):
        A = np.zeros((16, 32), dtype=np.int64)
        B = np.zeros((32, 16), dtype=np.int64)
        for l in range(64):
            n16, q4 = l & 15, l >> 4
            # B: the lane's own weights, k = 8 q4 + t <-> key (t < 4) 4 q4 + t, else 16 + 4 q4 + t - 4
            for t in range(8):
                key = 4 * q4 + t if t < 4 else 16 + 4 * q4 + (t - 4)
                B[8 * q4 + t][n16] = P[n16][key]
            # A: two transposed reads; lane j = n16 of group q4 points at its row / dims
            vx16 = swz(d, 4 * q4 + (n16 >> 2), (n16 & 3) >> 1) + ((n16 & 1) << 3)
            for h in range(2):
                addr = 32 * hoff * rowb + 16 * h * rowb + (vx16 ^ (db << 5))
                r, dim = decode_addr(d, addr)
                assert r == 32 * hoff + 16 * h + 4 * q4 + (n16 >> 2) and dim == 16 * db + 4 * (n16 & 3)
        for l in range(64):
            n16, q4 = l & 15, l >> 4
            for h in range(2):
                key0 = 32 * hoff + 16 * h + 4 * q4
                for t in range(4):
                    A[n16][8 * q4 + 4 * h + t] = V[key0 + t][16 * db + n16]
        Dm = A @ B
        for l in range(64):
            for i in range(4):   # the lane's outputs: dims 16 db + 4 q + i of row l % 16
                Ot[16 * db + 4 * (l >> 4) + i][l & 15] = Dm[4 * (l >> 4) + i][l & 15]
    assert np.array_equal(Ot, V[32 * hoff:32 * hoff + 32].T @ P.T)


@pytest.mark.parametrize("d", [64, 128])
def test_reads_stay_inside_their_tile(d):
    """Every K and V address of a wave lies inside the 64-row tile."""
    rowb = d * 2
    for hoff in range(2):
        for l in range(64):
            n16, q4 = l & 15, l >> 4
            for g in range(2):
                for kk in range(d // 32):
                    a = 32 * hoff * rowb + 16 * g * rowb + (swz(d, n16, q4) ^ (kk << 6))
                    assert 0 <= a and a + 16 <= 64 * rowb
            vx16 = swz(d, 4 * q4 + (n16 >> 2), (n16 & 3) >> 1) + ((n16 & 1) << 3)
            for h in range(2):
                for db in range(d // 16):
                    a = 32 * hoff * rowb + 16 * h * rowb + (vx16 ^ (db << 5))
                    assert 0 <= a and a + 8 <= 64 * rowb
