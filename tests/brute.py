"""Brute-force direct correlation in pure Python (tiny inputs only).

Written independently of ``oracle/oracle.cpp``: nested Python loops over Python
numbers (exact for integer-valued data), iterating output pixel by output
pixel, tap by tap.  Used only to pin the oracle.
"""


def out_size(n, k, s, p, d):
    return (n + 2 * p - d * (k - 1) - 1) // s + 1


def conv2d(x, w, stride, pad, dil):
    """x: nested lists [N][H][W][C]; w: [O][KH][KW][C]; returns [N][OH][OW][O]."""
    N, H, W, C = len(x), len(x[0]), len(x[0][0]), len(x[0][0][0])
    O, KH, KW = len(w), len(w[0]), len(w[0][0])
    sh, sw = stride
    ph, pw = pad
    dh, dw = dil
    OH, OW = out_size(H, KH, sh, ph, dh), out_size(W, KW, sw, pw, dw)
    y = [[[[0 for _ in range(O)] for _ in range(OW)] for _ in range(OH)] for _ in range(N)]
    for n in range(N):
        for i in range(OH):
            for j in range(OW):
                for o in range(O):
                    s = 0
                    for a in range(KH):
                        for b in range(KW):
                            r = i * sh - ph + a * dh
                            q = j * sw - pw + b * dw
                            if 0 <= r < H and 0 <= q < W:
                                for c in range(C):
                                    s += x[n][r][q][c] * w[o][a][b][c]
                    y[n][i][j][o] = s
    return y


def conv3d(x, w, stride, pad, dil):
    """x: [N][D][H][W][C]; w: [O][KD][KH][KW][C]; returns [N][OD][OH][OW][O]."""
    N, D, H, W, C = len(x), len(x[0]), len(x[0][0]), len(x[0][0][0]), len(x[0][0][0][0])
    O, KD, KH, KW = len(w), len(w[0]), len(w[0][0]), len(w[0][0][0])
    OD = out_size(D, KD, stride[0], pad[0], dil[0])
    OH = out_size(H, KH, stride[1], pad[1], dil[1])
    OW = out_size(W, KW, stride[2], pad[2], dil[2])
    y = [[[[[0] * O for _ in range(OW)] for _ in range(OH)] for _ in range(OD)] for _ in range(N)]
    for n in range(N):
        for e in range(OD):
            for i in range(OH):
                for j in range(OW):
                    for o in range(O):
                        s = 0
                        for t in range(KD):
                            for a in range(KH):
                                for b in range(KW):
                                    z = e * stride[0] - pad[0] + t * dil[0]
                                    r = i * stride[1] - pad[1] + a * dil[1]
                                    q = j * stride[2] - pad[2] + b * dil[2]
                                    if 0 <= z < D and 0 <= r < H and 0 <= q < W:
                                        for c in range(C):
                                            s += x[n][z][r][q][c] * w[o][t][a][b][c]
                        y[n][e][i][j][o] = s
    return y
