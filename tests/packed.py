"""The packed storage of a symmetric d x d key moment (d = 32, 64, 128), as
include/hla.h states it, written out index by index: the 32 x 32 tiles
(I, J), I <= J, in row-major tile order; an off-diagonal tile whole (row
major), a diagonal tile as its upper triangle (row r holding columns
r..31).  Test infrastructure: the reference the GPU pack/unpack and the
packed decode state are checked against."""
import numpy as np

TS = 32


def order(d: int):
    """(row, col) of every packed element, in storage order."""
    nt = d // TS
    idx = []
    for I in range(nt):
        for J in range(I, nt):
            for r in range(TS):
                for c in range(r if I == J else 0, TS):
                    idx.append((TS * I + r, TS * J + c))
    return np.array(idx, dtype=np.int64)


def pack(S):
    """[N,d,d] -> [N, d(d+1)/2] (upper triangle, storage order)."""
    S = np.asarray(S)
    d = S.shape[-1]
    ix = order(d)
    return np.ascontiguousarray(S[:, ix[:, 0], ix[:, 1]])


def unpack(P, d: int):
    """[N, d(d+1)/2] -> [N,d,d], both triangles."""
    P = np.asarray(P)
    ix = order(d)
    out = np.zeros((P.shape[0], d, d), dtype=P.dtype)
    out[:, ix[:, 0], ix[:, 1]] = P
    out[:, ix[:, 1], ix[:, 0]] = P
    return out
