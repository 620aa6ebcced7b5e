"""Oracle of the fused feature transforms (test infrastructure only).

"RecIS：阿里开源推荐系统统一训练框架", "Feature Engine": feature conversion with
Hash, Mod and Bucketize, several small operations merged into one GPU kernel
launch.  The pages name the operations and nothing more; the definitions
followed here (and by the HIP kernel, which shares no code with this file):

* every lookup of table t holds one 64-bit raw value (the table-major layout
  of the ids); table t's program says whether the raw value is an int64 or
  the bits of a float64, and lists up to four operations applied in order;
* Hash(seed): XXH64 (Collet's published xxHash64 algorithm) of the value's 8
  little-endian bytes with the given seed; the 64-bit digest, read as a
  signed int64, is the new value.  On a float64 value it hashes the bits;
* Mod(m), m > 0: floor modulo of the value read as a signed int64, a result
  in [0, m) (Python's and numpy's `%` on integers);
* Bucketize(boundaries), a float64 value x and boundaries sorted ascending:
  the number of boundaries b with b <= x (NaN counts every boundary), an
  integer in [0, len(boundaries)];
* an integer program may use Hash and Mod; a float program must start with
  Bucketize or Hash (after which the value is an integer); the final value
  is the id.

Written in numpy with wrapping uint64 arithmetic; each step follows its
definition directly.
"""

from __future__ import annotations

import numpy as np

INT64, FLOAT64 = 0, 1
IDENTITY, HASH, MOD, BUCKETIZE = 0, 1, 2, 3
MAX_OPS = 4

# xxHash64 primes (from the algorithm's specification)
P1 = np.uint64(0x9E3779B185EBCA87)
P2 = np.uint64(0xC2B2AE3D27D4EB4F)
P3 = np.uint64(0x165667B19E3779F9)
P4 = np.uint64(0x85EBCA77C2B2AE63)
P5 = np.uint64(0x27D4EB2F165667C5)


def _rotl(x, r):
    return (x << np.uint64(r)) | (x >> np.uint64(64 - r))


def xxh64_u64(values, seed: int) -> np.ndarray:
    """XXH64 of each 8-byte little-endian word, with `seed`: an input shorter
    than 32 bytes starts from seed + P5, adds the length, folds in the one
    8-byte lane (lane * P2, rotate 31, * P1; xor; rotate 27, * P1 + P4) and
    ends with the avalanche (shift-xor 33, * P2, shift-xor 29, * P3,
    shift-xor 32)."""
    v = np.asarray(values).view(np.uint64) if np.asarray(values).dtype != np.uint64 else np.asarray(values)
    with np.errstate(over="ignore"):
        acc = np.uint64(seed & (2**64 - 1)) + P5 + np.uint64(8)
        k1 = _rotl(v * P2, 31) * P1
        acc = acc ^ k1
        acc = _rotl(acc, 27) * P1 + P4
        acc = acc ^ (acc >> np.uint64(33))
        acc = acc * P2
        acc = acc ^ (acc >> np.uint64(29))
        acc = acc * P3
        acc = acc ^ (acc >> np.uint64(32))
    return acc.astype(np.uint64)


def floor_mod(values, m: int) -> np.ndarray:
    """Floor modulo of signed int64 values by m > 0: in [0, m) (numpy's mod
    on integers takes the sign of the divisor)."""
    return np.mod(np.asarray(values).view(np.int64), np.int64(m))


def bucketize(x, boundaries) -> np.ndarray:
    """Number of boundaries b with b <= x, for each float64 x; NaN gives
    len(boundaries)."""
    x = np.asarray(x, np.float64)
    b = np.asarray(boundaries, np.float64)
    out = np.empty(x.shape, np.int64)
    chunk = max(1, (1 << 22) // max(1, b.size))
    for s in range(0, x.size, chunk):
        xs = x[s:s + chunk]
        cnt = (b[None, :] <= xs[:, None]).sum(axis=1)
        out[s:s + chunk] = np.where(np.isnan(xs), b.size, cnt)
    return out


class Program:
    """One table's transform: input kind and a list of (op, argument)
    pairs: HASH seed, MOD modulus, BUCKETIZE boundaries (ascending)."""

    def __init__(self, input_kind=INT64, ops=()):
        self.input = input_kind
        self.ops = list(ops)

    def valid(self) -> bool:
        if len(self.ops) > MAX_OPS:
            return False
        is_float = self.input == FLOAT64
        for op, arg in self.ops:
            if op == BUCKETIZE:
                if not is_float:
                    return False
                b = np.asarray(arg, np.float64)
                if b.ndim != 1 or np.isnan(b).any() or (np.diff(b) < 0).any():
                    return False
                is_float = False
            elif op == HASH:
                is_float = False
            elif op == MOD:
                if is_float or int(arg) <= 0:
                    return False
            elif op != IDENTITY:
                return False
        return not is_float


def transform(raw, bounds, programs) -> np.ndarray:
    """ids[i] for every lookup: table t's program applied to raw[i] for
    bounds[t] <= i < bounds[t+1].  raw: 64-bit words (int64 view)."""
    raw = np.ascontiguousarray(raw).view(np.int64)
    out = np.empty(raw.shape, np.int64)
    for t, prog in enumerate(programs):
        if not prog.valid():
            raise ValueError(f"table {t}: invalid program")
        lo, hi = int(bounds[t]), int(bounds[t + 1])
        v = raw[lo:hi].copy()
        for op, arg in prog.ops:
            if op == HASH:
                v = xxh64_u64(v.view(np.uint64), int(arg)).view(np.int64)
            elif op == MOD:
                v = floor_mod(v, int(arg))
            elif op == BUCKETIZE:
                v = bucketize(v.view(np.float64), arg)
        out[lo:hi] = v
    return out
