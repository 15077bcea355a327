"""Independent numpy readings of the cache format and of softmax attention.

Used only to pin the oracle: it unpacks pool bytes with numpy bit arrays
(not the oracle's bit loop), dequantises in float64 and computes attention
with plain numpy softmax.  It shares no code with the oracle.
"""
from __future__ import annotations

import numpy as np

BT = 64


def pad128(x: int) -> int:
    return -(-x // 128) * 128


def layout(D: int, g: int, kb: int, vb: int) -> list[int]:
    """Section offsets [K codes, V codes, K scales, V scales, K zeros, V zeros, chunk]."""
    ng = 0 if kb == 16 else D // g
    sizes = [BT * D * kb // 8, D * BT * vb // 8, ng * BT * 4, ng * BT * 4, ng * BT, ng * BT]
    off, at = [], 0
    for s in sizes:
        off.append(at)
        at += pad128(s)
    return off + [at]


def unpack(buf: np.ndarray, n: int, bits: int) -> np.ndarray:
    """Fields of `bits` bits, LSB first, from a byte buffer -> uint32 [n]."""
    b = np.unpackbits(np.asarray(buf, np.uint8), bitorder="little")[: n * bits]
    b = b.reshape(n, bits).astype(np.uint64)
    w = (1 << np.arange(bits, dtype=np.uint64))
    return (b * w).sum(axis=1).astype(np.uint32)


def dequant_chunk(chunk: np.ndarray, D: int, g: int, kb: int, vb: int):
    """(K_hat, V_hat) float64 [64][D] of one chunk, plus raw codes/metadata."""
    off = layout(D, g, kb, vb)
    kc = unpack(chunk[off[0]:off[0] + BT * D * kb // 8], BT * D, kb).reshape(BT, D)
    vc = unpack(chunk[off[1]:off[1] + D * BT * vb // 8], D * BT, vb).reshape(D, BT).T
    if kb == 16:
        kh = kc.astype(np.uint16).view(np.float16).astype(np.float64)
        vh = vc.astype(np.uint16).view(np.float16).astype(np.float64)
        return kh, vh, dict(kc=kc, vc=vc)
    ng = D // g
    ks = chunk[off[2]:off[2] + ng * BT * 4].view(np.float32).reshape(ng, BT)
    vs = chunk[off[3]:off[3] + ng * BT * 4].view(np.float32).reshape(ng, BT)
    kz = chunk[off[4]:off[4] + ng * BT].reshape(ng, BT)
    vz = chunk[off[5]:off[5] + ng * BT].reshape(ng, BT)
    gidx = np.arange(D) // g
    kh = (kc.astype(np.float64) - kz[gidx, :].T.astype(np.float64)) * ks[gidx, :].T.astype(np.float64)
    vh = (vc.astype(np.float64) - vz[gidx, :].T.astype(np.float64)) * vs[gidx, :].T.astype(np.float64)
    return kh, vh, dict(kc=kc, vc=vc, ks=ks, vs=vs, kz=kz, vz=vz)


def dequant_sequence(pool: np.ndarray, chunk_bytes: int, Hkv: int, D: int, g: int, kb: int, vb: int,
                     block_row: np.ndarray, n: int, knorm_offset: int | None = None):
    """K_hat, V_hat float64 [Hkv][n][D] of one sequence.  knorm_offset: the
    byte offset of the per-slot fp32 norm factors of a direction-preserving
    K cache, which scale each K row."""
    K = np.zeros((Hkv, n, D))
    V = np.zeros((Hkv, n, D))
    for lb in range(-(-n // BT)):
        blk = int(block_row[lb])
        for h in range(Hkv):
            o = (blk * Hkv + h) * chunk_bytes
            kh, vh, _ = dequant_chunk(pool[o:o + chunk_bytes], D, g, kb, vb)
            if knorm_offset is not None:
                r = pool[o + knorm_offset:o + knorm_offset + 4 * BT].view(np.float32).astype(np.float64)
                kh = kh * r[:, None]
            m = min(BT, n - lb * BT)
            K[h, lb * BT:lb * BT + m] = kh[:m]
            V[h, lb * BT:lb * BT + m] = vh[:m]
    return K, V


def token_fields(pool: np.ndarray, chunk_bytes: int, Hkv: int, D: int, g: int, kb: int, vb: int,
                 block_row: np.ndarray, n: int) -> dict:
    """Raw fields of positions 0 .. n-1 of one sequence, every KV head:
    codes kc, vc [Hkv][n][D]; scales ks, vs as fp32 bit patterns and zero
    points kz, vz [Hkv][n][D/g] (quantised formats)."""
    out = {k: [] for k in ("kc", "vc", "ks", "vs", "kz", "vz")}
    for h in range(Hkv):
        rows = {k: [] for k in out}
        for lb in range(-(-n // BT)):
            o = (int(block_row[lb]) * Hkv + h) * chunk_bytes
            _, _, f = dequant_chunk(pool[o:o + chunk_bytes], D, g, kb, vb)
            m = min(BT, n - lb * BT)
            rows["kc"].append(f["kc"][:m])
            rows["vc"].append(f["vc"][:m])
            for k in ("ks", "vs", "kz", "vz"):
                a = f[k].view(np.uint32) if k in ("ks", "vs") else f[k]
                rows[k].append(a[:, :m].T)
        for k in out:
            out[k].append(np.concatenate(rows[k]) if rows[k] else np.zeros((0,), np.uint32))
    return {k: np.stack(v) for k, v in out.items()}


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float, keep=None) -> np.ndarray:
    """Brute-force softmax attention, float64.

    q [Hq][D]; K, V [Hkv][n][D]; query head h reads KV head h // (Hq/Hkv).
    keep: optional bool [Hq][n]; False drops the token's V term but keeps it
    in the denominator."""
    Hq = q.shape[0]
    Hkv = K.shape[0]
    G = Hq // Hkv
    out = np.zeros((Hq, K.shape[2]))
    for h in range(Hq):
        s = (K[h // G] @ q[h].astype(np.float64)) * float(sm_scale)
        w = np.exp(s - s.max())
        denom = w.sum()
        if keep is not None:
            w = w * keep[h]
        out[h] = (w @ V[h // G]) / denom
    return out
