"""Index map of the MFMA-order packed weight layout (oracle; test use only).

The model card "nunchaku-z-image-turbo-svdq" (section "Why row-major, and
what about consumer-card nunchaku kernels") describes a one-shot load-time
pack of qweight/wscales into a kernel-specific tile order, forming a
bit-exact pair with its unpack (section "Conversion source": round trip
verified bit-exact). The order used by this library is its own, chosen for
the gfx950 32x32x16 matrix instruction; it is stated here from its definition
so the GPU repack can be checked byte for byte:

* Panels: n-panel q covers output channels 32q .. 32q+31, k-panel p covers
  k = 64p .. 64p+63 (four 16-blocks). NP = ceil(N/32), KP = ceil(K/64).
* Code region, chunk (p, q) at byte offset 1024 * (p * NP + q): dword
  d = (h * 32 + c) * 4 + t (h in 0..1, c in 0..31, t in 0..3) holds the eight
  codes of channel n = 32q + c at k = 64p + 16t + 8h + 0..7, i.e. the four
  canonical qweight bytes [n, k/2 .. k/2 + 3] unchanged (low nibble = even k).
* Scale region, after all code chunks, chunk (p, q) at byte offset
  1024 * KP * NP + 128 * (p * NP + q): byte c * 4 + t holds wscales[4p + t, 32q + c].
* Positions outside N or K hold zero bytes (code 0 = +0.0, scale 0).
"""

import numpy as np

PANEL_N = 32
PANEL_K = 64


def packed_bytes(N, K):
    NP = -(-N // PANEL_N)
    KP = -(-K // PANEL_K)
    return NP * KP * (PANEL_N * PANEL_K // 2 + PANEL_N * PANEL_K // 16)


def repack(qweight, wscales):
    """qweight [N, K/2] uint8, wscales [K/16, N] uint8 -> packed uint8 buffer.

    Array form of the index map: pad to whole panels with zeros, then read the
    byte axis of a row as (p, t, h, byte) since k/2 = 32p + 8t + 4h + byte, and
    order the code bytes as [p, q, h, c, t, byte], the scales as [p, q, c, t].
    (repack_loops states the same map element by element.)
    """
    qweight = np.asarray(qweight, dtype=np.uint8)
    wscales = np.asarray(wscales, dtype=np.uint8)
    N, Kh = qweight.shape
    K = 2 * Kh
    NP = -(-N // PANEL_N)
    KP = -(-K // PANEL_K)
    qw = np.zeros((NP * 32, KP * 32), dtype=np.uint8)
    qw[:N, :Kh] = qweight
    ws = np.zeros((KP * 4, NP * 32), dtype=np.uint8)
    ws[:K // 16, :N] = wscales
    codes = qw.reshape(NP, 32, KP, 4, 2, 4).transpose(2, 0, 4, 1, 3, 5)   # [p, q, h, c, t, byte]
    scales = ws.reshape(KP, 4, NP, 32).transpose(0, 2, 3, 1)              # [p, q, c, t]
    return np.concatenate([codes.ravel(), scales.ravel()])


def unpack(packed, N, K):
    """Inverse of repack: packed buffer -> (qweight [N, K/2], wscales [K/16, N])."""
    packed = np.asarray(packed, dtype=np.uint8)
    NP = -(-N // PANEL_N)
    KP = -(-K // PANEL_K)
    nc = NP * KP * 1024
    codes = packed[:nc].reshape(KP, NP, 2, 32, 4, 4).transpose(1, 3, 0, 4, 2, 5)  # [q, c, p, t, h, byte]
    scales = packed[nc:nc + NP * KP * 128].reshape(KP, NP, 32, 4).transpose(0, 3, 1, 2)  # [p, t, q, c]
    qweight = codes.reshape(NP * 32, KP * 32)[:N, :K // 2]
    wscales = scales.reshape(KP * 4, NP * 32)[:K // 16, :N]
    return np.ascontiguousarray(qweight), np.ascontiguousarray(wscales)


def repack_loops(qweight, wscales):
    """The same map written element by element (used to pin the array form)."""
    qweight = np.asarray(qweight, dtype=np.uint8)
    wscales = np.asarray(wscales, dtype=np.uint8)
    N, Kh = qweight.shape
    K = 2 * Kh
    NP = -(-N // PANEL_N)
    KP = -(-K // PANEL_K)
    out = np.zeros(packed_bytes(N, K), dtype=np.uint8)
    code_region = NP * KP * 1024
    for p in range(KP):
        for q in range(NP):
            base = 1024 * (p * NP + q)
            sbase = code_region + 128 * (p * NP + q)
            for c in range(PANEL_N):
                n = PANEL_N * q + c
                if n >= N:
                    continue
                for t in range(4):
                    blk = 4 * p + t
                    if 16 * blk < K:
                        out[sbase + c * 4 + t] = wscales[blk, n]
                    for h in range(2):
                        k = PANEL_K * p + 16 * t + 8 * h
                        if k >= K:
                            continue
                        d = (h * 32 + c) * 4 + t
                        out[base + 4 * d: base + 4 * d + 4] = qweight[n, k // 2: k // 2 + 4]
    return out


def unpack_loops(packed, N, K):
    """Inverse of repack_loops, element by element."""
    packed = np.asarray(packed, dtype=np.uint8)
    NP = -(-N // PANEL_N)
    KP = -(-K // PANEL_K)
    qweight = np.zeros((N, K // 2), dtype=np.uint8)
    wscales = np.zeros((K // 16, N), dtype=np.uint8)
    code_region = NP * KP * 1024
    for p in range(KP):
        for q in range(NP):
            base = 1024 * (p * NP + q)
            sbase = code_region + 128 * (p * NP + q)
            for c in range(PANEL_N):
                n = PANEL_N * q + c
                if n >= N:
                    continue
                for t in range(4):
                    blk = 4 * p + t
                    if 16 * blk < K:
                        wscales[blk, n] = packed[sbase + c * 4 + t]
                    for h in range(2):
                        k = PANEL_K * p + 16 * t + 8 * h
                        if k >= K:
                            continue
                        d = (h * 32 + c) * 4 + t
                        qweight[n, k // 2: k // 2 + 4] = packed[base + 4 * d: base + 4 * d + 4]
    return qweight, wscales
