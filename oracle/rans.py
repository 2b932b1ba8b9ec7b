"""Reference (pure Python / numpy) of the code container written by the device's entropy coder.

TEST INFRASTRUCTURE ONLY. Only ``tests/`` may import this module. It shares no code with the HIP
path; it fixes the format bit for bit so that the device encoder can be compared byte by byte.

Why a coder: the WaterSIC page (§2 item 3) stores the integer codes without a fixed range and
compresses them with an entropy coder, so the rate of a layer is what that coder writes; the
pages name Huffman / Zstd (WaterSIC) and an ANS coder (EntQuant) but fix no format. This one is
range-variant ANS (rANS) with a static table built from the layer's pooled code histogram:

* alphabet: the codes in [lo, hi] (lo, hi: the extreme codes within +-2047) plus one escape
  symbol (the last); an escaped code is stored as a raw int32 in a side array;
* frequencies: counts scaled to M = 2^14 (f = max(1, floor(c M / N)) for every present symbol; the
  remainder M - sum f is added to the most frequent symbol, or taken one by one from the largest
  frequency above 1, lowest index first);
* streams: symbol p of the flattened codes belongs to group g = p // (64 L) and lane
  l = p % 64; lane l of group g holds the L symbols p = (g L + k) 64 + l, k = 0 .. L-1;
* coding: 32-bit state x in [2^16, 2^32), 16-bit renormalization; symbol s with frequency f and
  cumulative c is encoded as x -> ((x // f) << 14) + x % f + c after emitting the low 16 bits if
  x >= f << 18; decoding inverts it and reads one word when x < 2^16;
* word order: the words of a group are stored in the order the decoder consumes them: by step k,
  then by lane among the lanes that read a word at that step; escapes likewise by step, then lane.

Container (little endian): header u32[16] = (magic 0x534E5257, version 1, N lo, N hi, L, groups,
lo, nsym, 14, n_esc, payload words, 0...), u16 freq[nsym] (padded to 16 bytes), u32 group word
offsets[groups + 1], u32 group escape offsets[groups + 1], u32 initial states[64 groups], int32
escapes[n_esc], u16 payload[words]; every section starts at a multiple of 16 bytes and the
container ends with the payload.
"""
from __future__ import annotations

import numpy as np

PROB_BITS = 14
M = 1 << PROB_BITS
LANES = 64
WINDOW = 2047
MAGIC = 0x534E5257
RANS_L = 1 << 16


def _align16(x: int) -> int:
    return (x + 15) // 16 * 16


def build_table(codes: np.ndarray):
    """(lo, freq): the alphabet's first code and the normalized frequencies (escape last)."""
    q = np.asarray(codes, dtype=np.int64).ravel()
    inw = q[(q >= -WINDOW) & (q <= WINDOW)]
    lo, hi = (int(inw.min()), int(inw.max())) if inw.size else (0, 0)
    nsym = hi - lo + 2
    counts = np.zeros(nsym, dtype=np.int64)
    np.add.at(counts, inw - lo, 1)
    counts[-1] = q.size - inw.size
    N = int(q.size)
    f = np.where(counts > 0, np.maximum(1, (counts * M) // N), 0).astype(np.int64)
    diff = M - int(f.sum())
    if diff > 0:
        f[int(np.argmax(counts))] += diff
    while diff < 0:
        cand = np.where(f > 1, f, -1)
        f[int(np.argmax(cand))] -= 1
        diff += 1
    return lo, f


def encode(codes: np.ndarray, L: int) -> bytes:
    q = np.asarray(codes, dtype=np.int64).ravel()
    N = q.size
    lo, f = build_table(q)
    nsym = f.size
    cum = np.concatenate([[0], np.cumsum(f)[:-1]])
    esc = nsym - 1
    G = (N + LANES * L - 1) // (LANES * L)
    group_words, group_esc, states = [], [], []
    for g in range(G):
        x = [RANS_L] * LANES
        steps_words = []  # per step (reverse order of k): list of words by lane
        steps_esc = []
        for k in range(L - 1, -1, -1):
            wk, ek = [], []
            for l in range(LANES):
                p = (g * L + k) * LANES + l
                if p >= N:
                    continue
                v = int(q[p])
                s = v - lo if (-WINDOW <= v <= WINDOW) else esc
                if s == esc:
                    ek.append(v)
                fs, cs = int(f[s]), int(cum[s])
                xl = x[l]
                if xl >= (fs << 18):
                    wk.append(xl & 0xFFFF)
                    xl >>= 16
                x[l] = ((xl // fs) << PROB_BITS) + (xl % fs) + cs
            steps_words.append(wk)
            steps_esc.append(ek)
        # decoder order: k ascending; within a step, lanes ascending
        words = [w for wk in reversed(steps_words) for w in wk]
        escs = [e for ek in reversed(steps_esc) for e in ek]
        group_words.append(words)
        group_esc.append(escs)
        states.extend(x)
    payload = [w for gw in group_words for w in gw]
    escapes = [e for ge in group_esc for e in ge]
    gofs = np.concatenate([[0], np.cumsum([len(w) for w in group_words])]).astype(np.uint32)
    eofs = np.concatenate([[0], np.cumsum([len(e) for e in group_esc])]).astype(np.uint32)
    header = np.zeros(16, dtype=np.uint32)
    header[:11] = [MAGIC, 1, N & 0xFFFFFFFF, N >> 32, L, G, lo & 0xFFFFFFFF, nsym, PROB_BITS,
                   len(escapes), len(payload)]
    out = bytearray()
    out += header.tobytes()
    out += np.asarray(f, dtype=np.uint16).tobytes()
    out += bytes(_align16(len(out)) - len(out))
    out += gofs.tobytes()
    out += bytes(_align16(len(out)) - len(out))
    out += eofs.tobytes()
    out += bytes(_align16(len(out)) - len(out))
    out += np.asarray(states, dtype=np.uint32).tobytes()
    out += bytes(_align16(len(out)) - len(out))
    out += np.asarray(escapes, dtype=np.int32).tobytes()
    out += bytes(_align16(len(out)) - len(out))
    out += np.asarray(payload, dtype=np.uint16).tobytes()
    return bytes(out)


def decode(blob: bytes) -> np.ndarray:
    h = np.frombuffer(blob[:64], dtype=np.uint32)
    assert int(h[0]) == MAGIC
    N = int(h[2]) | (int(h[3]) << 32)
    L, G, lo, nsym, n_esc, nw = int(h[4]), int(h[5]), int(np.int32(h[6])), int(h[7]), int(h[9]), int(h[10])
    off = 64
    f = np.frombuffer(blob[off:off + 2 * nsym], dtype=np.uint16).astype(np.int64)
    off = _align16(off + 2 * nsym)
    gofs = np.frombuffer(blob[off:off + 4 * (G + 1)], dtype=np.uint32)
    off = _align16(off + 4 * (G + 1))
    eofs = np.frombuffer(blob[off:off + 4 * (G + 1)], dtype=np.uint32)
    off = _align16(off + 4 * (G + 1))
    states = np.frombuffer(blob[off:off + 4 * LANES * G], dtype=np.uint32)
    off = _align16(off + 4 * LANES * G)
    escapes = np.frombuffer(blob[off:off + 4 * n_esc], dtype=np.int32)
    off = _align16(off + 4 * n_esc)
    payload = np.frombuffer(blob[off:off + 2 * nw], dtype=np.uint16)
    cum = np.concatenate([[0], np.cumsum(f)])
    slot_sym = np.repeat(np.arange(nsym), f)
    out = np.zeros(N, dtype=np.int64)
    for g in range(G):
        x = [int(v) for v in states[LANES * g:LANES * (g + 1)]]
        wp, ep = int(gofs[g]), int(eofs[g])
        for k in range(L):
            for l in range(LANES):
                p = (g * L + k) * LANES + l
                if p >= N:
                    continue
                slot = x[l] & (M - 1)
                s = int(slot_sym[slot])
                xl = int(f[s]) * (x[l] >> PROB_BITS) + slot - int(cum[s])
                if s == nsym - 1:
                    out[p] = int(escapes[ep])
                    ep += 1
                else:
                    out[p] = lo + s
                if xl < RANS_L:
                    xl = (xl << 16) | int(payload[wp])
                    wp += 1
                x[l] = xl
    return out
