"""A CPU model of the dispatch unpack kernel's indexing (k_unpack with the row-streaming engine),
for finding out-of-bounds accesses without a GPU.

It follows the kernel step by step for every block: the rank bases one wave writes into LDS, the
per-row resolve (rank by a count over the bases, source by a count over the receive offsets, the
expert-major position from the counts table and the row's metadata), the row descriptors the
waves write into LDS, and the streaming engine's mapping of each thread's chunks to rows
(including its float reciprocal) and to source and destination addresses.  LDS is modelled as the
hardware lays it out for this kernel: the static descriptor array rows[RPB] (32 bytes each)
first, the dynamic rank-base table right after it; a descriptor index past RPB lands in that
table.  Every LDS index, table index and buffer address is checked, and the model also moves the
bytes, so a correct configuration reproduces the oracle's expert-major rows exactly.

rows_per_wave > 1 models the several-rows-per-wave form (wave w resolves rows w, w + 4, ...).
`check_slot` False leaves out the test that a resolved row's descriptor slot is below RPB.
"""
from __future__ import annotations

import numpy as np

WAVES = 4
THREADS = 256
DESC_INTS = 8  # one row descriptor: four 64-bit addresses


class Violation(AssertionError):
    pass


def _check(cond, msg):
    if not cond:
        raise Violation(msg)


LDS_GRANULE_WORDS = 128  # a block's LDS is allocated in 512-byte granules


class Lds:
    """Flat LDS of one block in 4-byte words: rows[RPB] descriptors, then the dynamic int table
    gb[rc + 1], the allocation rounded up to whole granules.  A write inside the allocation lands
    whatever variable it hits (an overrun of rows[] overwrites gb[]); one outside it is a
    violation."""

    def __init__(self, rpb, rc, stale):
        self.rpb, self.rc = rpb, rc
        self.desc_words = rpb * DESC_INTS
        used = self.desc_words + rc + 1
        alloc = -(-used // LDS_GRANULE_WORDS) * LDS_GRANULE_WORDS
        self.words = np.zeros(alloc, dtype=np.int64)
        n = min(alloc, len(stale))
        self.words[:n] = stale[:n]
        self.overruns = 0

    def set_gb(self, i, v):
        _check(0 <= i <= self.rc, f"gb[{i}] outside the table of {self.rc + 1}")
        self.words[self.desc_words + i] = v

    def gb(self, i):
        _check(0 <= i <= self.rc, f"gb[{i}] outside the table of {self.rc + 1}")
        return int(self.words[self.desc_words + i])

    def write_desc(self, slot, desc):
        # the hardware writes wherever the index points inside the block's LDS
        w0 = slot * DESC_INTS
        _check(0 <= w0 and w0 + DESC_INTS <= len(self.words),
               f"descriptor slot {slot} beyond the block's LDS allocation")
        if slot >= self.rpb:
            self.overruns += 1  # lands on gb[] (or on the allocation's unused tail)
        for k in range(4):      # each 64-bit address as two words
            self.words[w0 + 2 * k] = desc[k] & 0xFFFFFFFF
            self.words[w0 + 2 * k + 1] = desc[k] >> 32

    def read_desc(self, slot):
        _check(0 <= slot < self.rpb, f"descriptor slot {slot} read outside rows[{self.rpb}]")
        w0 = slot * DESC_INTS
        return [int(self.words[w0 + 2 * k]) | (int(self.words[w0 + 2 * k + 1]) << 32) for k in range(4)]


def emulate_unpack(D, counts, recv_off, recv_buf, recv_meta, expert_x, expert_scale, expert_src,
                   expert_rpos, rpb, u, rows_per_wave=1, check_slot=True, stride_blocks=None,
                   stale=None, write_unresolved=True):
    """Run the unpack model over the grid the launcher would use.  D: dict with N, T, H, E, R, B,
    fp8, rb, rc.  Buffers are numpy arrays laid out as on the device ([N][B][...]); recv_buf and
    expert_x as bytes per row.  stride_blocks: a capped grid whose blocks stride over the rows.
    stale: the words a block's LDS holds before the kernel writes it (another block's leftovers).
    write_unresolved False: a wave whose row lies past the total leaves its descriptor as it was."""
    N, T, H, E, R, B = D["N"], D["T"], D["H"], D["E"], D["R"], D["B"]
    rb, rc, fp8 = D["rb"], D["rc"], D["fp8"]
    L, TR = E // N, T * R
    P = H + H // 32 if fp8 else 2 * H
    P16, X16 = P // 16, (H if fp8 else 2 * H) // 16
    xrow = H if fp8 else 2 * H
    nsc = H // 128
    S16 = nsc * 4 // 16
    rbuf = recv_buf.view(np.uint8).reshape(N * B, P)
    xbuf = expert_x.view(np.uint8).reshape(N * B, xrow)
    sbuf = expert_scale.view(np.uint8).reshape(N * B, nsc * 4) if fp8 else None
    # per-rank receive totals -> the bound the launcher sizes the grid for
    per_rank = N * T * min(R, L)
    rows_bound = min(rc * per_rank, N * TR)
    blocks = max((rows_bound + rpb - 1) // rpb, rc)
    strided = stride_blocks is not None and blocks > stride_blocks
    if strided:
        blocks = stride_blocks
    if stale is None:
        stale = np.zeros(0, np.int64)
    stats = {"rows": 0, "blocks": blocks, "overruns": 0}
    for blk in range(blocks):
        lds = Lds(rpb, rc, stale)
        # rank bases over the call's ranks (wave 0)
        carry = 0
        for i in range(rc):
            lds.set_gb(i, carry)
            carry += int(recv_off[rb + i, N])
        lds.set_gb(rc, carry)
        total = lds.gb(rc)
        bases = range(blk * rpb, total, blocks * rpb) if strided else [blk * rpb]
        for base in bases:
            # each wave resolves its rows and writes their descriptors
            for w in range(WAVES):
                for j in range(rows_per_wave):
                    slot = w + WAVES * j
                    if check_slot and slot >= rpb:
                        continue
                    G = base + slot
                    desc = [0, 0, 0, 0]
                    if G < total:
                        dl = sum(1 for i in range(1, rc + 1) if lds.gb(i) <= G)
                        d = rb + dl
                        r = G - lds.gb(min(dl, rc))
                        _check(dl < rc and 0 <= d < N,
                               f"row {G}: rank index {dl} past the {rc} ranks of the table: the kernel "
                               f"reads receive offsets of rank {d} (the table has {N}) and receive row "
                               f"{d * B + r} (the buffers have {N * B})")
                        s = sum(1 for k in range(N) if recv_off[d, k] <= r) - 1
                        rrow = d * B + r
                        _check(0 <= rrow < N * B, f"row {G}: receive row {rrow}")
                        mx, my = int(recv_meta.reshape(N * B, 2)[rrow, 0]), int(recv_meta.reshape(N * B, 2)[rrow, 1])
                        e = mx // TR
                        i_ = mx - e * TR
                        jl = e - d * L
                        q = -1
                        if 0 <= jl < L and s >= 0:
                            base_q = 0
                            for sp in range(N):
                                for jj in range(jl + 1):
                                    _check(0 <= sp * E + d * L + jj < N * E, "counts index")
                                    if jj < jl or sp < s:
                                        base_q += int(counts[sp, d * L + jj])
                            q = base_q + my
                        if 0 <= q < B:
                            qrow = d * B + q
                            expert_src.reshape(-1)[qrow] = s * TR + i_
                            expert_rpos.reshape(-1)[qrow] = r
                            desc = [rrow + 1, rrow + 1, qrow + 1, qrow + 1]  # +1: 0 marks "no row"
                        else:
                            raise Violation(f"row {G}: expert-major position {q} outside {B}")
                    elif not write_unresolved:
                        continue
                    lds.write_desc(slot, desc)
            # the block streams its rows' chunks, U per thread per pass
            n16 = P16
            total_chunks = rpb * n16
            inv = np.float32(1.0) / np.float32(n16)
            for t in range(THREADS):
                for k0 in range(t, total_chunks, THREADS * u):
                    for uu in range(u):
                        k = k0 + uu * THREADS
                        kc = k if k < total_chunks else total_chunks - 1
                        r = int(np.float32(kc) * inv)
                        if r * n16 > kc:
                            r -= 1
                        elif (r + 1) * n16 <= kc:
                            r += 1
                        dsc = lds.read_desc(r)
                        c = kc - r * n16
                        _check(0 <= c < n16, f"chunk {c} of a {n16}-chunk row")
                        live = k < total_chunks and dsc[2] != 0
                        if not live:
                            continue  # the load reads chunk c of the source's first row: in bounds
                        srow = dsc[0] - 1
                        _check(0 <= srow < N * B, f"source row {srow}")
                        qrow = dsc[2] - 1
                        _check(0 <= qrow < N * B, f"destination row {qrow}")
                        chunk = rbuf[srow, c * 16:(c + 1) * 16]
                        if c < X16:
                            xbuf[qrow, c * 16:(c + 1) * 16] = chunk
                        else:
                            cs = c - X16
                            _check(0 <= cs < S16, f"scale chunk {cs} of {S16}")
                            sbuf[qrow, cs * 16:(cs + 1) * 16] = chunk
                        stats["rows"] += 1 if c == 0 else 0
        stats["overruns"] += lds.overruns
    return stats
