"""CPU model of the grouped GEMM's token-row ring (ffn_gemm.hip).

Token rows are staged a whole 128-byte line (64 k) per load: stream stage s
loads half s % 2 of the rows of the stage pair (s & ~1, s | 1) into token slot
s % GTST, GTST - 1 stages ahead of the step that multiplies stage s.  This
model replays the schedule the kernel runs (the DMA addresses and LDS offsets
of every lane, the fragment reads of every wave and lane, the per-step vmcnt
waits) and checks that every fragment read sees the token row and k it must,
that every load it needs has landed by the wait before its read, that no slot
is refilled before the last read of what it holds, and that the slot the
tile's last stage stages its bf16 output through has no load pending.  It
models the kernel's index arithmetic; the GPU parity tests run the kernel.
"""
import itertools

import pytest

GTST, NQ = 5, 4          # token ring depth, DMA instructions per wave per stage
LEAD = GTST - 1          # a token wave loads stream stage s + LEAD at step s


def _schedule(nst, n_my):
    S = n_my * nst

    def stream(q):        # stream stage -> (tile, k stage); past the end: the last again
        return (q // nst, q % nst) if q < S else (n_my - 1, nst - 1)

    lds, issued = {}, []

    def issue(q):
        j, ks = stream(q)
        h = ks & 1                               # half of the pair = stage parity
        for w, qi, lane in itertools.product(range(4), range(NQ), range(64)):
            row = 128 * h + 32 * w + 8 * qi + (lane >> 3)
            c8 = (lane & 7) ^ ((lane >> 3) & 7)  # slot lane % 8 holds chunk c8
            k0 = (ks - h) * 32 + 8 * c8
            assert 0 <= k0 and k0 + 8 <= nst * 32
            off = (32 * w + 8 * qi) * 128 + 16 * lane
            assert off + 16 <= 16384
            lds[(q % GTST, off)] = (j, row, k0, q)
        issued.append(q)

    def landed(par):
        pend = GTST - 3 - par                   # loads still pending after the wait
        return set(issued[:len(issued) - pend])

    def reads(st, ok, staged=None):
        j, ks = stream(st)
        for wn, jj, lane in itertools.product(range(4), range(4), range(64)):
            r16, kg = lane & 15, lane >> 4
            slot = ((st & ~1) + (wn >> 1)) % GTST
            assert slot != staged
            lo = r16 * 128 + ((kg ^ (r16 & 7)) * 16)
            addr = (wn & 1) * 64 * 128 + (lo ^ ((st & 1) << 6)) + jj * 2048
            got = lds[(slot, addr)]
            assert got[:3] == (j, wn * 64 + 16 * jj + r16, ks * 32 + 8 * kg)
            assert got[3] in ok

    for q in range(LEAD):                       # prologue: wait for pair 0, read stage 0
        issue(q)
    reads(0, landed(0))
    for st in range(S):
        par = st & 1
        ok = landed(par)                        # wait + barrier of step st
        q, slot = st + LEAD, (st + LEAD) % GTST
        for (s_, _), v in list(lds.items()):    # the refilled slot's last reader is done
            if s_ == slot:
                assert 2 * (v[3] >> 1) < st
        last = st % nst == nst - 1
        issue(q)
        staged = None
        if last:                                # the epilogue stages through slot st % GTST
            staged = st % GTST
            assert all(x % GTST != staged for x in issued[-(GTST - 3 - par) - 1:])
        if st + 1 < S:
            reads(st + 1, ok, staged)


@pytest.mark.parametrize("nst,n_my", [(2, 1), (4, 3), (16, 4), (48, 3), (40, 2), (6, 5)])
def test_token_pair_ring(nst, n_my):
    _schedule(nst, n_my)
