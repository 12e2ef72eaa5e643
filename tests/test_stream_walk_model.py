"""The decode walk's two cursors and pool tickets, as a CPU model (host logic).

`decode_stream` in csrc/kvc_kernels.hip walks each wave's main chunk and then
the pool pieces it wins, with a prefetch cursor PF + 1 blocks ahead of the
process cursor.  Its correctness rests on a protocol the kernel cannot check at
run time: a ticket is requested at the head of the turn before the prefetch
cursor reaches its range's end and read at the next head; pieces are at least
two turns long, so one pending range is handed between the cursors; chunk ids
follow the list order.  This model steps the same control flow (ring of TURN
slots, turn heads, range entry, segment begin/finish, per-range chunk records)
for many waves under random interleavings and asserts what the kernel relies
on: every block is walked exactly once, by the process cursor, with the chunk id
the merge expects; no pending range is overwritten; every query is loaded
before its segment starts; the per-sequence records name exactly the chunks
holding the sequence; and every partial slot the merge reads for a sequence
(slots b + c for its recorded chunks c) is written by the same call, exactly
once, while a sequence held by one chunk gets its output written by the walk
and nothing read by the merge.  The GPU parity tests check the kernel itself.
"""
import random

import pytest


def wave_first_block(w, total, W): return (w * total + W - 1) // W

class Geo:
    def __init__(s, total, W, KP, shift): s.total, s.W, s.KP, s.shift = total, W, KP, shift
    def wave_range(s, ww):
        r0 = wave_first_block(ww, s.total, s.W); r1 = wave_first_block(ww + 1, s.total, s.W)
        rm = r1 - ((r1 - r0) >> s.shift) if s.KP else r1
        return r0, r1, rm
    def chunk_of_block(s, y):
        ww = y * s.W // s.total
        r0, r1, rm = s.wave_range(ww)
        if y < rm: return ww * (s.KP + 1)
        return ww * (s.KP + 1) + 1 + (y - rm) * s.KP // (r1 - rm)
    def piece(s, t):
        ww, j = divmod(t, s.KP)
        r0, r1, rm = s.wave_range(ww)
        ln = r1 - rm
        return rm + (j * ln + s.KP - 1) // s.KP, rm + ((j + 1) * ln + s.KP - 1) // s.KP, ww * (s.KP + 1) + 1 + j

def run(seq_blocks, W_req, PF, pool_pieces, shift, rng, min_piece_turns=2, plant_whole_tail=False):
    TURN = PF + 1
    seq_start = [0]
    for nbk in seq_blocks: seq_start.append(seq_start[-1] + nbk)
    batch = len(seq_blocks); total = seq_start[-1]
    if total == 0: return
    W = min(W_req, total)
    KP = pool_pieces if (pool_pieces > 0 and shift >= 1 and ((total // W) >> shift) >= pool_pieces * min_piece_turns * TURN) else 0
    geo = Geo(total, W, KP, shift)
    counter = [0]
    processed = {}   # block -> chunk id
    seginfo = {}
    partials = {}    # (sequence, chunk id) -> times the walk wrote that partial slot
    outputs = {}     # sequence -> times the walk wrote its output directly
    def seq_holding(x):
        lo, hi = 0, batch - 1
        while lo < hi:
            mid = (lo + hi + 1) >> 1
            if seq_start[mid] <= x: lo = mid
            else: hi = mid - 1
        return lo
    def next_seq(bb, x):
        while True:
            bb += 1
            if not (seq_start[bb + 1] <= x): return bb
    def wave(w):
        st = {}
        xa, _, xb_main = geo.wave_range(w)
        b = seq_holding(xa)
        P = dict(b=b, xp=xa, xbp=xb_main, c=w * (KP + 1), sb=0, eb=0, x0=0, seg_end=0, nb_q=-1, proc_last=False,
                 p_valid=False, p=None, q=None, q_next=None)
        F = dict(xf=xa, xbf=xb_main, bf=b, ebf=seq_start[b + 1], ph_last=None, left=0, more=KP != 0,
                 req_out=False, have_next=False, nxt=None, ticket=None)
        def begin(x):
            b = P['b']; P['sb'] = seq_start[b]; P['eb'] = seq_start[b + 1]; P['x0'] = x
            P['seg_end'] = min(P['eb'], P['xbp'])
            P['proc_last'] = P['seg_end'] == P['xbp']
            if not P['proc_last']:
                P['nb_q'] = next_seq(b, P['seg_end']); P['q_next'] = P['nb_q']
            elif P['p_valid']:
                P['q_next'] = P['p'][3]
        def record_range(ra, rb, cc):
            b0 = seq_holding(ra)
            if seq_start[b0] < ra: b0 += 1
            for bb in range(b0, batch):
                if seq_start[bb] >= rb: break
                if seq_start[bb + 1] > seq_start[bb]:
                    assert bb not in seginfo
                    seginfo[bb] = (cc, geo.chunk_of_block(seq_start[bb + 1] - 1) - cc + 1)
        def finish():
            # the segment's result: the output when it is the whole sequence,
            # else the partial of (sequence, chunk)
            if (plant_whole_tail or P['x0'] == P['sb']) and P['seg_end'] == P['eb']:
                outputs[P['b']] = outputs.get(P['b'], 0) + 1
            else:
                key = (P['b'], P['c'])
                partials[key] = partials.get(key, 0) + 1
            if P['proc_last']:
                if not P['p_valid']: return
                P['p_valid'] = False
                pa, pb, pc, pbq = P['p']
                P['nb_q'] = pbq; P['xp'] = pa; P['xbp'] = pb; P['c'] = pc
            P['b'] = P['nb_q']; assert P['q_next'] == P['b'], "query not loaded"
            P['q'] = P['q_next']; begin(P['xp'])
        def next_phys():
            if F['xf'] == F['xbf'] and F['have_next']:
                F['have_next'] = False
                na, nb, nc = F['nxt']
                F['xf'] = na; F['xbf'] = nb; F['bf'] = seq_holding(na); F['ebf'] = seq_start[F['bf'] + 1]
                assert not P['p_valid'], "pending range overwritten"
                P['p_valid'] = True; P['p'] = (na, nb, nc, F['bf'])
                if P['proc_last']: P['q_next'] = F['bf']
            if F['xf'] < F['xbf']:
                if F['xf'] == F['ebf']:
                    F['bf'] = next_seq(F['bf'], F['xf']); F['ebf'] = seq_start[F['bf'] + 1]
                assert seq_start[F['bf']] <= F['xf'] < seq_start[F['bf'] + 1]
                F['ph_last'] = F['xf']; F['xf'] += 1; F['left'] += 1
                return (F['ph_last'], True)
            return (F['ph_last'], False)
        def process(blk):
            ph, real = blk
            assert real and ph == P['xp'], f"process got {blk}, expected block {P['xp']}"
            assert seq_start[P['b']] <= P['xp'] < seq_start[P['b'] + 1] and P['q'] == P['b']
            assert P['xp'] not in processed, f"block {P['xp']} twice"
            processed[P['xp']] = P['c']
            P['xp'] += 1; F['left'] -= 1
            if P['xp'] == P['seg_end']: finish()
        record_range(xa, xb_main, P['c'])
        P['q'] = b; begin(xa)
        buf = [None] * TURN
        for j in range(PF): buf[j] = next_phys()
        ph_next = next_phys()
        while F['left'] >= TURN:
            if F['req_out'] and F['xbf'] - F['xf'] <= PF:
                yield  # the ticket's answer: other waves may have run meanwhile
                t = F['ticket']; F['req_out'] = False
                if t < W * KP:
                    F['nxt'] = geo.piece(t); F['have_next'] = True; record_range(*F['nxt'])
                else: F['more'] = False
            if F['more'] and not F['req_out'] and not F['have_next'] and PF < F['xbf'] - F['xf'] <= PF + TURN:
                F['ticket'] = counter[0]; counter[0] += 1; F['req_out'] = True
            for j in range(TURN):
                ph = ph_next; ph_next = next_phys()
                buf[(j + PF) % TURN] = ph
                process(buf[j])
            yield
        rest = F['left']
        for j in range(PF):
            if j >= rest: break
            ph = ph_next; ph_next = next_phys(); buf[(j + PF) % TURN] = ph; process(buf[j])
        assert F['left'] == 0
    gens = [wave(w) for w in range(W)]
    live = list(range(W))
    while live:
        i = rng.choice(live)
        try: next(gens[i])
        except StopIteration: live.remove(i)
    assert sorted(processed) == list(range(total)), f"missing {set(range(total)) - set(processed)}"
    for y, c in processed.items(): assert c == geo.chunk_of_block(y), (y, c, geo.chunk_of_block(y))
    for b in range(batch):
        if seq_blocks[b] == 0: continue
        c0, cnt = seginfo[b]
        chunks = sorted({processed[y] for y in range(seq_start[b], seq_start[b + 1])})
        assert chunks == list(range(c0, c0 + cnt)), (b, chunks, c0, cnt)
        # what the merge reads for b was written by this call, once
        if cnt <= 1:
            assert outputs.get(b) == 1 and not any(k[0] == b for k in partials), (b, outputs.get(b))
        else:
            assert b not in outputs, ("a split sequence's output written by the walk", b)
            for c in range(c0, c0 + cnt):
                assert partials.get((b, c)) == 1, ("merge reads an unwritten or twice-written slot", b, c)
    assert all(v == 1 for v in partials.values())
    assert sum(1 for b in range(batch) if seq_blocks[b]) == len({k[0] for k in partials} | set(outputs))
    return KP



@pytest.mark.parametrize("seed", range(4))
def test_walk_covers_every_block_once(seed):
    rng = random.Random(seed)
    used = 0
    for _ in range(400):
        nb = rng.randint(1, 12)
        seq_blocks = [rng.choice([0, 1, 2, rng.randint(1, 30), rng.randint(10, 400)]) for _ in range(nb)]
        W = rng.choice([1, 2, 3, 5, 8, 16, 40, 64])
        PF = rng.choice([3, 4])
        pieces = rng.choice([0, 1, 2, 3, 5, 8])
        shift = rng.choice([1, 2, 3])
        used += bool(run(seq_blocks, W, PF, pieces, shift, rng))
    assert used > 40   # the pool took part in a fair share of the trials


def test_planted_short_piece_is_caught():
    # pieces shorter than a turn break the one-pending-range hand-off; the
    # model must notice (the kernel's size test keeps them out)
    rng = random.Random(7)
    with pytest.raises(AssertionError):
        for _ in range(300):
            run([rng.randint(20, 300) for _ in range(6)], rng.choice([2, 4, 8]), 4, rng.choice([4, 8]), 1, rng,
                min_piece_turns=0)


@pytest.mark.parametrize("W,KP", [(1, 1), (2, 1), (1, 3), (3, 1)])
def test_one_byte_ring_single_wave_pool(W, KP):
    # the one-byte decode's deeper ring (PF 6, turns of 7 blocks) with a
    # single wave or a single pool piece per wave: the wave's own pool piece
    # comes back through its own ticket, read a turn late; tickets arrive in
    # random order relative to the other waves' progress
    rng = random.Random(100 * W + KP)
    engaged = 0
    for _ in range(150):
        nb = rng.randint(1, 8)
        seq_blocks = [rng.choice([0, 1, rng.randint(1, 40), rng.randint(60, 500)]) for _ in range(nb)]
        engaged += bool(run(seq_blocks, W, 6, KP, rng.choice([1, 2]), rng))
    assert engaged > 20


def test_planted_unwritten_merge_slot_is_caught():
    # a walk that takes a split sequence's last segment for the whole
    # sequence writes the output there instead of its partial, so the merge
    # would read a slot this call never wrote: the check must fail
    rng = random.Random(3)
    with pytest.raises(AssertionError, match="unwritten|written by the walk"):
        for _ in range(50):
            run([rng.randint(30, 200) for _ in range(3)], 4, 6, 0, 1, rng, plant_whole_tail=True)
