"""Host models of the GPU kernels' lane maps and LDS schedules (no GPU).

These check properties of index maps that the HIP sources compute, the way a
reviewer would check them by hand: every element of a staged step lands in
exactly one LDS slot and is read back by the lane that the matrix
instruction's operand layout expects; the reads of one LDS pass fall on
distinct banks; and the step pipelines never overwrite a buffer another wave
may still read, nor read one whose loads have not been waited for. The maps
below restate the kernels' formulas (pda_prefill_mfma.h, pda_decode_mfma.h);
a change there must be mirrored here, and the properties re-proved.

LDS is modelled as 64 banks of 4 bytes; a 16-byte read (ds_read_b128) is
served 16 lanes per pass, an 8-byte read (ds_read_b64_tr_b16) 32 lanes per
pass.
"""

import itertools

import pytest

BANKS = 64


def banks_of(addr: int, nbytes: int) -> set:
    return {((addr + b) // 4) % BANKS for b in range(0, nbytes, 4)}


def conflict_free(addrs, nbytes, lanes_per_pass):
    for p in range(0, len(addrs), lanes_per_pass):
        seen = set()
        for a in addrs[p:p + lanes_per_pass]:
            b = banks_of(a, nbytes)
            if seen & b:
                return False
            seen |= b
    return True


# ---- prefill kernel: one 64-key step of K and V in LDS (fp16) ----

def prefill_geometry(D, waves):
    NK = D // 16                 # K blocks (16-dim k-steps) per 32-key half
    NDV = D // 32                # V blocks (32 dims) per 16-key tile
    KH = NK * 1024               # bytes of K of one half
    VT = NDV * 1024              # bytes of V of one tile
    PER = 2 * NK // (waves // 2)  # 1 KB loads per wave and step
    return NK, NDV, KH, VT, PER


def prefill_dma_writes(D, waves):
    """(lds byte offset in the step buffer) -> ('K' or 'V', key, first dim)
    for every lane of every direct load of one step, as the kernel issues
    them (K waves: wave < waves / 2)."""
    NK, NDV, KH, VT, PER = prefill_geometry(D, waves)
    out = {}
    for wave in range(waves):
        kwave = wave < waves // 2
        wk = wave if kwave else wave - waves // 2
        ta = 2 * ((wk * PER) // NK) if kwave else (wk * PER) // NDV
        for lane in range(64):
            if kwave:
                t0 = (wk * PER) % NK
                tile = ta + ((lane >> 4) & 1)
                row = lane & 15
                for i in range(PER):
                    byte_in_row = 32 * (t0 + i) + 16 * (lane >> 5)
                    dst = (ta // 2) * KH + (t0 + i) * 1024 + 16 * lane
                    assert dst not in out
                    out[dst] = ("K", 16 * tile + row, byte_in_row // 2)
            else:
                vrow = 8 * (lane >> 5) + 4 * ((lane >> 4) & 1) + ((lane >> 2) & 3)
                for q in range(PER // NDV):
                    for dg in range(NDV):
                        byte_in_row = 64 * dg + 16 * (lane & 3)
                        dst = 2 * KH + (ta + q) * VT + dg * 1024 + 16 * lane
                        assert dst not in out
                        out[dst] = ("V", 16 * (ta + q) + vrow, byte_in_row // 2)
    return out


@pytest.mark.parametrize("D,waves", [(128, 8), (128, 4), (256, 8), (256, 4)])
def test_prefill_step_is_covered_once(D, waves):
    """Every 16-byte piece of the step's 64 K rows and 64 V rows is loaded
    into exactly one slot, and the slots tile the buffer."""
    NK, NDV, KH, VT, PER = prefill_geometry(D, waves)
    w = prefill_dma_writes(D, waves)
    assert sorted(w) == list(range(0, 2 * KH + 4 * VT, 16))
    pieces = set(w.values())
    assert len(pieces) == len(w)
    want = {(kv, key, d) for kv in "KV" for key in range(64) for d in range(0, D, 8)}
    assert pieces == want


@pytest.mark.parametrize("D,waves", [(128, 8), (256, 8)])
def test_prefill_k_fragments_are_the_mfma_a_operand(D, waves):
    """Lane l's 16-byte read at k-step t of half h holds key 32 h + l % 32,
    dims 16 t + 8 (l / 32) .. + 7: the A fragment of v_mfma_f32_32x32x16_f16
    (row l % 32, k = 8 (l / 32) .. + 7)."""
    NK, NDV, KH, VT, PER = prefill_geometry(D, waves)
    w = prefill_dma_writes(D, waves)
    for h in range(2):
        for t in range(NK):
            addrs = [h * KH + 1024 * t + 16 * lane for lane in range(64)]
            for lane, a in enumerate(addrs):
                assert w[a] == ("K", 32 * h + lane % 32, 16 * t + 8 * (lane // 32))
            assert conflict_free(addrs, 16, 16)


@pytest.mark.parametrize("D,pair", [(128, False), (256, True)])
def test_prefill_v_transposing_reads(D, pair):
    """The transposing reads of tile 2 h + ks, dims dcol + 32 dt: lane
    (hh, q16, i16) reads 8 bytes that must hold V[key 16 (2h + ks) + 8 hi +
    4 hh + i16 / 4][dims dcol + 32 dt + 16 (q16 % 2) + 4 (i16 % 4) .. + 3],
    the elements a row-major V tile gave the same lane (so the transposing
    read still hands the MFMA its V^T operand). Both 32-lane passes are
    conflict-free."""
    NK, NDV, KH, VT, PER = prefill_geometry(D, 8)
    w = prefill_dma_writes(D, 8)
    NDT = (D // 2 if pair else D) // 32
    for dh in (range(2) if pair else [0]):
        dcol = dh * (D // 2)
        for h, ks, dt, hi in itertools.product(range(2), range(2), range(NDT), range(2)):
            addrs = []
            for lane in range(64):
                hh, q16, i16 = lane >> 5, lane >> 4, lane & 15
                v_lane = 16 * (16 * hh + 4 * (i16 >> 2) + 2 * (q16 & 1) + ((i16 & 3) >> 1)) + 8 * (i16 & 1)
                a = 2 * KH + (2 * h + ks) * VT + (dcol // 32 + dt) * 1024 + 512 * hi + v_lane
                addrs.append(a)
                slot, half = a - (a % 16), (a % 16) // 2   # which 16-byte slot, which 4-dim half
                kv, key, d0 = w[slot]
                assert kv == "V"
                assert key == 16 * (2 * h + ks) + 8 * hi + 4 * hh + (i16 >> 2)
                assert d0 + half == dcol + 32 * dt + 16 * (q16 & 1) + 4 * (i16 & 3)
            assert conflict_free(addrs, 8, 32)


# ---- prefill pipeline: buffers, waits and barriers ----

def simulate_prefill_pipeline(nbuf, n_steps, per=4):
    """The fp16 step loop: steps 0 .. nbuf - 2 are issued before the loop;
    step s computes on buffer s % nbuf and first issues the loads of step
    s + nbuf - 1 (into the buffer step s - 1 used); its end waits for step
    s + 1 with the issued steps after it (at most two) in flight (vmcnt of
    their loads), then a barrier. Returns the events for the checks."""
    issued = []             # order of issue: (step, buffer)
    waits = []              # (loads issued so far, allowed outstanding, step needed)
    events = []             # ('issue', step, buf, epoch) / ('read', step, buf, epoch)
    epoch = 0               # barriers passed

    def allowed(need, issued_to):
        after = min(issued_to, n_steps - 1) - need
        return per * min(max(after, 0), 2)

    for j in range(min(nbuf - 1, n_steps)):
        issued.append((j, j % nbuf))
        events.append(("issue", j, j % nbuf, epoch))
    waits.append((len(issued), allowed(0, nbuf - 2), 0))
    epoch += 1
    for s in range(n_steps):
        j = s + nbuf - 1
        if j < n_steps:
            issued.append((j, j % nbuf))
            events.append(("issue", j, j % nbuf, epoch))
        events.append(("read", s, s % nbuf, epoch))
        if s + 1 < n_steps:
            waits.append((len(issued), allowed(s + 1, s + nbuf - 1), s + 1))
            epoch += 1
    return issued, waits, events


@pytest.mark.parametrize("nbuf", [2, 3, 4])
@pytest.mark.parametrize("n_steps", range(1, 10))
def test_prefill_pipeline_is_race_free(nbuf, n_steps):
    per = 4
    issued, waits, events = simulate_prefill_pipeline(nbuf, n_steps, per)
    assert sorted(s for s, _ in issued) == list(range(n_steps))
    # Each wait before the barrier that precedes step s's reads leaves at
    # most `allowed` loads in flight; loads complete in issue order, so the
    # loads of step s (each wave's per of them) are complete exactly when
    # no more than the loads issued after them may stay outstanding.
    for n_issued, allowed, s in waits:
        last_of_s = max(i for i, (j, _) in enumerate(issued) if j == s) + 1
        assert allowed <= (n_issued - last_of_s) * per, (s, allowed)
        assert allowed == (n_issued - last_of_s) * per or allowed == 2 * per
    # A load into a buffer is issued in a later barrier epoch than every read
    # of the step that buffer held before.
    for kind, j, b, ep in events:
        if kind != "issue":
            continue
        for kind2, s2, b2, ep2 in events:
            if kind2 == "read" and b2 == b and s2 < j:
                assert ep2 < ep, (j, s2, b)
    # Every read happens in an epoch after its step's load was issued and waited.
    for kind, s, b, ep in events:
        if kind == "read":
            issue_ep = next(e for k, j, _, e in events if k == "issue" and j == s)
            assert issue_ep < ep


@pytest.mark.parametrize("mistake", ["load_one_step_further", "skip_a_wait"])
def test_prefill_pipeline_model_catches_planted_mistakes(mistake):
    """The checks above fail on a schedule that loads into the buffer the
    current step reads, or that waits too little."""
    nbuf, n_steps, per = 3, 6, 4
    issued, waits, events = simulate_prefill_pipeline(nbuf, n_steps, per)
    if mistake == "load_one_step_further":
        # step s loads step s + nbuf into buffer s % nbuf, read by step s itself
        events = [("issue", j + 1, (j + 1) % nbuf, ep) if k == "issue" and ep > 0 else (k, j, b, ep)
                  for k, j, b, ep in events]
        bad = any(k == "issue" and any(k2 == "read" and b2 == b and s2 < j and ep2 >= ep
                                       for k2, s2, b2, ep2 in events)
                  for k, j, b, ep in events)
        assert bad
    else:
        n_issued, allowed, s = waits[1]
        last_of_s = max(i for i, (j, _) in enumerate(issued) if j == s) + 1
        assert allowed + per > (n_issued - last_of_s) * per


@pytest.mark.parametrize("D,pair", [(128, False), (256, True)])
def test_prefill_q_staging(D, pair):
    """Q through LDS (fp16 KV): a row block's 32 rows of 2 D bytes, row after
    row; 1 KB direct load k of a wave (lane l lands at 16 l) covers rows r0 +
    k * RPL + l / SPR, piece slot l % SPR, and fetches the row's 16-byte piece
    slot ^ (row % 16) (r0 = 0, or 16 dh for the D=256 pairs, whose two waves
    load half the rows each). Every piece of every row is staged exactly once,
    lane (rr = l % 32, hh = l / 32) reads back the B operand of k-step t
    (row rr, dims 16 t + 8 hh ..) from slot (2 t + hh) ^ (rr % 16), and a
    16-lane read pass is conflict-free."""
    RB = 2 * D
    RPL, SPR = 1024 // RB, RB // 16
    waves = (0, 1) if pair else (0,)
    held = {}  # LDS byte offset in the row block -> (row, piece)
    for dh in waves:
        r0 = 16 * dh if pair else 0
        for k in range(8):
            for lane in range(64):
                r, sl = r0 + k * RPL + lane // SPR, lane % SPR
                dst = (r0 + k * RPL) * RB + 16 * lane
                assert dst == r * RB + 16 * sl
                assert dst not in held
                held[dst] = (r, sl ^ (r % 16))
    assert sorted(held.values()) == [(r, c) for r in range(32) for c in range(SPR)]
    for t in range(D // 16):
        addrs = []
        for lane in range(64):
            rr, hh = lane % 32, lane // 32
            a = rr * RB + 16 * ((2 * t + hh) ^ (rr % 16))
            assert held[a] == (rr, 2 * t + hh)
            addrs.append(a)
        assert conflict_free(addrs, 16, 16)


def test_prefill_out_tile_swizzle():
    """The output tile of a wave: 32 rows of 256 bytes; lane l's 8-byte
    piece (dims 32 dt + 8 j + 4 hh .. + 3 of row rr = l % 32, hh = l / 32)
    goes to piece (4 dt + j) ^ (rr % 16) of the row, half hh ^ (rr / 16); the
    reads take 16-byte piece pc = l % 16 of row r = (64 p + l) / 16 from piece
    pc ^ (r % 16), halves swapped back when r >= 16 (p >= 4). Every byte is
    written once, each read returns the 8 dims it names in order, and the
    writes (32 lanes a pass) and reads (16 a pass) are conflict-free."""
    RS = 256
    slot = {}
    for dt in range(4):
        for j in range(4):
            addrs = []
            for lane in range(64):
                rr, hh = lane % 32, lane // 32
                a = rr * RS + 16 * ((4 * dt + j) ^ (rr % 16)) + 8 * (hh ^ (rr // 16))
                addrs.append(a)
                assert a not in slot
                slot[a] = (rr, 32 * dt + 8 * j + 4 * hh)
            assert conflict_free(addrs, 8, 32)
    assert sorted(slot) == list(range(0, 32 * RS, 8))
    for p in range(8):
        addrs = []
        for lane in range(64):
            r, pc = (64 * p + lane) // 16, lane % 16
            a = r * RS + 16 * (pc ^ (r % 16))
            addrs.append(a)
            lo, hi = (a + 8, a) if p >= 4 else (a, a + 8)
            assert slot[lo] == (r, 8 * pc) and slot[hi] == (r, 8 * pc + 4)
        assert conflict_free(addrs, 16, 16)


# ---- decode kernel: the wave-private V tile and its transposing reads ----

@pytest.mark.parametrize("D", [128, 256])
def test_decode_v_tile_reads_are_conflict_free(D):
    """The matrix decode kernel's V tile has rows of D + 16 halves; lane
    (s, c) of a transposing read points at row 4 s + c / 4, dims 16 dt +
    4 (c % 4): each 32-lane pass (8 rows x 32 bytes) falls on distinct banks
    (with D + 8 they overlap 2-way)."""
    def addrs(lr):
        out = []
        for dt in range(D // 16):
            out.append([2 * ((4 * (lane >> 4) + ((lane & 15) >> 2)) * lr + 16 * dt + 4 * (lane & 3))
                        for lane in range(64)])
        return out
    assert all(conflict_free(a, 8, 32) for a in addrs(D + 16))
    assert not all(conflict_free(a, 8, 32) for a in addrs(D + 8))


# ---- prefill at D=256: the pairs' score exchange ----

def test_prefill_pair_score_exchange():
    """Waves 2 r and 2 r + 1 of an 8-wave D=256 workgroup share the row
    block r and compute opposite 32-key halves, and sit on different SIMDs
    (waves w and w + 4 share one); wave w writes its 16 scores per lane to
    its own 4 KB (float 4 c + e of lane l at 1024 c + 16 l + 4 e) and reads
    its partner's at the same offsets: every float is read by the lane of
    the same row (the MFMA C layout puts row l % 32 in lane l), no two waves
    write the same byte, each 16-lane pass of the 16-byte accesses is
    conflict-free, and the region fits after the two 64 KB step buffers in
    the 160 KB of LDS."""
    waves, step_bytes, nbuf = 8, 2 * 4 * 16 * 256 * 2, 2
    base = nbuf * step_bytes
    written = {}
    for w in range(waves):
        for lane in range(64):
            for c in range(4):
                for e in range(4):
                    a = base + w * 4096 + 1024 * c + 16 * lane + 4 * e
                    assert a not in written
                    written[a] = (w, lane, 4 * c + e)
    for w in range(waves):
        p = w ^ 1
        assert p >> 1 == w >> 1 and (p & 1) != (w & 1) and p % 4 != w % 4
        for lane in range(64):
            for c in range(4):
                for e in range(4):
                    src_w, src_lane, idx = written[base + p * 4096 + 1024 * c + 16 * lane + 4 * e]
                    assert (src_w, src_lane % 32, idx) == (p, lane % 32, 4 * c + e)
        for c in range(4):
            assert conflict_free([base + w * 4096 + 1024 * c + 16 * lane for lane in range(64)], 16, 16)
    assert max(written) < 160 * 1024 and base + waves * 4096 == 160 * 1024


def pair_exchange_reads(active, tag_of):
    """The pair handshake over a run of steps: the writer's block starts
    tagged 1; at each step both waves of the pair compute or both skip
    (same rows); a computing wave writes all its words with tag_of(k, step)
    (k: steps computed so far) and accepts the partner's words once they
    carry that tag. Returns, per computing step, the step whose data a
    reader polling right away (before the partner's write lands) would
    accept: None when it would wait, as it must."""
    block = ("init", 1)  # (step written, tag)
    accepted = []
    k = 0
    for step, act in enumerate(active):
        if not act:
            continue
        tag = tag_of(k, step)
        accepted.append(block[0] if block[1] == tag else None)
        block = (step, tag)  # the partner's write lands
        k += 1
    return accepted


@pytest.mark.parametrize("pattern", ["all", "gap", "gaps", "late"])
def test_prefill_pair_handshake_never_takes_old_scores(pattern):
    """With the tag = parity of the count of computed steps, a reader never
    accepts a block left from an earlier step, whatever steps the pair skips;
    a tag from the step index (planted mistake) does, after a skipped step."""
    active = {"all": [1] * 8, "gap": [1, 1, 0, 1, 1], "gaps": [1, 0, 1, 0, 0, 1, 1, 0, 1],
              "late": [0, 0, 0, 1, 1, 1]}[pattern]
    assert all(a is None for a in pair_exchange_reads(active, lambda k, step: k & 1))
    wrong = pair_exchange_reads(active, lambda k, step: step & 1)
    assert all(a is None for a in wrong) == (pattern == "all")


# ---- prefill at D=128: persistent workgroups' item order ----

def persistent_slots(P, n):
    """The slots workgroup b of a grid of P takes, round by round, as the
    prefill kernel's item loop computes them (snake order within each XCD's
    workgroups when P is a multiple of 8, else one slot per workgroup)."""
    per = P >> 3
    out = {}
    for blk in range(P):
        x8, j8 = blk & 7, blk >> 3
        r, mine = 0, []
        while True:
            v = blk + r * P if (P & 7) else 8 * (r * per + ((per - 1 - j8) if (r & 1) else j8)) + x8
            if v >= n:
                break
            mine.append(v)
            r += 1
        out[blk] = mine
    return out


def slot_item(v, n):
    xcd, k = v & 7, v >> 3
    return xcd * (n >> 3) + min(xcd, n & 7) + k


@pytest.mark.parametrize("P,n", [(256, 1024), (256, 512), (256, 1568), (512, 1024), (256, 300),
                                 (8, 8), (5, 5), (256, 256), (512, 513)])
def test_prefill_persistent_slots_cover_every_item_once(P, n):
    """Every item is taken exactly once; a multiple-of-8 grid keeps each
    workgroup's slots on its own XCD (slot % 8 == workgroup % 8); and the
    slot -> item map is a bijection on [0, n)."""
    slots = persistent_slots(P, n)
    taken = sorted(v for s in slots.values() for v in s)
    assert taken == list(range(n))
    if P % 8 == 0:
        assert all(v % 8 == blk % 8 for blk, s in slots.items() for v in s)
    assert sorted(slot_item(v, n) for v in range(n)) == list(range(n))


def test_prefill_persistent_order_evens_out_causal_blocks():
    """A fresh prefill's 32 token blocks per (sequence, KV head) come longest
    first (block j of the reversed order has 32 - j steps); with 256
    workgroups and 1024 items every workgroup gets the same number of steps
    in the snake order, while plain round robin would give the first XCD
    slots four of the longest."""
    P, n = 256, 1024
    steps = lambda lg: 32 - (lg % 32)  # items of one (sequence, KV head) are consecutive
    snake = [sum(steps(slot_item(v, n)) for v in s) for s in persistent_slots(P, n).values()]
    assert max(snake) == min(snake) == sum(steps(i) for i in range(n)) // P
    plain = [sum(steps(slot_item(b + r * P, n)) for r in range(n // P)) for b in range(P)]
    assert max(plain) > 1.5 * min(plain)
