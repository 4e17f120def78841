"""Host model of the balanced schedule's bookkeeping (no GPU).

The balanced decode kernel cuts the (sequence, kv head) segments, laid end to
end in 32-token units, into W equal runs. A wave parks the cut pieces of its
run in LDS (the first piece, continuing a segment begun before the run, in
slot 0; the last, beginning a segment that goes on past the run, in slot 1).
After the workgroup's barrier the wave where a segment begins folds its own
piece and the slot-0 pieces of the following waves of its workgroup, and
writes the output if the segment ends inside the workgroup, else record
2w + 1; the first wave of a workgroup folds the slot-0 pieces that continue
a segment from an earlier workgroup into record 2w, and publishes the one
segment that ends in the workgroup after beginning earlier. The merge kernel
folds the records of those segments.

This model makes the same decisions with the same integer rules and checks,
over many shapes and wave counts and for workgroups of four and of eight
waves, that every unit of every segment reaches exactly one output exactly
once, that every parked piece and every record is used exactly once, and that
a workgroup never has two segments to publish.
The GPU parity tests check the kernel's numbers against the oracle; this
checks the schedule over far more shapes and wave counts than a GPU run can.
"""

import random

import pytest

UNIT = 32


def units_of(length):
    return (length + UNIT - 1) // UNIT


def simulate(lens, hkv, num_waves, waves_per_group=4):
    segs = []                       # (segment id, first unit, units)
    base = 0
    for i, length in enumerate(lens):
        nu = units_of(length)
        for g in range(hkv):
            if nu:
                segs.append((i * hkv + g, base, nu))
                base += nu
    total = base
    q = -(-total // num_waves) if total else 0

    finals = {}                     # segment -> units written as its output
    slot0, slot1, pending, ends_earlier = {}, {}, {}, {}

    def emit(sid, units):
        assert sid not in finals, f"segment {sid} written twice"
        finals[sid] = units

    seg_of_unit = {}
    for k, (sid, seg0, nu) in enumerate(segs):
        for u in range(seg0, seg0 + nu):
            seg_of_unit[u] = k

    for w in range(num_waves):
        u0, u1 = w * q, min(w * q + q, total)
        if u0 >= u1:
            continue
        wl = w % waves_per_group
        g_lo = (w - wl) * q
        g_hi = g_lo + waves_per_group * q
        g_room = min(g_hi - u1, 2**31 - 1)
        k = seg_of_unit[u0]
        _, seg0, nu = segs[k]
        if seg0 < g_lo and seg0 + nu <= u1:
            ends_earlier[w] = seg0 // q
        u = u0
        while u < u1:
            sid, seg0, nu = segs[k]
            k0, k1 = u - seg0, min(u1, seg0 + nu) - seg0
            units = set(range(seg0 + k0, seg0 + k1))
            if k0 == 0 and k1 == nu:
                emit(sid, units)
            elif k0 > 0:
                assert w not in slot0, "two continuation pieces in one run"
                slot0[w] = (sid, units)
            else:
                assert w not in slot1, "two beginning pieces in one run"
                slot1[w] = (sid, units)
                pending[w] = (sid, nu - k1 <= g_room)
            u = seg0 + k1
            if u == seg0 + nu:
                k += 1

    records, used_slot0, entries = {}, set(), {}
    groups = -(-num_waves // waves_per_group)
    for b in range(groups):
        w0 = b * waves_per_group
        for w in range(w0, min(w0 + waves_per_group, num_waves)):
            if w not in pending:
                continue
            sid, ends_here = pending[w]
            units = set(slot1[w][1])
            n = 1
            while w % waves_per_group + n < waves_per_group and slot0.get(w + n, (None,))[0] == sid:
                units |= slot0[w + n][1]
                used_slot0.add(w + n)
                n += 1
            if ends_here:
                emit(sid, units)
            else:
                records[2 * w + 1] = (sid, units)
        if w0 in slot0:
            sid = slot0[w0][0]
            units = set(slot0[w0][1])
            used_slot0.add(w0)
            n = 1
            while n < waves_per_group and slot0.get(w0 + n, (None,))[0] == sid:
                units |= slot0[w0 + n][1]
                used_slot0.add(w0 + n)
                n += 1
            records[2 * w0] = (sid, units)
        enders = [ends_earlier[w] for w in range(w0, w0 + waves_per_group) if w in ends_earlier]
        assert len(enders) <= 1, "two segments to publish in one workgroup"
        if enders:
            entries[b] = (slot0[w0][0], enders[0])

    used_records = set()
    for b, (sid, wf) in entries.items():
        wg0 = wf // waves_per_group
        rows = [2 * wf + 1] + [2 * (wg * waves_per_group) for wg in range(wg0 + 1, b + 1)]
        units = set()
        for r in rows:
            assert r in records and records[r][0] == sid, f"record {r} missing for {sid}"
            assert not units & records[r][1]
            units |= records[r][1]
            used_records.add(r)
        emit(sid, units)

    assert used_slot0 == set(slot0), "a parked piece was never folded"
    assert used_records == set(records), "a record was never merged"
    for sid, seg0, nu in segs:
        assert finals.get(sid) == set(range(seg0, seg0 + nu)), f"segment {sid}"
    return len(records), len(entries)


def random_case(rng):
    b = rng.randint(1, 12)
    hkv = rng.choice([1, 2, 3, 8])
    kind = rng.random()
    if kind < 0.3:
        lens = [rng.randint(0, 64) for _ in range(b)]
    elif kind < 0.7:
        lens = [rng.randint(0, 3000) for _ in range(b)]
    else:
        lens = [rng.choice([0, 1, 31, 32, 33, 4096, rng.randint(1, 20000)]) for _ in range(b)]
    num_waves = rng.choice([1, 2, 3, 4, 5, 7, 8, 12, 16, 31, 64, 100, 256, rng.randint(1, 400)])
    return lens, hkv, num_waves


@pytest.mark.parametrize("waves_per_group", [4, 8])
def test_every_unit_reaches_one_output_once(waves_per_group):
    rng = random.Random(20261203 + waves_per_group)
    merged = 0
    for _ in range(3000):
        lens, hkv, num_waves = random_case(rng)
        records, entries = simulate(lens, hkv, num_waves, waves_per_group)
        merged += entries
    assert merged > 0        # the cases do reach the merge kernel


@pytest.mark.parametrize("num_waves", [4, 8, 2048])
def test_layer_shapes(num_waves):
    # the OPT-13B and LLaMA-13B layers' segment counts, lengths drawn the same way
    rng = random.Random(num_waves)
    simulate([rng.randint(32, 2048) for _ in range(64)], 40, num_waves)
    simulate([min(4096, max(1, round(rng.lognormvariate(5.858, 0.9)))) for _ in range(256)], 40,
             num_waves)


def test_segments_inside_a_workgroup_need_no_record():
    # one segment over exactly the four waves of workgroup 0: folded in LDS
    records, entries = simulate([4 * UNIT], 1, 4)
    assert (records, entries) == (0, 0)
    # the same segment over waves 2..5 crosses into workgroup 1: one record each side
    records, entries = simulate([2 * UNIT, 4 * UNIT, 2 * UNIT], 1, 8)
    assert (records, entries) == (2, 1)
