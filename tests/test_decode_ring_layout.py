"""CPU model of the small-token kernels' LDS ring (decode.hip): one operand of a k step is 16
rows x 128 bytes in 128 16-byte slots.  Load instruction i (0, 1) of a wave brings rows 8i ..
8i + 7 with whole-line direct loads: lane l fetches chunk (l % 8) ^ (l / 8) of row 8i + l / 8 into
slot 64i + l.  The MFMA operand read of sub-step m gives lane L row L % 16, chunk 4m + L / 16.

Checked here, on the index arithmetic alone: the two instructions fill every slot once and fetch
every (row, chunk) once, each instruction's lanes cover whole 128-byte lines, every read finds
the slot holding its (row, chunk), the reads of a sub-step cover 16 rows x 4 chunks once, and the
eight lanes that share a row group (L / 8) read eight different 16-byte bank groups."""


def load_row(lane, i):
    return 8 * i + lane // 8


def load_chunk(lane):
    return (lane % 8) ^ (lane // 8)


def read_slot(lane, m):
    r, c = lane % 16, 4 * m + lane // 16
    return 64 * (r // 8) + 8 * (r % 8) + (c ^ (r % 8))


def _filled():
    """slot -> (row, chunk) after both load instructions of a stage."""
    slots = {}
    for i in range(2):
        for lane in range(64):
            slot = 64 * i + lane
            assert slot not in slots
            slots[slot] = (load_row(lane, i), load_chunk(lane))
    return slots


def test_loads_fill_every_slot_with_every_row_chunk_once():
    slots = _filled()
    assert sorted(slots) == list(range(128))
    assert sorted(slots.values()) == [(r, c) for r in range(16) for c in range(8)]


def test_each_load_instruction_reads_whole_lines():
    for i in range(2):
        rows = {}
        for lane in range(64):
            rows.setdefault(load_row(lane, i), set()).add(load_chunk(lane))
        assert len(rows) == 8 and all(ch == set(range(8)) for ch in rows.values())


def test_reads_find_their_row_and_chunk():
    slots = _filled()
    for m in range(2):
        seen = set()
        for lane in range(64):
            want = (lane % 16, 4 * m + lane // 16)
            assert slots[read_slot(lane, m)] == want
            seen.add(want)
        assert seen == {(r, 4 * m + g) for r in range(16) for g in range(4)}


def test_rows_of_a_bank_group_read_distinct_banks():
    # 64 banks of 4 bytes: a 16-byte slot s occupies bank group s % 16
    for m in range(2):
        for base in range(0, 64, 8):
            groups = [read_slot(lane, m) % 16 for lane in range(base, base + 8)]
            assert len(set(groups)) == 8, (m, base, groups)
