"""A CPU model of the LL128 slice's index arithmetic (the kernel's
`slice_ll128`, `ll128_rows_iter` and `ll128_packets`), checked before any GPU
run sees a new layout: for every part size a slice can carry, aligned or
not, one and two inputs,

  * every data byte of the part is read from the user buffer and from the
    FIFO, and written to the FIFO and the user buffer (the FIFO side moves
    whole 16-byte packets, 8 bytes in column 7 of a line that goes packet by
    packet);
  * data byte u of the part lives at FIFO byte 128 (u // 120) + u % 120 (the
    pages' LL128 line: 120 data bytes, then the 8-byte flag, [ARCH] §七.2);
  * no access leaves the part or the slot; data loads never touch the flag
    bytes 120..127; every line's flag is written exactly once, either with
    the line's data in one full-line store (whole rows) or by a flag store
    after the batch's data have completed, and the batch's last line (the
    flag a consumer waits for) always the latter way;
  * the only user bytes written twice are bytes 104..111 of whole lines, by
    the lanes of columns 6 and 7 within one store instruction of one row
    iteration, after that iteration's loads (so in place stays correct).

Accesses through a range-limited buffer resource past its end are dropped
(stores) or read zeros (loads), as the hardware's range check does; the model
applies the same limits the kernel builds."""
import numpy as np
import pytest

SLOT_LINES = 256
BATCH = 256                     # lines per flag round trip: a whole slot
ROWS = 8                        # kLL128WholeRows (one input); two inputs take half


def model(nbytes, vec, two_inputs):
    """Per-byte access counts of one slice: user reads/writes, FIFO data
    reads/writes, flag writes with their kind (in a full-line store, or
    after the batch's data), plus the (instruction, row, lane) of user
    writes to check the double-written bytes."""
    R = ROWS // 2 if two_inputs else ROWS
    nlines = (nbytes + 119) // 120
    whole = nbytes // 120 if vec else 0
    user_rd = np.zeros(nbytes, np.int32)
    user_wr = np.zeros(nbytes, np.int32)
    fifo_rd = np.zeros(SLOT_LINES * 128, np.int32)
    fifo_wr = np.zeros(SLOT_LINES * 128, np.int32)
    flag_with_data = np.zeros(SLOT_LINES, np.int32)
    flag_after = np.zeros(SLOT_LINES, np.int32)
    last_lines = set()
    user_out_of_range = []
    writers = {}                 # user byte -> set of (instr, row, lane)
    instr = 0

    def user_access(arr, base, size, lim, tag=None):
        for b in range(base, base + size):
            if b >= lim:
                continue        # dropped / zero by the resource's range check
            if b >= nbytes:
                user_out_of_range.append(b)
                continue
            arr[b] += 1
            if tag is not None:
                writers.setdefault(b, set()).add(tag)

    def fifo_access(arr, base, size, lim, store=False):
        for b in range(base, base + size):
            if b >= lim:
                continue
            assert b < SLOT_LINES * 128, "FIFO access past the slot"
            if b % 128 >= 120:
                assert store and base % 128 == 112 and size == 16, f"flag byte {b % 128} touched by data"
                if b % 128 == 120:
                    flag_with_data[b // 128] += 1
                continue
            arr[b] += 1

    for b0 in range(0, nlines, BATCH):
        b1 = min(nlines, b0 + BATCH)
        last_lines.add(b1 - 1)
        bw = min(b1 - 1, max(b0, whole))
        if bw > b0:
            for l0 in range(b0, bw, 8 * R):
                instr += 1
                for lane in range(64):
                    col = lane & 7
                    coff = 104 if col == 7 else col * 16
                    for u in range(R):
                        line = l0 + 8 * u + (lane >> 3)
                        fifo_access(fifo_rd, line * 128 + coff, 16, bw * 128)
                        user_access(user_rd, line * 120 + coff, 16, bw * 120)
                for lane in range(64):
                    col = lane & 7
                    coff = 104 if col == 7 else col * 16
                    soff = 112 if col == 7 else coff
                    for u in range(R):
                        line = l0 + 8 * u + (lane >> 3)
                        fifo_access(fifo_wr, line * 128 + soff, 16, bw * 128, store=True)
                        user_access(user_wr, line * 120 + coff, 16, bw * 120, tag=(instr, u, lane))
        for lane in range(64):
            for p in range(bw * 8 + lane, b1 * 8, 64):
                line, col = p >> 3, p & 7
                uoff = line * 120 + col * 16
                if uoff >= nbytes:
                    continue
                nb = min(8 if col == 7 else 16, nbytes - uoff)
                fsz = 8 if col == 7 else 16
                fifo_access(fifo_rd, line * 128 + col * 16, fsz, SLOT_LINES * 128)
                fifo_access(fifo_wr, line * 128 + col * 16, fsz, SLOT_LINES * 128)
                instr += 1
                user_access(user_rd, uoff, nb, nbytes)
                user_access(user_wr, uoff, nb, nbytes, tag=(instr, 0, lane))
        # after the batch's data: the flags of the lines that went packet by
        # packet (at most the flags a lane holds per batch)
        for lane in range(64):
            for j in range(BATCH // 64):
                line = bw + 64 * j + lane
                if line < b1:
                    flag_after[line] += 1
    return dict(nlines=nlines, whole=whole, user_rd=user_rd, user_wr=user_wr, fifo_rd=fifo_rd,
                fifo_wr=fifo_wr, flag_with_data=flag_with_data, flag_after=flag_after, last=last_lines,
                out=user_out_of_range, writers=writers)


def _sizes():
    es_sizes = set()
    for n in list(range(1, 600, 7)) + [119, 120, 121, 239, 240, 241, 960, 7680, 7681, 15360, 15361,
                                        16384, 22528, 23040, 30712, 30720]:
        es_sizes.add(min(n, 30720))
    rng = np.random.default_rng(5)
    es_sizes.update(int(v) for v in rng.integers(1, 30721, 40))
    return sorted(es_sizes)


@pytest.mark.parametrize("two_inputs", [False, True])
@pytest.mark.parametrize("vec", [True, False])
def test_ll128_slice_covers_every_byte_once_and_stays_in_bounds(vec, two_inputs):
    for nbytes in _sizes():
        m = model(nbytes, vec, two_inputs)
        assert not m["out"], (nbytes, m["out"][:4])
        assert np.all(m["user_rd"] >= 1) and np.all(m["user_wr"] >= 1), nbytes
        u = np.arange(nbytes)
        fifo_pos = 128 * (u // 120) + u % 120
        # the FIFO side moves whole packets: it touches every image of a
        # data byte, and nothing outside the data bytes of the slice's lines
        touched = np.nonzero(m["fifo_wr"])[0]
        assert np.all(m["fifo_wr"][fifo_pos] >= 1) and np.all(m["fifo_rd"][fifo_pos] >= 1), nbytes
        assert np.all(touched < 128 * m["nlines"]), nbytes
        assert np.array_equal(np.nonzero(m["fifo_rd"])[0], touched), nbytes
        # bytes written twice: 104..111 of whole lines only, by one instruction
        twice = np.nonzero(m["user_wr"] > 1)[0]
        assert np.all(m["user_wr"] <= 2), nbytes
        assert np.all((twice % 120 >= 104) & (twice % 120 < 112)), (nbytes, twice[:4])
        assert np.all(twice // 120 < m["whole"]), nbytes
        for b in twice:
            tags = m["writers"][b]
            assert len({t[0] for t in tags}) == 1 and len({t[1] for t in tags}) == 1, (nbytes, b, tags)
            assert sorted(t[2] & 7 for t in tags) == [6, 7], (nbytes, b, tags)
        # a flag for every line of the slice, each written once; the last
        # line of every batch only after the batch's data
        flags = m["flag_with_data"] + m["flag_after"]
        assert np.array_equal(flags[:m["nlines"]], np.ones(m["nlines"], np.int32)), nbytes
        assert not flags[m["nlines"]:].any(), nbytes
        for ln in m["last"]:
            assert m["flag_after"][ln] == 1 and m["flag_with_data"][ln] == 0, (nbytes, ln)
