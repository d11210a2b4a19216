"""Host logic of the phase-timeline tool: the summary of a stamp table (no GPU, no library)."""
import numpy as np

from dsa_pooled_key_amd import phase_trace as pt


def _tables(stamps):
    """stamps: {kernel: {block: {slot: tick}}} -> the per-file tables read_tables returns."""
    out = {name: np.zeros((pt.N_KERNELS, pt.N_BLOCKS, pt.N_SLOTS), dtype=np.uint64)
           for name in set(pt.TABLE_OF.values())}
    for k, blocks in stamps.items():
        for b, slots in blocks.items():
            for s, tick in slots.items():
                out[pt.TABLE_OF[k]][k, b, s] = tick
    return out


def _row(text, label):
    line = next(ln for ln in text.splitlines() if ln.startswith(f"| {label}"))
    return [c.strip() for c in line.strip("|").split("|")]


def test_summary_times_are_relative_to_the_first_block_and_phases_are_per_block():
    # Combine kernel (3): block b starts at 1000 + 100 b ticks and stores 250 + 50 b ticks later.
    blocks = {b: {0: 1000 + 100 * b, 1: 1000 + 100 * b + 250 + 50 * b} for b in range(5)}
    text = pt.summarise(_tables({3: blocks}))
    assert "sparse_mla combine: 5 blocks" in text
    start = _row(text, "0 block start")
    assert start[1] == "5" and start[3] == f"{200 * pt.TICK_US:.2f}"  # median start: block 2
    end = _row(text, "1 outputs stored")
    # block 2 ends at 1000 + 200 + 350 = 1550 ticks: 550 ticks after the first start
    assert end[3] == f"{550 * pt.TICK_US:.2f}"
    assert end[5] == f"{350 * pt.TICK_US:.2f}"  # median per-block phase (250 + 50 b, b = 2)
    span = (1000 + 400 + 450) - 1000
    assert f"{span * pt.TICK_US:.2f} us from the first block's start" in text


def test_points_a_block_skips_are_left_out_of_that_point():
    # Top-k kernel (1): block 1 skips point 3 (a row with at most Kw candidates).
    blocks = {0: {0: 10, 2: 20, 3: 30, 4: 40}, 1: {0: 10, 2: 22, 4: 44}}
    text = pt.summarise(_tables({1: blocks}))
    assert _row(text, "3 histogram scanned")[1] == "1"
    assert _row(text, "4 cutoff key known")[1] == "2"
    # the phase ending at point 4 is taken over the blocks that also have point 3
    assert _row(text, "4 cutoff key known")[5] == f"{10 * pt.TICK_US:.2f}"


def test_kernels_without_stamps_are_omitted():
    text = pt.summarise(_tables({}))
    assert text == ""
