"""bench.phase_summary on hand-made stamps (CPU): the phase arithmetic, the
work-group grouping and the merge timing follow the trace layout that
include/kvq.h documents for kvq_trace_set."""
import numpy as np

import bench


def wave(t, chunks, split, head, seq, xcc):
    return [*t, chunks | (split << 20) | (head << 36) | (seq << 44), 1 | (xcc << 8) | (0x1234 << 16)]


def test_phase_summary():
    # two work-groups of two waves; stamps in 10 ns ticks
    waves = [
        wave([1000, 1040, 1100, 1300, 2100, 2200], 3, 0, 0, 0, xcc=0),
        wave([1010, 1050, 1100, 1350, 2300, 2400], 3, 0, 0, 0, xcc=0),
        wave([1020, 1060, 1120, 1400, 2020, 2120], 2, 1, 0, 0, xcc=1),
        wave([1000, 1040, 1120, 0, 1120, 2130], 0, 1, 0, 0, xcc=1),   # no chunk: no first-chunk stamp
    ]
    decode_words = 8 * 8
    dec = np.zeros(decode_words, dtype=np.uint64)
    dec[:32] = np.array(waves, dtype=np.uint64).reshape(-1)
    mer = np.array([2700, 2750, 2900, 1, 0, 0, 0, 0, 2710, 2760, 2950, 1], dtype=np.uint64)
    raw = np.concatenate([dec, mer])
    s = bench.phase_summary(raw, decode_words, len(mer))
    assert s["waves"] == 4 and s["work_groups"] == 2
    assert s["start_skew"]["max"] == 0.2                       # 1020 - 1000 ticks
    assert s["seq_len"] == {"med": 0.4, "p10": 0.4, "p90": 0.4, "max": 0.4}
    assert s["first_chunk"]["max"] == 2.8                      # 1400 - 1120, waves with a chunk only
    assert s["chunk_loop"]["max"] == 12.0                      # 2300 - 1100
    assert s["intra_wg_loop_spread"]["max"] == 9.0             # (2020 - 1120) - (1120 - 1120)
    assert s["wg_slowest_wave_loop"]["max"] == 12.0
    assert s["per_xcc_loop_med"] == {0: 11.0, 1: 4.5}
    assert s["per_xcc_decode_end_max"] == {0: 14.0, 1: 11.3}
    assert s["merge_rows"] == 2
    assert s["merge_start_after_decode_end"]["max"] == 3.1     # 2710 - 2400
    assert s["call_end"] == 19.5                               # 2950 - 1000
