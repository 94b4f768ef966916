"""Host-side pieces of bench.py that need no GPU: the shader-clock reader and
the algorithmic byte count of a decode route."""
import bench


def test_sclk_reader_takes_the_marked_line(tmp_path):
    p = tmp_path / "pp_dpm_sclk"
    p.write_text("S: 97Mhz\n0: 500Mhz\n1: 2400Mhz *\n")
    assert bench.read_sclk_mhz(str(p)) == 2400
    p.write_text("S: 97Mhz *\n0: 500Mhz\n1: 2400Mhz\n")
    assert bench.read_sclk_mhz(str(p)) == 97
    p.write_text("0: 500Mhz\n1: 1325Mhz *\n2: 2400Mhz\n")
    assert bench.read_sclk_mhz(str(p)) == 1325
    p.write_text("0: 500Mhz\n1: 2400Mhz\n")
    assert bench.read_sclk_mhz(str(p)) is None
    assert bench.read_sclk_mhz(str(tmp_path / "absent")) is None


def test_decode_bytes_formula():
    # both weights once (51,380,224 + 25,690,112 bytes) plus, per row, the
    # hidden row, latent, logits, ids and weights
    assert bench.decode_bytes(1) == 77_070_336 + 25_216
    assert bench.decode_bytes(8) == 77_272_064
    assert bench.decode_bytes(20) - bench.decode_bytes(19) == 14_336 + 7_168 + 3_584 + 64 + 64


class _StubGraph:
    def __init__(self, log, count):
        self.log, self.count = log, count

    def replay(self):
        self.log.append(self.count)


class _StubSetup(bench.DecodeSetup):
    """DecodeSetup with graphs replaced by counters of the calls they hold."""

    def __init__(self, copies):
        self.copies = list(range(copies))
        self.replayed = []

    def capture(self, count=None):
        return _StubGraph(self.replayed, len(self.copies) if count is None else count)


def test_runner_replays_exactly_the_requested_routes():
    for copies in (1, 3, 8):
        for cycles in (1, 25):
            g = cycles * copies
            for steps, warm in ((1600, 80), (20, 5), (7, 0), (8, 8), (1, 1), (200, 400)):
                d = _StubSetup(copies)
                run = d.runner([steps, warm], cycles=cycles)
                assert run.graph_routes == g
                for n in (steps, warm):
                    d.replayed.clear()
                    run(n)
                    assert sum(d.replayed) == n, (copies, cycles, n)
                    # whole graphs of `cycles` passes over the copies, then
                    # one shorter graph at most
                    assert all(c == g for c in d.replayed[:n // g])
                    assert len(d.replayed) == n // g + (1 if n % g else 0)


def test_default_graph_is_whole_passes_over_the_copies():
    d = _StubSetup(8)
    run = d.runner([1600])
    assert run.graph_routes == bench.GRAPH_CYCLES * 8
    assert 1600 % run.graph_routes == 0
