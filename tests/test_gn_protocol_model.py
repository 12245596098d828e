"""Why a single-launch GroupNorm did not finish: a host-threaded model (CPU).

A one-launch form of the GroupNorm (statistics and normalisation items
taken from one queue, a per-frame counter whose last finisher reduces the
partials and raises the frame's flag, normalisation items polling that flag
with a bounded wait) was tried once on the GPU and its smallest case,
3 frames of 140 pixels with 32-pixel chunks (the last one ragged, 12
pixels), did not finish within 120 s; the code was not kept. The model in
tests/gn_protocol/model.cpp replays that protocol with threads for
work-groups and the same chunk arithmetic, and separates the forms that
finish from those that spin every normalisation item to its bound:

- the protocol as described finishes for every lag, lag >= frames included;
- a counter target that the ragged last chunk cannot reach (pixels counted
  against chunks * chunk_px) never raises a flag: every normalisation item
  runs to its bound;
- a poll that reads the flag once (a plain load the compiler may hoist, or
  a line served from a cache that is not refreshed) runs every item taken
  while its frame was in flight to its bound;
- items whose normalisation chunks precede their statistics deadlock once
  they occupy every worker, until the bounds expire;
- emitting normalisation items only while t < frames drops the last lag
  frames (wrong output, not a hang).
"""
import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path_factory.mktemp("gn") / "model")
    subprocess.run(["g++", "-std=c++17", "-O2", "-pthread", "-Wall",
                    os.path.join(HERE, "gn_protocol", "model.cpp"), "-o", exe], check=True)

    def run(variant, lag, workers, stats_us=0, frames=3, pixels=140, chunk=32, bound=20000):
        r = subprocess.run([exe, variant, str(frames), str(pixels), str(chunk), str(lag),
                            str(workers), str(bound), str(stats_us)],
                           capture_output=True, text=True, timeout=120, check=True)
        m = re.search(r"timeouts=(\d+) frames_normalised=(\d+) of (\d+)", r.stdout)
        return int(m.group(1)), int(m.group(2)), int(m.group(3))
    return run


@pytest.mark.parametrize("lag", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("workers", [2, 4, 8])
def test_protocol_as_described_finishes(model, lag, workers):
    timeouts, done, frames = model("ok", lag, workers, stats_us=100)
    assert timeouts == 0 and done == frames


def test_unreachable_counter_target_spins_every_item(model):
    timeouts, _, _ = model("pixel_target", 1, 4)
    assert timeouts == 15           # all 3 x 5 normalisation chunks ran to the bound


def test_read_once_poll_spins_items_taken_early(model):
    timeouts, _, _ = model("hoisted", 0, 8, stats_us=200)
    assert timeouts > 0


def test_consumers_ahead_of_producers_block_every_worker(model):
    timeouts, _, _ = model("norm_first", 0, 4, stats_us=200)
    assert timeouts > 0


def test_short_item_loop_drops_frames_but_finishes(model):
    timeouts, done, frames = model("lag_short", 3, 4)
    assert timeouts == 0 and done == 0 < frames
