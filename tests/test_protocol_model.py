"""The single-pass look-back scan's inter-workgroup protocol, replayed on the
CPU under seeded random schedules (protocol_model): every tile folds exactly
the tiles before it from words of its own launch, superblock and block
aggregates are exact, the epoch hand-over leaves the claims word clean, the
cycle's last launch clears the words, and every schedule finishes (also with
one workgroup resident at a time). Each planted protocol mistake is caught.
"""
import re
from pathlib import Path

import pytest

from protocol_model import Faults, ProtocolError, run_launches

# Launches on one workspace with an epoch cycle of 3 (epochs 1, 2, 3, 1, ...):
# the 4th meets the 1st's epoch-1 words beyond the 8 tiles the 2nd and 3rd
# rewrote, so a missing end-of-cycle clear shows; tile counts from 1 to the
# three-level maximum of 4^3, grids larger and smaller than the tile count,
# and residency limits down to one running workgroup.
LAUNCHES = [(64, 6, 3), (8, 2, 2), (5, 3, 3), (64, 8, 8), (30, 4, 2), (3, 2, 1), (2, 1, 1),
            (64, 5, 5), (1, 1, 1), (17, 5, 3), (40, 8, 8)]


def kernel_constant(name):
    src = (Path(__file__).resolve().parents[1] / "mamba_s6_selective_amd" / "csrc"
           / "linear_scan.hip").read_text()
    return int(re.search(rf"constexpr int {name} = (\d+);", src).group(1))


def test_model_matches_kernel_window_shape():
    """The model's windows assume what the kernel's do: a block-closing
    tile's recent superblocks all lie in its own block (fan >= recent)."""
    fan, recent = kernel_constant("kFan"), kernel_constant("kRecent")
    assert fan >= recent >= 1
    run_launches([(3 * 8 + 5, 4, 4)], fan=8, recent=min(recent, 8), cycle=2, seed=1)


@pytest.mark.parametrize("seed", range(12))
def test_protocol_random_schedules(seed):
    run_launches(LAUNCHES, fan=4, recent=3, cycle=3, seed=seed)


@pytest.mark.parametrize("recent", [1, 2, 4])
def test_protocol_window_depths(recent):
    run_launches(LAUNCHES, fan=4, recent=recent, cycle=2, seed=100 + recent)


def test_protocol_kernel_depth():
    """The kernel's look-back depth (6 recent superblocks) with 8-tile
    superblocks, up to 512 tiles (all three levels), two-epoch cycle."""
    recent = kernel_constant("kRecent")
    run_launches([(512, 16, 9), (100, 3, 2), (300, 40, 40)], fan=8, recent=recent, cycle=2,
                 seed=7)


def test_protocol_one_resident_workgroup():
    """Progress without co-residency: one workgroup runs at a time, so each
    one must finish with only lower tiles published before it."""
    run_launches([(n, g, 1) for n, g, _ in LAUNCHES], fan=4, recent=3, cycle=3, seed=5)


FAULTS = ["check_a_only", "no_cycle_clear", "handoff_one_early", "publish_without_wait",
          "lvl1_window_one_short", "block_needs_only_own"]


@pytest.mark.parametrize("fault", FAULTS)
def test_planted_protocol_fault_is_caught(fault):
    """Each mistake (a pair accepted on one current word, no clear at the end
    of the cycle, the next epoch handed over one claim early, a superblock
    aggregate published before its window is complete, a level-1 window one
    superblock short, a block aggregate published from its own window only)
    fails every schedule tried."""
    for seed in range(5):
        with pytest.raises(ProtocolError):
            run_launches(LAUNCHES, fan=4, recent=3, cycle=3, seed=seed,
                         faults=Faults(**{fault: True}))
