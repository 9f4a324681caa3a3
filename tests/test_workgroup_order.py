"""CPU checks of the workgroup renumbering the decode and prefill kernels share (xcd_unit, exported as
gdn_workgroup_order): every work unit runs exactly once, whatever the grid size and run length, and
each run of 2^xcd_shift consecutive units inside a whole span lands on one XCD (ids are dealt to the
8 XCDs round-robin, so the XCD of workgroup id bx is bx % 8).  The kernels' correctness rests on the
first property; the second is what the renumbering is for."""
import numpy as np
import pytest

import recurrent_state_decode_amd as rsd

# grid sizes of the workloads and launch shapes in use, small grids, and sizes around whole spans
WORKLOAD_GRIDS = [256 * 32 * 16, 256 * 32 * 4, 64 * 32 * 4, 128 * 32 * 8, 512 * 32 * 2, 16 * 32, 1, 7, 8, 9]
SPAN_EDGES = sorted({m * 8 * (1 << gs) + d for gs in range(7) for m in (1, 2, 3) for d in (-1, 0, 1)})


@pytest.mark.parametrize("gs", range(7))
def test_every_unit_runs_once(gs):
    for grid in list(range(0, 700)) + WORKLOAD_GRIDS + SPAN_EDGES:
        if grid < 0:
            continue
        units = np.array(rsd.workgroup_order(grid, gs), dtype=np.int64)
        assert units.shape == (grid,)
        assert np.array_equal(np.sort(units), np.arange(grid)), (grid, gs)


@pytest.mark.parametrize("gs", range(7))
def test_runs_of_consecutive_units_share_an_xcd(gs):
    G = 1 << gs
    for grid in WORKLOAD_GRIDS + [8 * G * 5 + 3]:
        units = np.array(rsd.workgroup_order(grid, gs), dtype=np.int64)
        xcd_of_unit = np.empty(grid, dtype=np.int64)
        xcd_of_unit[units] = np.arange(grid) % 8
        nfull = (grid // (8 * G)) * 8 * G
        runs = xcd_of_unit[:nfull].reshape(-1, G)
        assert np.all(runs == runs[:, :1]), (grid, gs)
        # the ids past the last whole span run their own unit
        assert np.array_equal(units[nfull:], np.arange(nfull, grid))


def test_refuses_bad_arguments():
    for grid, gs in ((-1, 0), (4, -1), (4, 17)):
        with pytest.raises(rsd.GdnError):
            rsd.workgroup_order(grid, gs)
