"""Host-side model of the persistent wgrad kernel's work distribution (the
grid size rule of persistent_grid in gg_internal.hpp and the walks of
gg_wgrad.hip): under both schedules every item is computed exactly once and
every workgroup's walk ends.  Item t belongs to queue t % 8; workgroup b
serves queue b % 8.  Dynamic: a queue's positions go to its workgroups in
some order.  Static: workgroup b takes positions b // 8, b // 8 + W, ...,
W = grid // 8, or 1 when the grid has fewer than 8 workgroups."""
import pytest


def persistent_grid(items, cus=256):
    g = cus & ~7
    if g > items:
        g = items if items < 8 else items & ~7
    if g < 8 and items >= 8:
        g = 8
    return g


def static_walk(total, grid):
    step = grid >> 3 if grid >= 8 else 1
    for b in range(grid):
        x, pos, n = b & 7, b >> 3, 0
        while 8 * pos + x < total:
            yield b, 8 * pos + x
            pos += step
            n += 1
            assert n <= total, "a walk that does not end"


@pytest.mark.parametrize("cus", [256, 80, 8])
def test_static_walk_covers_every_item_once(cus):
    for total in list(range(1, 70)) + [600, 1000, 8192, 9001]:
        grid = persistent_grid(total, cus)
        assert 1 <= grid <= max(total, 8)
        items = sorted(t for _, t in static_walk(total, grid))
        assert items == list(range(total)), (total, grid)


def test_every_queue_is_served():
    """Each queue that holds items has at least one workgroup (the dynamic
    schedule relies on the same property)."""
    for total in list(range(1, 70)) + [600, 8192]:
        grid = persistent_grid(total)
        queues = {t % 8 for t in range(total)}
        served = {b % 8 for b in range(grid)}
        assert queues <= served, (total, grid)
