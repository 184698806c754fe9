"""The fp16 Gram-space route is taken only when every value it stores fits fp16 (host
logic, no GPU).  Checked independently of the library's own bound: for each coefficient
table the route accepts, the scalar recurrences the route's matrices follow are iterated
in fp64 over a dense grid of initial singular values in [0, 1] (X0 is normalised), and
the stored quantities -- R = sigma^2 and R P = sigma p(sigma), both stored times 2^14, the
polynomial q(sigma^2) and the accumulated Q = prod q -- must stay below fp16's largest
value; tables that overflow somewhere on the grid must be refused."""
import numpy as np
import pytest

ma = pytest.importorskip("adamw_optimizer_step_muon_amd")

F16_MAX = 65504.0
R_SCALE = 2.0 ** 14
QUINTIC = (3.4445, -4.7750, 2.0315)


def _max_stored(table):
    """Largest stored magnitude over the grid when running `table` (a list of (a, b, c))."""
    sig = np.linspace(0.0, 1.0, 20001)
    h = np.ones_like(sig)
    worst = 0.0
    with np.errstate(over="ignore", invalid="ignore"):  # diverging tables reach inf
        for a, b, c in table:
            t = sig * sig
            q = a + b * t + c * t * t
            p = sig * q
            h = h * q
            worst = max(worst, np.max(t) * R_SCALE, np.max(np.abs(sig * p)) * R_SCALE,
                        np.max(np.abs(q)), np.max(np.abs(h)))
            sig = np.abs(p)
    return float("inf") if np.isnan(worst) else worst


TABLES = [
    ("quintic x5", [QUINTIC] * 5),
    ("quintic x8", [QUINTIC] * 8),
    ("quintic x9", [QUINTIC] * 9),
    ("quintic x12", [QUINTIC] * 12),
    ("cubic x30", [(1.5, -0.5, 0.0)] * 30),
    ("mixed", [QUINTIC, (2.0, -1.5, 0.5), (1.5, -0.5, 0.0)]),
    ("steep", [(40.0, -4.0, 0.1)] * 2),
    ("growing", [(1.0, 3.0, 0.0)] * 3),
    ("one big step", [(8.0, -1.0, 0.0)]),
]


@pytest.mark.parametrize("name,table", TABLES)
def test_route_only_where_fp16_holds(name, table):
    taken = ma.muon_route_of(512, 2048, len(table), ns_mode=1, ns_coeffs=table).ns_mode_run
    worst = _max_stored(table)
    if taken:
        assert worst < F16_MAX, (name, worst)
    if worst >= F16_MAX:
        assert not taken, (name, worst)


def test_quintic_step_limit():
    """The quintic fits up to 8 steps (Q grows as a^N on a zero singular value)."""
    for n in range(1, 13):
        taken = ma.muon_route_of(512, 2048, n, ns_mode=1).ns_mode_run
        assert taken == (1 if n <= 8 else 0), n
        assert (_max_stored([QUINTIC] * n) < F16_MAX) or not taken


def test_random_tables():
    rng = np.random.default_rng(0)
    taken_any = refused_any = False
    for _ in range(200):
        n = int(rng.integers(1, 7))
        table = [(float(rng.uniform(0.5, 6.0)), float(rng.uniform(-8.0, 2.0)),
                  float(rng.uniform(-1.0, 4.0))) for _ in range(n)]
        taken = ma.muon_route_of(300, 1200, n, ns_mode=1, ns_coeffs=table).ns_mode_run
        worst = _max_stored(table)
        if taken:
            taken_any = True
            assert worst < F16_MAX, (table, worst)
        else:
            refused_any = True
    assert taken_any and refused_any
