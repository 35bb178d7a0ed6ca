"""Worst parity margin per test family, collected by ``_helpers.report`` and
printed at the end of the run by ``conftest.pytest_terminal_summary`` (so the
margins survive a quiet run). A family is the test module plus the test
function's name without its parameters."""
from __future__ import annotations

WORST: dict = {}


def record(family: str, case: str, ratio: float, max_err: float, max_ref: float) -> None:
    cur = WORST.get(family)
    if cur is None or not (ratio <= cur[0]):
        WORST[family] = (ratio, case, max_err, max_ref)
