"""Largest measured errors of the parity tests, per case, so that the margin
under each bar can be written down (conftest dumps them at session end when
DDT_PARITY_REPORT names a file)."""
import json

ERRORS = {}


def record(case: str, quantity: str, value: float, bar: float) -> None:
    key = f"{case}:{quantity}"
    prev = ERRORS.get(key, {}).get("max", -1.0)
    ERRORS[key] = {"max": max(prev, float(value)), "bar": float(bar)}


def dump(path: str) -> None:
    with open(path, "w") as f:
        json.dump(dict(sorted(ERRORS.items())), f, indent=1)
