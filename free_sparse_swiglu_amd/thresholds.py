"""Saved calibration artifacts: per-layer thresholds written once and
reloaded, never re-estimated at inference time.

The paper calibrates its thresholds once on calibration text and evaluates
with the saved artifacts only (App. A.7: calibration artifacts are saved and
the thresholds are neither re-estimated nor updated during inference).  Here
an artifact is a small JSON file holding the thresholds of one workload's
layers together with the recipe that produced them (shapes, quantiles,
number of calibration tokens, seeds); a file whose recipe differs from the
one asked for is not used.
"""
from __future__ import annotations

import json
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CALIB_DIR = os.path.join(ROOT, "calib")


def path_for(name: str) -> str:
    return os.path.join(CALIB_DIR, f"{name}.json")


def load(name: str, recipe: dict):
    """The saved thresholds of `name` if its recipe matches, else None."""
    p = path_for(name)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        art = json.load(f)
    if art.get("recipe") != recipe:
        return None
    return art["thresholds"]


def save(name: str, recipe: dict, thresholds: dict, out_dir: str | None = None) -> str:
    """Write the artifact (thresholds: a dict of lists of floats)."""
    d = out_dir or CALIB_DIR
    os.makedirs(d, exist_ok=True)
    p = os.path.join(d, f"{name}.json")
    with open(p, "w") as f:
        json.dump(dict(recipe=recipe, thresholds=thresholds), f, indent=1)
        f.write("\n")
    return p
