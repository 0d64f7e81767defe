"""Reads the small text fixtures in this folder (comment lines start with '#')."""

import os

HERE = os.path.dirname(os.path.abspath(__file__))


def lines(name):
    with open(os.path.join(HERE, name)) as fh:
        return [ln.strip() for ln in fh if ln.strip() and not ln.lstrip().startswith("#")]


def int_list(name):
    return [int(x) for x in " ".join(lines(name)).split()]


def table(name):
    out = {}
    for ln in lines(name):
        key, val = ln.split()
        out[key] = float(val)
    return out
