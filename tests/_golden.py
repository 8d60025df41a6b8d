"""Readers for the text fixtures under tests/golden (each fixture cites the page it follows)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _floats(s):
    return [float(x) for x in s.split(",")] if s.strip() else []


def _ints(s):
    s = s.strip()
    return [] if s == "-" else [int(x) for x in s.split(",")]


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            yield [p.strip() for p in line.split("|")]


def topk_cases():
    return [(_floats(d), int(k), _ints(e)) for d, k, e in _rows("topk_cases.txt")]


def doc_span_cases():
    return [(_floats(d), _ints(b), int(k), _ints(e)) for d, b, k, e in _rows("doc_span_cases.txt")]


def page_numbers(kind):
    return [r[1:] for r in _rows("page_numbers.txt") if r[0] == kind]
