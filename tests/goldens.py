"""Reader for tests/golden/*.txt (hand-built fixtures with citations)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def blocks():
    """{name: {"header": bytes16, "qs_fill": int|None, "expect": [8 floats]|None}}"""
    out, cur = {}, None
    with open(os.path.join(GOLDEN, "blocks.txt")) as f:
        for raw in f:
            line = raw.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("[block "):
                cur = {"header": None, "qs_fill": None, "expect": None}
                out[line[len("[block "):-1]] = cur
                continue
            key, _, val = line.partition("=")
            key, val = key.strip(), val.strip()
            if key == "header":
                cur["header"] = bytes(int(t, 16) for t in val.split())
                assert len(cur["header"]) == 16
            elif key == "qs_fill":
                cur["qs_fill"] = int(val, 16)
            elif key == "expect_subblock":
                cur["expect"] = [float(t) for t in val.split()]
                assert len(cur["expect"]) == 8
    return out


def block_bytes(spec, qs=None):
    if qs is None:
        qs = bytes([spec["qs_fill"]] * 128)
    assert len(qs) == 128
    return spec["header"] + bytes(qs)


def accounting():
    rows = []
    with open(os.path.join(GOLDEN, "accounting.txt")) as f:
        for raw in f:
            line = raw.strip()
            if not line or line.startswith("#"):
                continue
            kind, *kv = line.split()
            rows.append((kind, {k: float(v) for k, v in (t.split("=") for t in kv)}))
    return rows
