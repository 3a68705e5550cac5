"""Parity margins (max|err| / tolerance per compared tensor) gathered over a
test session and printed at its end, so that a quiet run still records how
close each comparison came to its bound."""

RECORDS = []


def record(what, err, tol):
    RECORDS.append((str(what), float(err), float(tol)))


def summary_lines(top=20):
    if not RECORDS:
        return []
    ranked = sorted(RECORDS, key=lambda r: (r[1] / r[2]) if r[2] > 0 else float("inf"),
                    reverse=True)
    out = [f"parity margins: {len(RECORDS)} tensors compared; worst max|err|/tol first"]
    for what, err, tol in ranked[:top]:
        ratio = err / tol if tol > 0 else float("inf")
        out.append(f"  {ratio:8.4f}  max|err| {err:.3e}  tol {tol:.3e}  {what}")
    return out
