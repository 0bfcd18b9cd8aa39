"""Per-comparison record of the parity tests: the raw max-abs output error, how many
elements exceed the literal tolerance (1e-2 for bf16 / fp16, 2e-5 for fp32; the gate adds
half an output ulp there, except on the five stated configurations, which must meet it
literally) and the max-abs LSE error.  conftest.py prints a summary at the end of the
session and writes the records to $PARITY_LOG_JSON when that is set."""

RECORDS = []


def record(where, dtype, n, max_abs, beyond_tol, lse_max_abs, literal):
    RECORDS.append({"where": where, "dtype": dtype, "elements": int(n),
                    "max_abs": float(max_abs), "beyond_tol": int(beyond_tol),
                    "lse_max_abs": float(lse_max_abs), "literal_gate": bool(literal)})
