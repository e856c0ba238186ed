"""Markdown table of the measured parity errors that the GPU tests record.

    DOCMASK_PARITY_LOG=/tmp/parity_rows.jsonl python -m pytest tests -m gpu
    python tests/parity_table.py /tmp/parity_rows.jsonl > profiles/parity_errors_all_workloads.md

One row per full-size check (workload, seed, what was compared): max abs
error of O, LSE, dQ, dK, dV against the float64 oracle, the GPU call's time,
and the oracle's wall time on the host cores of the same run."""
import json
import sys

NAMES = {1: "2048 tokens, docs [512,1024,256,256], 8/8 heads, d64 (fwd)",
         2: "32768 lognormal(1024,1.2), 32/8, d128 (fwd)",
         3: "CP rank 3 of 8, 131072 lognormal(2048,1.5), 32/8, d128 (fwd partials + merge)",
         4: "65536 lognormal(1024,1.2), 32/8, d128 (fwd+bwd)",
         5: "131072 bimodal, 64/8, d128 (fwd+bwd)",
         6: "65536 lognormal(2048,1.3), 16/4, d64 (fwd+bwd; head size 64 at full size)"}


def fmt(x, spec=".2e"):
    return "—" if x is None else format(x, spec)


def main(path):
    rows = [json.loads(line) for line in open(path) if line.strip()]
    rows.sort(key=lambda r: (r["config"], r["seed"] != r["config"], r["seed"], r["check"]))
    out = ["| workload | seed | check | compared | O | LSE | dQ | dK | dV | GPU ms | oracle s | host cores |",
           "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| {r['config']}: {NAMES.get(r['config'], '')} | {r['seed']} | {r['check']} | {r['compared']} | "
                   f"{fmt(r.get('err_O'))} | {fmt(r.get('err_LSE'))} | {fmt(r.get('err_dQ'))} | "
                   f"{fmt(r.get('err_dK'))} | {fmt(r.get('err_dV'))} | {fmt(r.get('gpu_ms'), '.3f')} | "
                   f"{fmt(r.get('oracle_s'), '.2f')} | {r.get('cores', '—')} |")
    worst = {k: max((r[k] for r in rows if r.get(k) is not None), default=None)
             for k in ("err_O", "err_LSE", "err_dQ", "err_dK", "err_dV")}
    out.append("")
    out.append("Largest error over all rows: " + ", ".join(f"{k[4:]} {fmt(v)}" for k, v in worst.items())
               + " (tolerances: 2e-2 on O, dQ, dK, dV; 1e-3 on LSE).")
    print("\n".join(out))


if __name__ == "__main__":
    main(sys.argv[1])
