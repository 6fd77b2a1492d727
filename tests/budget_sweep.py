"""Budget sweep of page top-K attention against the fp64 oracle (run on a GPU
box; prints a markdown table):

    python tests/budget_sweep.py

For both input laws of tests/test_gpu_budget_error.py and K in 4, 8, 16, 32,
64 and every page: the library's sparse fwd+bwd against the oracle's dense
result (relative Frobenius norm of the difference, cosine similarity) and
against the oracle's sparse result on the library's selection (max-abs /
max |ref|, which must stay within 1e-2)."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from tests.test_gpu_budget_error import LAWS, NAMES, _budget, _dense  # noqa: E402


def main() -> int:
    rows = []
    for law, cfg in LAWS.items():
        f, dense = _dense(cfg)
        for k in (4, 8, 16, 32, 64, cfg.n_pages):
            r = _budget(cfg, f, dense, k)
            bad = [n for n in NAMES if r["impl"][n] > 1e-2]
            kname = "all" if k >= cfg.n_pages else str(k)
            rows.append(f"| {law} | {kname} | {r['page_frac']:.3f} | "
                        + " | ".join(f"{r['approx'][n]:.4f}" for n in NAMES) + " | "
                        + " | ".join(f"{r['cos'][n]:.5f}" for n in NAMES) + " | "
                        + f"{max(r['impl'].values()):.1e} |")
            print(rows[-1], flush=True)
            if bad:
                print(f"implementation error above 1e-2 for {bad}", flush=True)
                return 1
    print("\n| law | K | pages attended / dense | O | dQ | dK | dV | cos O | cos dQ | cos dK "
          "| cos dV | max impl. error |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|")
    print("\n".join(rows), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
