"""Writes tests/golden/stack_beta.json: the bias strength of the 48-layer
stack recipe, chosen by oracle.stack.calibrate_stack_beta (oracle code only).

    python -m oracle.calibrate_stack
"""
import json
import os

from .stack import calibrate_stack_beta

SEED = 0


def main():
    beta, fit = calibrate_stack_beta(SEED)
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "tests",
                        "golden", "stack_beta.json")
    with open(path, "w") as f:
        json.dump({"seed": SEED, "target_exponent": 1.1, "beta": beta,
                   "fitted_exponent": round(fit, 4),
                   "source": "oracle.stack.calibrate_stack_beta (synthetic logits, K=8, E=256)"},
                  f, indent=1)
        f.write("\n")
    print(path, beta, fit)


if __name__ == "__main__":
    main()
