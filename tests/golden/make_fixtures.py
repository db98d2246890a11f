"""Writes the block-mass fixtures shaped like the pages' worked examples.

The digest page "CRISP: Cliff-awaRe Input-adaptive Sparse Prefilling with
Structural-Mass-Motivated Routing" describes, in its Figure 1 caption and its
appendix-D figure caption, four VS heads whose sorted block masses show the two
failure modes of the gamma = 0.95 cumulative-coverage rule and the noise floor
(alpha = 1.0) isolating the signal:

* Figure 1 left: sink = 0.93; gamma-cumsum stops inside the sink block and the
  8 important blocks are never visited.
* Figure 1 right: sink = 0.91; gamma-cumsum runs past the signal into the
  noise and gathers 13 near-zero blocks.
* Appendix D: sink = 0.94, gamma never reaches the signal; sink = 0.61,
  gamma-cumsum gathers 14 noise blocks.

The exact vectors are not printed, so each fixture is constructed from those
printed quantities (sink mass, number of signal blocks, number of noise blocks
gamma-cumsum gathers): block 0 is the sink, block N_b-1 the local window,
signal blocks carry equal mass, and the leftover mass is spread evenly over the
remaining (noise) blocks.  The expected outcomes are the pages' counts; they
follow from the construction alone (this script imports nothing from the
oracle):

  gamma-cumsum keeps sink, local, then signal blocks (descending mass), then
  ceil(residual / eps) noise blocks, residual = gamma - (sink + local + signal);
  the noise floor keeps exactly anchors + signal because
  signal > mu = (1 - sink - local)/(N_b - 2) > eps.

Run:  python tests/golden/make_fixtures.py
"""
import json
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
GAMMA = 0.95


def build(name, cite, nb, sink, local, sig_pos, sig_mass, expect_noise):
    p = [0.0] * nb
    p[0] = sink
    p[nb - 1] = local
    for j in sig_pos:
        p[j] = sig_mass
    noise_pos = [j for j in range(1, nb - 1) if j not in set(sig_pos)]
    eps = (1.0 - sink - local - sig_mass * len(sig_pos)) / len(noise_pos)
    for j in noise_pos:
        p[j] = eps
    mu = (1.0 - sink - local) / (nb - 2)
    assert sig_mass > mu > eps, (name, sig_mass, mu, eps)
    residual = GAMMA - sink - local - sig_mass * len(sig_pos)
    if sink >= GAMMA or sink + local >= GAMMA:
        # gamma is met before any signal block is reached
        kept_gamma = 1 if sink >= GAMMA else 2
        noise_gamma = 0
        signal_visited = 0
    else:
        noise_gamma = max(0, math.ceil(residual / eps))
        kept_gamma = 2 + len(sig_pos) + noise_gamma
        signal_visited = len(sig_pos)
    assert noise_gamma == expect_noise, (name, noise_gamma)
    return dict(
        name=name, citation=cite, gamma=GAMMA, alpha=1.0, k_min_blocks=8,
        p=p, signal_blocks=sorted(sig_pos),
        expect_floor_set=sorted({0, nb - 1} | set(sig_pos)),
        expect_gamma_kept=kept_gamma, expect_gamma_noise_blocks=noise_gamma,
        expect_gamma_signal_visited=signal_visited,
    )


def main():
    fx = [
        build("fig1_left_sink_only_collapse",
              "digest page, Figure 1 caption (left panel: sink = 0.93, gamma = 0.95 stops "
              "inside the sink, 8 important blocks never visited)",
              64, 0.93, 0.03, [5, 12, 20, 27, 33, 41, 50, 58], 0.003, 0),
        build("fig1_right_noise_accumulation",
              "digest page, Figure 1 caption (right panel: sink = 0.91, gamma = 0.95 "
              "accumulates 13 near-zero noise blocks)",
              144, 0.91, 0.02, [9, 30, 51, 77, 100, 121], 0.0025, 13),
        build("appD_sink094_signal_never_reached",
              "digest page, appendix-D figure caption (sink = 0.94: gamma = 0.95 never "
              "reaches the signal)",
              64, 0.94, 0.02, [3, 11, 19, 26, 34, 45, 52, 60], 0.002, 0),
        build("appD_sink061_accumulates_14",
              "digest page, appendix-D figure caption (sink = 0.61: gamma = 0.95 gathers "
              "14 noise blocks)",
              128, 0.61, 0.05, [7, 18, 29, 40, 52, 63, 75, 88, 99, 111],
              (GAMMA - 0.66 - 0.675 / 102.5) / 10, 14),
    ]
    for f in fx:
        f["expect_gamma_missed_signal"] = len(f["signal_blocks"]) - f["expect_gamma_signal_visited"]
    with open(os.path.join(HERE, "block_mass_examples.json"), "w") as fh:
        json.dump(fx, fh, indent=1)
        fh.write("\n")


if __name__ == "__main__":
    main()
