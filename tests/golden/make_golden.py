"""Write tests/golden/tiny_prefill_oracle.npz from the seeded inputs and the oracle.

The fixture is a regression record of the oracle on the tiny prefill workload
(B=1, H=4, T=S=16, past_len=0, seed 0): it calls only the oracle package and
the seeded input generator, never the HIP library.

    python tests/golden/make_golden.py
"""

import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import mla_attention  # noqa: E402
from seeded_inputs import WORKLOADS, host_inputs  # noqa: E402


def main():
    wl = WORKLOADS["tiny_prefill"]
    x = host_inputs(wl, seed=0)
    out = mla_attention(x["q_nope"], x["q_pe"], x["k_nope"], x["k_pe"], x["v"], wl.past_len, wl.softmax_scale)
    np.savez_compressed(os.path.join(HERE, "tiny_prefill_oracle.npz"), out=out, **x)


if __name__ == "__main__":
    main()
