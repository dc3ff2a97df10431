"""Child process for the serialized-runtime test: greedy decode of a small streamed Q6_K model, printing
the tokens and a sha256 of each step's logits as one JSON line.  Arguments: workload id, n_resident,
number of tokens."""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from quantized_weight_streaming_gemv_amd import synthetic  # noqa: E402


def main():
    wid, n_res, n = int(sys.argv[1]), int(sys.argv[2]), int(sys.argv[3])
    wl = synth.tiny(synth.Q6_K, n_layers=6, wid=wid)
    m = synthetic.make_model(wl, n_resident=n_res)
    synthetic.load(m, wl)
    t, toks, digests = wl.first_token(), [], []
    for _ in range(n):
        t, lg = m.decode_step(t, want_logits=True)
        toks.append(t)
        digests.append(hashlib.sha256(lg.tobytes()).hexdigest())
    b, _ = m.stream_stats()
    m.close()
    print(json.dumps({"tokens": toks, "logit_sha256": digests, "h2d_bytes": b}))


if __name__ == "__main__":
    main()
