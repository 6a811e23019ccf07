"""The seeded input generators (synth) draw the same inputs on every machine and run: SHA-256 pins of their
float32 bytes (first 16 hex digits), recorded from this repository's generators.  A change to a generator's
draw order, distribution or seed shows up here before it silently changes what the parity tests and the
benchmark measure."""
import hashlib

import numpy as np
import torch

import synth


def _sha(t) -> str:
    a = t.float().numpy() if isinstance(t, torch.Tensor) else np.asarray(t, dtype=np.float32)
    return hashlib.sha256(np.ascontiguousarray(a, dtype=np.float32).tobytes()).hexdigest()[:16]


PINS = {
    "tiny_f32": {"h0": "c606bdcce3c5cc73", "Wq": "433f3483c0cc2278", "Wk": "06dd9472a89ea472",
                 "Wv": "813fc7c16b76b421", "wa": "6d56b8e22e2bebb4", "wb": "b32545ececa4adf5",
                 "rho": "862fb94861637cdc"},
    # bf16 workload (values rounded to bf16 before hashing as float32); 64-token prefix of the full draw
    "prefill_b1_l4096": {"h0": "19975d82fc68d80d", "Wq": "19b0aefcfb48ba56", "Wk": "0935b524594ccd20",
                         "Wv": "b0615fcbafdf74e2", "wa": "95777137ae5b10c8", "wb": "c6f3b5ddada4a07a",
                         "rho": "ae8b0a3001acb70e"},
}


def test_prefill_generators_pinned():
    got = {k: _sha(v) for k, v in synth.prefill_inputs(synth.workload("tiny_f32")).items()}
    assert got == PINS["tiny_f32"]
    got = {k: _sha(v) for k, v in synth.prefill_inputs(synth.workload("prefill_b1_l4096"), L=64).items()}
    assert got == PINS["prefill_b1_l4096"]


def test_decode_state_generator_pinned():
    assert _sha(synth.decode_state_init(synth.workload("decode_n64_s256"))) == "000c430f94d7ef99"
