"""Small builders shared by the tests (no verify arithmetic here)."""
import numpy as np

import synth


def pack(seqs, V, dtype="f32", name="hand"):
    """Pack per-sequence dicts {target [g+1,V], draft [g,V], tokens [g], T}
    into the library layout. Logits are given as float arrays."""
    gam = np.array([len(s["tokens"]) for s in seqs], np.int32)
    conv = (lambda a: synth.to_bf16_bits(np.asarray(a, np.float32))) if dtype == "bf16" else \
        (lambda a: np.asarray(a, np.float32))
    target = np.concatenate([conv(np.asarray(s["target"], np.float32).reshape(-1, V)) for s in seqs])
    drafts = [conv(np.asarray(s["draft"], np.float32).reshape(-1, V)) for s in seqs if len(s["tokens"])]
    sdt = np.uint16 if dtype == "bf16" else np.float32
    draft = np.concatenate(drafts) if drafts else np.zeros((0, V), sdt)
    tokens = np.concatenate([np.asarray(s["tokens"], np.int32) for s in seqs]) if gam.sum() else \
        np.zeros(0, np.int32)
    T = np.array([s["T"] for s in seqs], np.float32)
    return synth.Inputs(name, V, int(max(gam.max(initial=0), 1)), dtype, target, draft, tokens, gam, T)


def run_oracle(x, r=None, u=None, seed=None, row_offset=None, max_gamma=None, nthreads=None,
               lenience="none", epsilon=1.0):
    import oracle
    return oracle.verify(x.target, x.draft, x.tokens, x.gamma, x.temperature, vocab=x.vocab,
                         max_gamma=x.max_gamma if max_gamma is None else max_gamma,
                         seed=x.seed if seed is None else seed,
                         row_offset=x.row_offset if row_offset is None else row_offset,
                         r=r, u=u, lenience=lenience, epsilon=epsilon, nthreads=nthreads)


def subset(x, seqs):
    """The packed inputs of sequences `seqs` (in order) of x."""
    return synth.subset(x, seqs)
