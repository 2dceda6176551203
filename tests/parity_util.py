"""Helpers of the GPU parity tests: oracle-side preparation of the same seeded
inputs (oracle quantisation in a thread pool) and the comparison rules."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import moe_synth as S
from oracle import formats as F
from oracle import moe as M
from oracle.quantize import quantize

# relative Frobenius bound on block outputs vs the fp64 oracle
REL_FROB_TOL = 1e-2
# routing weights: absolute bound (fp32 softmax and renormalisation)
TOPK_W_TOL = 4e-6
# near-tie band on the logits within which the GPU may pick another expert
TIE_BAND = 1e-6


def _workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _quantize_one(args):
    layer, proj, e, seed = args
    w = F.bf16_bits_to_f64(S.expert_weight(layer, proj, e, seed))
    return quantize(w)


class OracleExperts:
    """Oracle-quantised expert weights of one model-shaped layer, made on
    demand for the experts a test touches (the oracle quantises the same bf16
    values the GPU quantiser got)."""

    def __init__(self, layer=0, seed=S.SEED):
        self.layer, self.seed = layer, seed
        self.q = {}

    def prefetch(self, experts):
        todo = [(self.layer, p, int(e), self.seed) for e in sorted(set(int(x) for x in experts))
                for p in (S.GATE, S.UP, S.DOWN) if (p, int(e)) not in self.q]
        if not todo:
            return
        # threads, not processes: numpy releases the GIL in the array work, and
        # no child process is forked from a process that holds the GPU
        with ThreadPoolExecutor(_workers()) as ex:
            for args, res in zip(todo, ex.map(_quantize_one, todo)):
                self.q[(args[1], args[2])] = res

    def fn(self, proj):
        def get(e):
            if (proj, e) not in self.q:
                self.prefetch([e])
            p, s, g = self.q[(proj, e)]
            return F.dequantize(p, s, g)
        return get


def router_f64(p):
    return dict(w_router=F.bf16_bits_to_f64(p["w_router"]), scale=F.bf16_bits_to_f64(p["scale"]),
                per_expert_scale=F.bf16_bits_to_f64(p["per_expert_scale"]), bias=p["bias"])


def check_route(gpu_idx, gpu_w, gpu_w_raw, ref, pes, tol_w=TOPK_W_TOL):
    """Indices: equal as sets, except for tokens the oracle flags as near-ties,
    where the GPU set may differ only inside the tie band.  Weights: compared
    against the oracle's weights for the GPU's own id set.  Returns the list of
    tokens whose set differed (all flagged)."""
    T, k = gpu_idx.shape
    differ = []
    for t in range(T):
        gs, os_ = set(gpu_idx[t].tolist()), set(ref["idx"][t].tolist())
        if gs != os_:
            assert ref["near_tie"][t], f"token {t}: ids {sorted(gs)} vs oracle {sorted(os_)}"
            assert (gs ^ os_) <= ref["band"][t], f"token {t}: differing ids outside the tie band"
            differ.append(t)
    w_ref, w_raw_ref = M.weights_for_ids(ref["logits"], pes, gpu_idx.astype(np.int64))
    assert np.max(np.abs(gpu_w - w_ref)) <= tol_w
    assert np.max(np.abs(gpu_w_raw - w_raw_ref)) <= tol_w
    assert np.max(np.abs(gpu_w_raw.sum(1) - 1.0)) <= 1e-6
    return differ


def rel_frob(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def row_rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.linalg.norm(a - b, axis=1) / np.maximum(np.linalg.norm(b, axis=1), 1e-300)
