"""bench.py's oracle and parity legs on the CPU: the oracle run of the tiny workload gives the teacher-forcing tokens
and logits, and the parity bookkeeping (max-abs error, greedy ids outside the margin, free-running agreement) is
checked against stand-in engines built from the oracle itself: one exact, one that flips a pick mid-run."""
import numpy as np

import bench
import oracle
import synth


class OracleEngine:
    """Engine stand-in (host-only) that computes each step with the oracle; `flip_at` makes its greedy chain pick a
    different token at that step (its logits for teacher-forced steps stay the oracle's)."""

    def __init__(self, w, ws, flip_at=None):
        self.w, self.model = w, oracle.OracleModel.from_weightset(ws)
        self.flip_at = flip_at
        self.reset_state()

    def reset_state(self):
        self.cache = oracle.RowCache(self.model, self.w.cap, self.w.kv_dtype)

    def step(self, tok, pos):
        lg = oracle.decode_step(self.model, self.cache, int(tok[0]), int(pos[0]))
        return lg[None, :].astype(np.float32), 0

    def step_greedy(self, tok, pos, n):
        ids, t = [], int(tok[0])
        for i in range(n):
            lg = oracle.decode_step(self.model, self.cache, t, int(pos[0]) + i)
            t = int(np.argmax(lg))
            if self.flip_at is not None and i == self.flip_at:
                t = (t + 1) % self.w.model.vocab
            ids.append([t])
        return np.array(ids, np.int32), np.zeros(n, np.uint32)


def test_oracle_leg_and_parity_bookkeeping():
    w = synth.workload("tiny-fp32")
    ws = synth.make_weights(w.model)
    sp, st = synth.start_positions(w), synth.start_tokens(w)
    cpu, ref = bench.cpu_baseline(w, ws, sp, st, budget_s=60.0, single_core_s=0.5)
    n = len(ref["tokens"])
    assert n == 32 and ref["tokens"][0] == int(st[0])
    assert all(ref["tokens"][i + 1] == int(np.argmax(ref["logits"][i])) for i in range(n - 1))
    assert cpu["single_core"]["cores"] == 1 and cpu["s_per_step"] > 0 and cpu["gbs_of_algorithmic_bytes"] > 0
    exact = bench.parity_leg(OracleEngine(w, ws), w, sp, st, ref)
    assert exact["within_tolerance"] and exact["logits_max_abs_err"] < 1e-5
    assert exact["greedy_equal"] == exact["greedy_checked"] and exact["greedy_checked"] + exact["greedy_inside_margin"] == n
    assert exact["free_running_agreement"] == n - 1
    flipped = bench.parity_leg(OracleEngine(w, ws, flip_at=5), w, sp, st, ref)
    assert flipped["free_running_agreement"] == 5 and flipped["within_tolerance"]
