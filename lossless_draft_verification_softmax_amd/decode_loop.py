"""Multi-step speculative decoding on a synthetic Markov target, driven
through the C ABI: the loop the pages' eval server runs to report mean
accepted length and position-wise acceptance over whole generations
(tradepoint.io page, "The MTP path"; "AngelSpec: specialize the drafter...",
section "MTP": a drafted block is verified in one target pass and one
rejection invalidates the rest).

The "models" are first-order Markov chains over V tokens: the target row for
a context is row `prev` of the target table P, the draft row row `prev` of
the draft table Q.  One step, per request:
  1. draft D tokens with sv_sample_rows, call k reading the token call k - 1
     wrote (row = previous token), on word 2 of the Philox block of counter
     (k, request_id, step, 0);
  2. gather the target rows of the D + 1 contexts and the draft rows of the
     first D (a device-side row gather standing in for the target forward
     that produces these rows in a real system);
  3. sv_verify_batch (words 0 and 1 of the same blocks), then
     sv_accept_stats_accumulate, which adds the step to the running totals
     (tokens emitted, requests, expected accepted lengths, verified and
     accepted counts per position) and derives MAL, expected MAL, mean
     acceptance and the position-wise acceptance P(tau >= k);
  4. the last emitted token is the next step's first context.
Nothing here synchronises the host inside a step; every computation of the
method runs in the library's kernels.
"""
from __future__ import annotations

import torch

from . import specverify as sv


class MarkovDecodeLoop:
    def __init__(self, P_table: torch.Tensor, Q_table: torch.Tensor, start: torch.Tensor, D: int,
                 temperature: torch.Tensor, seed: int = 0, request_id: torch.Tensor | None = None):
        assert P_table.shape == Q_table.shape and P_table.shape[0] == P_table.shape[1]
        assert P_table.dtype == Q_table.dtype
        self.P, self.Q = P_table, Q_table
        self.V = P_table.shape[1]
        self.dev = P_table.device
        self.B = start.shape[0]
        self.D = D
        self.seed = seed
        self.T = temperature.to(device=self.dev, dtype=torch.float32).contiguous()
        self.rid = request_id
        self.last = start.to(device=self.dev, dtype=torch.int32).clone()
        B, V = self.B, self.V
        self.drafts = torch.zeros((B, max(D, 1)), dtype=torch.int32, device=self.dev)
        self.depth = torch.full((B,), D, dtype=torch.int32, device=self.dev)
        self.tr0 = torch.arange(B, dtype=torch.int64, device=self.dev) * (D + 1)
        self.dr0 = torch.arange(B, dtype=torch.int64, device=self.dev) * D
        self.target_rows = torch.empty((B * (D + 1), V), dtype=P_table.dtype, device=self.dev)
        self.draft_rows = torch.empty((max(B * D, 1), V), dtype=P_table.dtype, device=self.dev)
        self.verifier = sv.Verifier(B, D, V, self.dev, alpha=True, diag=True)
        self.verifier.prepare(self.target_rows, self.draft_rows, self.tr0, self.dr0,
                              self.drafts[:, :D], self.depth, self.T, seed=seed, step=0)
        self.step_no = 0
        # running statistics, kept by the library on the device
        self.stats = sv.AcceptAccumulator(D, self.dev)
        self.steps_done = 0

    def step(self):
        """One decode step for every request; returns the step's outputs
        (device tensors: accepted_len [B], out_tokens [B, D + 1])."""
        B, D = self.B, self.D
        for k in range(D):
            idx = self.last if k == 0 else self.drafts[:, k - 1]
            sv.sample_rows(self.Q, idx, self.T, self.drafts[:, k], seed=self.seed,
                           step=self.step_no, position=k, request_id=self.rid)
        ctx = torch.cat([self.last[:, None], self.drafts[:, :D]], dim=1)  # (B, D + 1)
        torch.index_select(self.P, 0, ctx.reshape(-1), out=self.target_rows)
        if D:
            torch.index_select(self.Q, 0, ctx[:, :D].reshape(-1), out=self.draft_rows)
        self.verifier.args.step = self.step_no
        out = self.verifier.run()
        self.stats.add(self.depth, out.alpha, out.accepted_len)
        tau = out.accepted_len.to(torch.int64)
        self.last = out.out_tokens.gather(1, tau[:, None]).reshape(B).to(torch.int32)
        self.steps_done += 1
        self.step_no += 1
        return out

    def summary(self) -> dict:
        """The library's statistics over every step so far: MAL (tokens
        emitted per request and step), expected MAL from the acceptance
        rates, mean acceptance (accepted over verified positions) and the
        position-wise acceptance P(tau >= k), k = 1..D."""
        s = self.stats.summary.cpu().tolist()
        return {"steps": self.steps_done, "mal": s[0], "expected_mal": s[1],
                "mean_acceptance": s[2], "position_acceptance": s[3:]}
