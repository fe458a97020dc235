"""The n-gram self-drafter that proposes the draft tokens, as a plain model.

Test infrastructure only (see the package header).  Written from the AX
Engine page, "Core Technical Architecture & Methods": bigram and trigram
tables are built at run time from the tokens a sequence has seen, up to 4
draft tokens are proposed per step, and an exponential moving average of the
acceptance rate (tau = 0.1) switches speculation off when it falls below 0.5;
no second model is involved.

Readings taken (the page fixes none of them):
* the tables count continuations over every token the sequence has seen
  (prompt and accepted output): trigram (a, b) -> t and bigram b -> t;
* a draft continues the context with the trigram of its last two tokens when
  that pair has been seen, else with the bigram of its last token, else the
  draft stops; the continuation is the most frequent one, ties going to the
  one seen most recently; every drafted token extends the context for the
  next one, up to max_drafts tokens; drafted tokens never enter the tables;
* the average starts at 1 and moves whenever tokens are observed after a
  prediction of m > 0 tokens: rate <- (1 - tau) * rate + tau * matched / m,
  matched being the length of the common prefix of the prediction and the
  observed tokens; drafts are offered while rate >= threshold.  Predictions
  are made and scored while speculation is off as well, so the gate opens
  again when the text turns repetitive.
"""


class NgramModel:
    """One sequence's drafter state."""

    def __init__(self, max_drafts=4, tau=0.1, threshold=0.5):
        self.max_drafts = max_drafts
        self.tau = tau
        self.threshold = threshold
        self.history = []
        self.tri = {}  # (a, b) -> {t: [count, last index]}
        self.bi = {}  # b -> {t: [count, last index]}
        self.rate = 1.0
        self.pending = []  # the last prediction, scored by the next observe

    @staticmethod
    def _best(conts):
        # most frequent; among equals the one seen last
        return max(conts.items(), key=lambda kv: (kv[1][0], kv[1][1]))[0]

    def predict(self):
        ctx = list(self.history)
        out = []
        while len(out) < self.max_drafts:
            if len(ctx) >= 2 and (ctx[-2], ctx[-1]) in self.tri:
                t = self._best(self.tri[(ctx[-2], ctx[-1])])
            elif len(ctx) >= 1 and ctx[-1] in self.bi:
                t = self._best(self.bi[ctx[-1]])
            else:
                break
            out.append(t)
            ctx.append(t)
        return out

    def enabled(self):
        return self.rate >= self.threshold

    def draft(self):
        """The drafts to verify now (empty while the gate is closed); the
        prediction is kept for scoring either way."""
        self.pending = self.predict()
        return list(self.pending) if self.enabled() else []

    def observe(self, tokens):
        """Tokens the sequence has accepted (prompt or output), in order."""
        tokens = list(tokens)
        if self.pending and tokens:
            matched = 0
            while matched < min(len(self.pending), len(tokens)) and self.pending[matched] == tokens[matched]:
                matched += 1
            self.rate = (1.0 - self.tau) * self.rate + self.tau * (matched / len(self.pending))
        if tokens:
            self.pending = []
        for t in tokens:
            i = len(self.history)
            if i >= 1:
                e = self.bi.setdefault(self.history[-1], {}).setdefault(t, [0, -1])
                e[0] += 1
                e[1] = i
            if i >= 2:
                e = self.tri.setdefault((self.history[-2], self.history[-1]), {}).setdefault(t, [0, -1])
                e[0] += 1
                e[1] = i
            self.history.append(t)
