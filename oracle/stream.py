"""TEST INFRASTRUCTURE ONLY -- the delayed-stream bookkeeping of the oracle.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
it. It shares nothing with the library's wrapper (csrc/stream.cpp): this
version keeps every stream column of every channel (a dict per channel, no
ring) and recomputes each column from its definition.

What it computes (mobius PR #368, "P3 - ONNX Runtime example": the LMGen.step
port with a ring cache, per-codebook delays [0,0,1,1,1,1,1,1,1,0,1,1,1,1,1,1,1]
and delayed output collection; the persona/voice commit: teacher-forced agent
audio and text for priming), in the reading the repository's design notes
give:
* channel k (0 text, 1..A agent audio, A+1..S user audio) has delay d_k;
  stream column c of channel k holds the token of acoustic frame c - d_k, the
  initial token (Vt for text, card for audio) where c - d_k < 0, and column 0
  of the generated channels (0..A) is initial;
* step t feeds column t to the frame step and stores the text and agent
  codes it returns (forced where forced) as column t+1; the user's frame t is
  column t + d_k of the user channels;
* after step t the acoustic frame tau = t + 1 - max(d) is returned if
  tau >= 1: channel k's token sits in column tau + d_k.
"""


def default_delays(n_substeps, n_agent):
    """The pages' pattern: text 0; first agent and first user codebook 0; the
    other codebooks 1."""
    return [0 if k in (0, 1, n_agent + 1) else 1 for k in range(1 + n_substeps)]


class DelayedStream:
    """step_fn(frame [1+S], forced_text, forced_codes [S]) -> (text, codes [S])
    is one frame of the model (forced_* = -1 where the model chooses)."""

    def __init__(self, step_fn, n_substeps, n_agent, text_vocab, audio_card, delays=None):
        self.step_fn = step_fn
        self.S, self.A = n_substeps, n_agent
        self.Vt, self.card = text_vocab, audio_card
        self.d = list(delays) if delays is not None else default_delays(n_substeps, n_agent)
        self.D = max(self.d)
        self.cols = [dict() for _ in range(1 + n_substeps)]
        self.t = 0
        self.inputs = []  # every frame fed to step_fn

    def _initial(self, k):
        return self.Vt if k == 0 else self.card

    def column(self, k, c):
        """Token of channel k in stream column c (by the definition)."""
        if c - self.d[k] < 0 or (k <= self.A and c == 0):
            return self._initial(k)
        return self.cols[k][c]

    def step(self, user, forced=None):
        """user: the user's codes of acoustic frame t (S - A of them); forced:
        [1 + A] tokens for column t+1 (-1 = the model's choice) or None.
        Returns the completed acoustic frame [1 + A] or None."""
        S, A, t = self.S, self.A, self.t
        assert len(user) == S - A
        for j, u in enumerate(user):
            k = A + 1 + j
            self.cols[k][t + self.d[k]] = int(u)
        frame = [self.column(k, t) for k in range(1 + S)]
        self.inputs.append(frame)
        ft = -1 if forced is None else int(forced[0])
        fc = [-1] * S
        if forced is not None:
            for k in range(1, A + 1):
                fc[k - 1] = int(forced[k])
        text, codes = self.step_fn(frame, ft, fc)
        self.cols[0][t + 1] = ft if ft >= 0 else int(text)
        for k in range(1, A + 1):
            self.cols[k][t + 1] = fc[k - 1] if fc[k - 1] >= 0 else int(codes[k - 1])
        self.t = t + 1
        tau = t + 1 - self.D
        if tau < 1:
            return None
        return [self.column(k, tau + self.d[k]) for k in range(A + 1)]


def oracle_step_fn(session):
    """A step function over an oracle session (teacher forcing where forced)."""
    import numpy as np

    def fn(frame, forced_text, forced_codes):
        r = session.step(np.asarray(frame, np.int32), forced_text=forced_text,
                         forced_codes=np.asarray(forced_codes, np.int32))
        return r["text_token"], r["codes"]
    return fn
