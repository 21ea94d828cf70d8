"""Zero-shot text control of streaming TTS -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg may import
this module; the HIP path shares no code with it.

Source: the walkthrough of the Moshi technical report on 139.9.1.231, appendix C
("延迟文本语言模型作为zero-shot流式ASR和TTS"), TTS mode and Fig. 9:
  * the text to speak comes without padding, so the model is left to sample PAD
    and EPAD freely at the end of each word;
  * whenever it would sample any other token, the next word's tokens are fed
    instead;
  * an online average of the padding ratio is kept, and while it is below a
    target, a small bonus is added to the padding logit, which keeps the
    speaking rate in check.

READINGS (the page gives the rule, not its arithmetic):
  * a word of n tokens is fed on n consecutive steps. Between its tokens the
    model is not consulted: it may only pick PAD or EPAD "at the end of" a word;
  * the padding ratio is (number of PAD tokens emitted so far) / (number of
    text tokens emitted so far), taken before the current step; it is below the
    target when n_pad < target * max(n_steps, 1), evaluated in float32 (so the
    bonus applies at the first step whenever the target is positive);
  * the bonus is added to the PAD logit only. A bonus on EPAD would start the
    next word sooner, the opposite of slowing down;
  * once every word has been fed, the controller keeps answering PAD;
  * the decision is the step's draw from the boosted logits: the argmax (lowest
    index first on ties) when decoding greedily, the temperature draw of
    ``oracle.sampling`` otherwise (the pages sample TTS at temperature 0.6),
    computed in the precision of the logits it is given.
"""
from __future__ import annotations

from typing import List, Sequence

import numpy as np


class TtsTextControl:
    """Chooses the text token of each TTS step from the text logits.

    ``words`` is a list of token-id lists, one per word, in speaking order;
    ``pad_id`` and ``epad_id`` are the text vocabulary's PAD and EPAD ids.
    Use ``choose`` as ``Session.step(..., text_choice=ctl.choose)``.
    """

    def __init__(self, words: Sequence[Sequence[int]], pad_id: int, epad_id: int, target_pad_ratio: float,
                 bonus: float):
        if bonus < 0:
            raise ValueError("the padding bonus must be >= 0")
        if any(len(w) == 0 for w in words):
            raise ValueError("empty word")
        self.tokens: List[int] = [int(t) for w in words for t in w]
        self.word_start: List[bool] = [i == 0 for w in words for i in range(len(w))]
        self.cursor = 0
        self.pad_id, self.epad_id = int(pad_id), int(epad_id)
        self.target = float(np.float32(target_pad_ratio))
        self.bonus = float(np.float32(bonus))
        self.n_pad = 0
        self.n_steps = 0

    def choose(self, logits: np.ndarray, pick=None) -> int:
        """The text token of one step. ``pick`` maps the (PAD-boosted) logits to a
        token; the default is the greedy argmax (``Session`` passes its sampler)."""
        tok = self._decide(np.asarray(logits), pick or (lambda lg: int(np.argmax(lg))))
        self.n_steps += 1
        self.n_pad += int(tok == self.pad_id)
        return tok

    def _decide(self, logits: np.ndarray, pick) -> int:
        n = len(self.tokens)
        # inside a word: its next token, without consulting the model
        if 0 < self.cursor < n and not self.word_start[self.cursor]:
            self.cursor += 1
            return self.tokens[self.cursor - 1]
        lg = logits.copy()
        if self.below_target():
            lg[self.pad_id] = lg[self.pad_id] + lg.dtype.type(self.bonus)
        choice = int(pick(lg))
        if choice in (self.pad_id, self.epad_id):
            return choice
        if self.cursor < n:
            self.cursor += 1
            return self.tokens[self.cursor - 1]
        return self.pad_id

    def below_target(self) -> bool:
        f = np.float32
        return bool(f(self.n_pad) < f(self.target) * f(max(self.n_steps, 1)))
