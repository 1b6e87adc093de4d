"""Plain Python model of page-budget admission and lazy page assignment.

TEST INFRASTRUCTURE ONLY.  Only the tests may import this module; it shares no
code with the library's scheduler and imports nothing from it.

What it models, and where the pages say so (web pages describing the
samir-vllm teaching engine):
  [README] "6 Hours of YouTube and 85 handtyped pages of notes on LLM
           Inference - Start here" (memedata.com copy of the project README),
           paragraphs on admission, FIFO waiting and --stats.
  [NF]     news-factory.app article, section "How does the engine manage KV
           cache memory?".
  [RR]     roxreport.com article, paragraph on admission credits.

* Budget: a request reserves room for its longest processed prefix,
  prompt_tokens + allowed_new_tokens - 1 tokens (the last predicted token is
  returned without being processed), rounded up to 16-token pages in each of
  the layers; the allowed output is max_new_tokens clamped to the context
  ([README] admission paragraph).
* Credits are separate from physical pages; pages are assigned only when a
  position needs one ([README]; [RR]).
* Waiting requests are admitted in first-in, first-out order when their budget
  fits beside the active ones; a request whose budget exceeds the whole pool is
  rejected ([README]; [NF]).
* Finishing (also early) releases the assigned pages and the unused credits
  ([README]; [RR]).
* Continuous mode admits as credits free up; static mode admits the next group
  only after the whole current group has finished ([README]; [NF]).
* Statistics: pool size, peak active requests, largest decode batch, peak
  assigned pages, admission waits, free pages ([README] --stats paragraph).

Readings where the pages are silent:
  * FIFO is strict: when the oldest waiting request does not fit, no younger
    one is admitted ahead of it.
  * "admission waits" counts requests that could not be admitted by the first
    admission pass after they were submitted.
  * a static group is every waiting request that fits, in FIFO order, taken
    when no request is active.
  * physical pages are handed out lowest free page id first.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

PAGE_TOKENS = 16


def budget_pages(prompt_tokens: int, max_new_tokens: int, context: int, n_layers: int) -> int:
    """Pages a request reserves: its longest processed prefix in 16-token pages, in every layer."""
    allowed_new = min(max_new_tokens, context - prompt_tokens)
    processed = prompt_tokens + allowed_new - 1
    return -(-processed // PAGE_TOKENS) * n_layers


@dataclass
class Request:
    rid: int
    prompt: int
    max_new: int
    credits: int
    limit: int                  # longest processed prefix (tokens)
    length: int = 0             # positions backed by pages
    tables: List[List[int]] = field(default_factory=list)  # [layer][block] page ids
    waited: bool = False


class SchedModel:
    def __init__(self, pool_pages: int, n_layers: int = 16, context: int = 2048, static: bool = False):
        self.pool = pool_pages
        self.layers = n_layers
        self.context = context
        self.static = static
        self.free = list(range(pool_pages))       # free page ids; lowest first out
        self.credits_free = pool_pages
        self.waiting: List[Request] = []
        self.active: Dict[int, Request] = {}
        self.next_id = 0
        self.stats = dict(pool_pages=pool_pages, peak_active=0, largest_decode_batch=0,
                          peak_assigned_pages=0, admission_waits=0, rejected=0, completed=0)

    # -------------------------------------------------------------- requests
    def submit(self, prompt: int, max_new: int) -> Optional[int]:
        """Queue a request; None when it is rejected (budget above the whole pool)."""
        assert 1 <= prompt < self.context and max_new >= 1
        credits = budget_pages(prompt, max_new, self.context, self.layers)
        if credits > self.pool:
            self.stats["rejected"] += 1
            return None
        r = Request(self.next_id, prompt, max_new, credits,
                    prompt + min(max_new, self.context - prompt) - 1,
                    tables=[[] for _ in range(self.layers)])
        self.next_id += 1
        self.waiting.append(r)
        return r.rid

    def admit(self) -> List[int]:
        """Admit waiting requests by the mode's rule; returns their ids in order."""
        out = []
        if self.static and self.active:
            pass
        else:
            while self.waiting and self.waiting[0].credits <= self.credits_free:
                r = self.waiting.pop(0)
                self.credits_free -= r.credits
                self.active[r.rid] = r
                out.append(r.rid)
        for r in self.waiting:  # every request still waiting after a pass has waited
            if not r.waited:
                r.waited = True
                self.stats["admission_waits"] += 1
        self.stats["peak_active"] = max(self.stats["peak_active"], len(self.active))
        return out

    def grow(self, rid: int, new_length: int) -> bool:
        """Back positions 0..new_length-1 with pages in every layer; False beyond the budget."""
        r = self.active[rid]
        if new_length > r.limit:
            return False
        need = -(-new_length // PAGE_TOKENS)
        for table in r.tables:
            while len(table) < need:
                self.free.sort()
                table.append(self.free.pop(0))
        r.length = max(r.length, new_length)
        assigned = self.pool - len(self.free)
        self.stats["peak_assigned_pages"] = max(self.stats["peak_assigned_pages"], assigned)
        return True

    def decode_batch(self, n: int) -> None:
        self.stats["largest_decode_batch"] = max(self.stats["largest_decode_batch"], n)

    def finish(self, rid: int) -> None:
        r = self.active.pop(rid)
        for table in r.tables:
            self.free.extend(table)
        self.credits_free += r.credits
        self.stats["completed"] += 1

    # -------------------------------------------------------------- views
    def assigned_pages(self) -> int:
        return self.pool - len(self.free)

    def snapshot(self) -> dict:
        d = dict(self.stats)
        d.update(free_pages=len(self.free), assigned_pages=self.assigned_pages(), active=len(self.active),
                 waiting=len(self.waiting), credits_free=self.credits_free)
        return d
