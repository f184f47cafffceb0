"""Working-set delta between consecutive agent steps, and the bounded page pool.

KVMem paper, Sec. 4.4 ("retrieval-aware hierarchical reuse"): with W_{t-1}
and W_t the working sets of two consecutive steps, the transition splits into
retained R_t = W_{t-1} & W_t, incoming L_t = W_t - W_{t-1} and outgoing
E_t = W_{t-1} - W_t. With G_{t-1} the blocks still resident in the bounded
GPU page pool, only L_t^physical = W_t - G_{t-1} must be staged in; the GPU
hits W_t & G_{t-1} keep their pages (V untouched; K re-encoded only when the
compact position changed). The displayed set equations were lost; these are
the set identities the prose states.

The pool itself (``PagePool``) is the plain model of G_t: a fixed number of
pages, one block per page. The pages say a page of a block outside the
current view can be reclaimed at once because the block keeps a lower-tier
copy (Sec. 4.4), and that freshly completed blocks stay GPU-resident after
prefill (Sec. 5); they do not say which page goes first. Reading taken: the
least recently used block outside the current view (the latest selection and
the blocks registered since), ties to the lower block id; free pages are used
before any block is evicted.
"""
from __future__ import annotations


def working_set_delta(W_prev, W_t, G_prev) -> dict:
    W_prev, W_t, G_prev = set(W_prev), set(W_t), set(G_prev)
    return {
        "retained": W_prev & W_t,
        "incoming": W_t - W_prev,
        "outgoing": W_prev - W_t,
        "hits": W_t & G_prev,
        "physical_in": W_t - G_prev,
    }


class PoolFull(Exception):
    """No free page and no resident block outside the current view."""


class PagePool:
    """G_t of KVMem Sec. 4.4 as a set of resident blocks with their last use.

    step counts working-set updates. A block's last use is the step of the
    last selection that contained it, or the step at which it was registered
    (prefilled). The current view is every resident block whose last use is
    the current step; only blocks outside it are evicted."""

    def __init__(self, n_pages: int):
        if n_pages < 1:
            raise ValueError("n_pages")
        self.n_pages = n_pages
        self.step = 0
        self.last_use: dict[int, int] = {}

    @property
    def resident(self) -> set:
        return set(self.last_use)

    def _victim(self) -> int:
        old = [(u, b) for b, u in self.last_use.items() if u < self.step]
        if not old:
            raise PoolFull
        return min(old)[1]

    def _room(self, n_new: int) -> None:
        """Raise PoolFull unless n_new more blocks fit (free pages plus blocks
        outside the current view)."""
        free = self.n_pages - len(self.last_use)
        old = sum(1 for u in self.last_use.values() if u < self.step)
        if n_new > free + old:
            raise PoolFull

    def register(self, blocks) -> list:
        """Freshly prefilled blocks become resident at the current step.
        All or nothing: PoolFull leaves the pool unchanged. Returns the blocks
        evicted to make room."""
        blocks = sorted(set(int(b) for b in blocks))
        new = [b for b in blocks if b not in self.last_use]
        self._room(len(new))
        evicted = []
        for b in blocks:
            if b not in self.last_use and len(self.last_use) == self.n_pages:
                v = self._victim()
                del self.last_use[v]
                evicted.append(v)
            self.last_use[b] = self.step
        return evicted

    def update(self, selection) -> dict:
        """One working-set update with the new view W_t = selection: hits keep
        their pages, misses (L_t^physical) take free pages, then pages of the
        least recently used blocks outside W_t."""
        W = sorted(set(int(b) for b in selection))
        if len(W) > self.n_pages:
            raise PoolFull
        G_prev = self.resident
        self.step += 1
        hits = [b for b in W if b in G_prev]
        misses = [b for b in W if b not in G_prev]
        for b in W:
            if b in self.last_use:
                self.last_use[b] = self.step
        evicted = []
        for b in misses:
            if len(self.last_use) == self.n_pages:
                v = self._victim()
                del self.last_use[v]
                evicted.append(v)
            self.last_use[b] = self.step
        return {"hits": hits, "misses": misses, "evicted": evicted, "G_prev": G_prev}

    def evict(self, blocks) -> None:
        for b in blocks:
            self.last_use.pop(int(b), None)
