"""Seeded synthetic packed-sequence layouts (per-token metadata tracks).

This module only *generates inputs*: it decides where samples, spans, groups and
generated (noise) spans sit in a packed sequence and writes the four per-token
integer tracks that describe them.  It holds none of the attention arithmetic,
none of the mask predicate and none of the planner; both the CPU oracle and the
GPU path consume what it returns.

Track encoding (MARBLE page, section "01 Packed multimodal masks", the paragraph
after the mode table): every token carries four integers
  sample  - id of the packed sample the token belongs to,
  seg     - id shared by all tokens of one bidirectional span; one id shared by
            every span of a group; -1 for causal / window tokens,
  noise   - id of a generated (noise) span; -1 for every other token,
  pos     - the token's original packed position (global index, strictly
            increasing in the original order).
plus one per-layer scalar W (the sliding window; WINDOW_INF for global layers).

Length draws for packed text follow the heavy-tailed corpus the Libra page
describes (section 1: median 644 tokens); the lognormal with sigma 1.5 and the
16384-token cap complete the recipe (the page gives the median only).
"""
from __future__ import annotations

from dataclasses import dataclass, field
import numpy as np

WINDOW_INF = 0x7FFFFFFF


@dataclass
class Layout:
    name: str
    sample: np.ndarray          # int32[N]
    seg: np.ndarray             # int32[N]
    noise: np.ndarray           # int32[N]
    pos: np.ndarray             # int32[N]
    window: int                 # >= 1, WINDOW_INF for global layers
    ranks: int                  # ring degree P
    order: str                  # "contiguous" | "ptrr" | "explicit"
    block: int = 128            # tile / PTRR block size in tokens
    hq: int = 1
    hkv: int = 1
    d: int = 128
    seed: int = 0
    backward: bool = False
    # human-readable span list: (start, end, mode, sample) for docs / tests
    spans: list = field(default_factory=list)
    # order "explicit": new block position -> original block
    block_perm: object = None

    @property
    def n(self) -> int:
        return int(self.sample.shape[0])

    def tracks(self):
        return self.sample, self.seg, self.noise, self.pos


def lognormal_lengths(rng: np.random.Generator, median: float, sigma: float,
                      cap: int, count: int) -> np.ndarray:
    """Draw `count` integer lengths: clamp(rint(exp(ln(median) + sigma*z)), 1, cap)."""
    z = rng.standard_normal(count)
    return np.clip(np.rint(np.exp(np.log(median) + sigma * z)), 1, cap).astype(np.int64)


def _finish(name, sample, seg, noise, window, ranks, order, spans, **kw) -> Layout:
    n = len(sample)
    return Layout(name=name,
                  sample=np.asarray(sample, np.int32),
                  seg=np.asarray(seg, np.int32),
                  noise=np.asarray(noise, np.int32),
                  pos=np.arange(n, dtype=np.int32),
                  window=window, ranks=ranks, order=order, spans=spans, **kw)


class _Builder:
    """Appends spans to a packed sequence, truncating at a fixed capacity."""

    def __init__(self, n: int):
        self.n = n
        self.sample = np.empty(n, np.int32)
        self.seg = np.empty(n, np.int32)
        self.noise = np.empty(n, np.int32)
        self.fill = 0
        self.spans = []

    @property
    def full(self) -> bool:
        return self.fill >= self.n

    def add(self, length: int, sample: int, seg: int, noise: int, mode: str) -> None:
        length = int(min(length, self.n - self.fill))
        if length <= 0:
            return
        a, b = self.fill, self.fill + length
        self.sample[a:b] = sample
        self.seg[a:b] = seg
        self.noise[a:b] = noise
        self.spans.append((a, b, mode, sample))
        self.fill = b


def ring_toy() -> Layout:
    """16 tokens, one sample, one bidirectional span (no mask), 4 contiguous shards.

    The tutorial ring simulation on the NumPy ring page uses N=16, d=8, P=4 and
    plain unmasked attention; an unmasked sequence is one sample whose tokens all
    share one bidirectional span.
    """
    n = 16
    return _finish("ring_toy", [0] * n, [0] * n, [-1] * n, WINDOW_INF, 4, "contiguous",
                   [(0, n, "full", 0)], hq=1, hkv=1, d=8, seed=0)


def packed_text(n: int = 32768, seed: int = 2, ranks: int = 8) -> Layout:
    """Packed text documents, block-diagonal causal (one sample per document)."""
    rng = np.random.default_rng(seed)
    b = _Builder(n)
    s = 0
    while not b.full:
        ln = lognormal_lengths(rng, 644, 1.5, 16384, 1)[0]
        b.add(ln, s, -1, -1, "causal")
        s += 1
    return _finish("packed_text_32k", b.sample, b.seg, b.noise, WINDOW_INF, ranks, "ptrr",
                   b.spans, hq=32, hkv=8, d=128, seed=seed)


def packed_multimodal(n: int = 65536, seed: int = 3, ranks: int = 8,
                      p_generated: float = 0.3) -> Layout:
    """Samples of [text, image A, text, image B, text].

    Text is causal (lognormal lengths, median 512).  Images are 1024 tokens; the
    two images of a sample form one bidirectional group (one shared seg id).  Each
    image is independently a generated image with probability p_generated: it
    then carries its own noise id, so no later token of its sample reads it.
    """
    rng = np.random.default_rng(seed)
    b = _Builder(n)
    s = seg_id = noise_id = 0
    while not b.full:
        t = lognormal_lengths(rng, 512, 1.5, 16384, 3)
        gen = rng.random(2) < p_generated
        group = seg_id
        seg_id += 1
        b.add(t[0], s, -1, -1, "causal")
        for img in range(2):
            nz = -1
            if gen[img]:
                nz = noise_id
                noise_id += 1
            b.add(1024, s, group, nz, "noise-group" if nz >= 0 else "group")
            b.add(t[img + 1], s, -1, -1, "causal")
        s += 1
    return _finish("packed_multimodal_64k", b.sample, b.seg, b.noise, WINDOW_INF, ranks,
                   "ptrr", b.spans, hq=24, hkv=24, d=128, seed=seed)


def sliding_window(n: int = 131072, clip: int = 16384, clips_per_doc: int = 4,
                   window: int = 4096, ranks: int = 8) -> Layout:
    """Video-like clips under a sliding-window layer.

    Each clip is one bidirectional span; across clips the window mode applies
    (0 <= pos_q - pos_k < W); a document is `clips_per_doc` consecutive clips and
    no document reads another.  Contiguous shards, so with n/ranks == clip every
    shard is one clip.
    """
    b = _Builder(n)
    c = 0
    while not b.full:
        b.add(clip, c // clips_per_doc, c, -1, "full+window")
        c += 1
    return _finish("sliding_window_128k", b.sample, b.seg, b.noise, window, ranks,
                   "contiguous", b.spans, hq=16, hkv=4, d=128, seed=4, backward=True)


def long_mixed(n: int = 1048576, seed: int = 5, ranks: int = 8, clip: int = 16384) -> Layout:
    """Causal text documents (median 644) alternating with bidirectional clips.

    Text documents are drawn until at least `clip` text tokens have been placed
    since the last clip; then one clip (its own sample, one bidirectional span).
    """
    rng = np.random.default_rng(seed)
    b = _Builder(n)
    s = seg_id = 0
    while not b.full:
        since = 0
        while since < clip and not b.full:
            ln = lognormal_lengths(rng, 644, 1.5, 16384, 1)[0]
            b.add(ln, s, -1, -1, "causal")
            s += 1
            since += int(ln)
        b.add(clip, s, seg_id, -1, "full")
        s += 1
        seg_id += 1
    return _finish("long_mixed_1m", b.sample, b.seg, b.noise, WINDOW_INF, ranks, "ptrr",
                   b.spans, hq=16, hkv=4, d=128, seed=seed, backward=True)


def video_group(n: int = 131072, seed: int = 6, ranks: int = 8, frame: int = 196, stamp: int = 8,
                min_frames: int = 16, max_frames: int = 96) -> Layout:
    """Video samples whose frames form one bidirectional group (MARBLE section
    01: the group mode, as Molmo2 combines all image spans of a sample).

    Each sample: a causal text prompt (16-128 tokens), then per frame a causal
    timestamp of `stamp` tokens followed by the frame (`frame` tokens), then a
    causal answer (16-256 tokens).  Every frame of a sample carries the
    sample's one seg id, so frames see each other in both directions but not
    the timestamps between them.  Frame counts are drawn uniformly in
    [min_frames, max_frames]; the last sample is cut at n.  The pages give no
    frame or text sizes; 196 tokens is a 14 x 14 patch grid.
    """
    rng = np.random.default_rng(seed)
    b = _Builder(n)
    s = 0
    while not b.full:
        b.add(int(rng.integers(16, 129)), s, -1, -1, "causal")
        for _ in range(int(rng.integers(min_frames, max_frames + 1))):
            b.add(stamp, s, -1, -1, "causal")
            b.add(frame, s, s, -1, "group")
        b.add(int(rng.integers(16, 257)), s, -1, -1, "causal")
        s += 1
    return _finish("video_group_128k", b.sample, b.seg, b.noise, WINDOW_INF, ranks, "ptrr", b.spans,
                   hq=16, hkv=4, d=128, seed=seed, backward=True)


def permuted(lay: Layout, new_to_orig, name: str = None) -> Layout:
    """The layout with its tokens permuted (position i holds token
    new_to_orig[i]); every token keeps its tracks, its position included."""
    import dataclasses
    idx = np.asarray(new_to_orig, np.int64)
    return dataclasses.replace(lay, name=name or lay.name + "_permuted", sample=lay.sample[idx],
                               seg=lay.seg[idx], noise=lay.noise[idx], pos=lay.pos[idx], spans=[])


CONFIGS = {
    1: ring_toy,
    2: packed_text,
    3: packed_multimodal,
    4: sliding_window,
    5: long_mixed,
    6: video_group,
}


def config(idx: int) -> Layout:
    return CONFIGS[idx]()


def random_small(rng: np.random.Generator, n: int, max_span: int = 12,
                 window_choices=(1, 2, 3, 5, 8, WINDOW_INF)) -> Layout:
    """Tiny random layouts exercising all five modes, for brute-force checks.

    Each sample is a random list of spans; a span's mode is one of causal, full,
    noise, group, window.  Group spans of one sample share one seg id; full and
    noise spans get their own seg id; noise spans also get their own noise id.
    """
    b = _Builder(n)
    s = seg_id = noise_id = 0
    window = int(rng.choice(np.asarray(window_choices, dtype=np.int64)))
    while not b.full:
        nspans = int(rng.integers(1, 5))
        group = None
        for _ in range(nspans):
            mode = ["causal", "full", "noise", "group", "window"][int(rng.integers(0, 5))]
            ln = int(rng.integers(1, max_span + 1))
            if mode in ("causal", "window"):
                b.add(ln, s, -1, -1, mode)
            elif mode == "full":
                b.add(ln, s, seg_id, -1, mode)
                seg_id += 1
            elif mode == "noise":
                b.add(ln, s, seg_id, noise_id, mode)
                seg_id += 1
                noise_id += 1
            else:
                if group is None:
                    group = seg_id
                    seg_id += 1
                b.add(ln, s, group, -1, mode)
        s += 1
    return _finish("random_small", b.sample, b.seg, b.noise, window, 1, "contiguous",
                   b.spans)
