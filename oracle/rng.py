"""Counter-based random streams for the per-head rotation and projection state.

The method draws one random orthogonal rotation and one Gaussian projection per
(layer, KV head) and keeps them fixed ("5x Faster LLM Inference? ...",
"Example 1: Complete Generation Pipeline": a rotation precomputed and fixed per
head; "How 0xsero/turboquant works", "Compression Pipeline": rotation and
projection state).  The pages do not say how the state is drawn, so both the
oracle and the library implement the same published generators, each from its
definition:

* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014; constants as in Vigna's reference C code): a
  Weyl sequence with increment 0x9E3779B97F4A7C15 passed through a 64-bit
  mixing function.
* Box-Muller (Box and Muller, 1958): two uniforms -> two N(0, 1) variates.

Stream key for (seed, layer, head, tag):
    s0 = mix64(mix64(mix64(mix64(seed) ^ layer) ^ head) ^ tag)
then draw with SplitMix64 from state s0.  tag 1 = rotation, tag 2 = projection.

Uniforms: u1 = ((x >> 11) + 1) * 2**-53 in (0, 1],  u2 = (x >> 11) * 2**-53 in
[0, 1), u1 drawn first.  z0 = sqrt(-2 ln u1) cos(2 pi u2) is emitted before
z1 = sqrt(-2 ln u1) sin(2 pi u2).  The transcendental functions are the
platform libm's (Python's math module), evaluated in the order written.
"""

import math

MASK64 = (1 << 64) - 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15
TAG_ROTATION = 1
TAG_PROJECTION = 2
TAG_SIGNS = 3  # random sign diagonal of the structured (Hadamard) rotation


def mix64(z):
    """SplitMix64 output function (variant 13 of Stafford's mixer)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


class SplitMix64:
    def __init__(self, state):
        self.state = state & MASK64

    def next_u64(self):
        self.state = (self.state + GOLDEN_GAMMA) & MASK64
        return mix64(self.state)


def stream_key(seed, layer, head, tag):
    s = mix64(seed & MASK64)
    s = mix64(s ^ (layer & MASK64))
    s = mix64(s ^ (head & MASK64))
    s = mix64(s ^ (tag & MASK64))
    return s


def gaussians(seed, layer, head, tag, count):
    """First `count` N(0,1) draws of the (seed, layer, head, tag) stream."""
    g = SplitMix64(stream_key(seed, layer, head, tag))
    out = []
    two_pi = 2.0 * math.pi
    while len(out) < count:
        u1 = ((g.next_u64() >> 11) + 1) * (2.0 ** -53)
        u2 = (g.next_u64() >> 11) * (2.0 ** -53)
        r = math.sqrt(-2.0 * math.log(u1))
        theta = two_pi * u2
        out.append(r * math.cos(theta))
        out.append(r * math.sin(theta))
    return out[:count]


def random_signs(seed, layer, head, count):
    """count values in {+1, -1} from the tag-3 stream: +1 when the top bit of the
    next SplitMix64 output is 0."""
    g = SplitMix64(stream_key(seed, layer, head, TAG_SIGNS))
    return [1.0 if (g.next_u64() >> 63) == 0 else -1.0 for _ in range(count)]
