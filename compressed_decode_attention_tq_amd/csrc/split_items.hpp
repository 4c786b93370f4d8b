// Work items of the split-K decode launches (device side).
//
// A launch has one workgroup per (sequence b, split s, KV head g) of the plan's
// bound: batch x n_splits x Hkv, as a one-dimensional grid.  Workgroups are
// handed to the eight XCDs round-robin by linear id, and the device dispatches
// them in id order, so the order of items in the id space decides how the
// work spreads over the XCDs and what runs last.  In both orders below the KV
// head is the fastest index: the heads of a sequence have the same length, so
// at 8 KV heads every XCD gets exactly the same work (one head each), and at
// fewer heads it gets whole heads of interleaved items.
//
// Plain order (grids that fit in one round of resident workgroups): the id is
// g + Hkv (s + n_splits b); items past a sequence's end exit at once.
//
// Work list (larger grids, ragged batches): the live items only, numbered
// densely at the front of the id space, the splits that are whole first and
// each sequence's shorter last split after them, so that the workgroups that
// start last are the short ones.  Each wave derives its item from seq_lens on
// its own: per-sequence counts of whole and last splits, a prefix sum over the
// wave, and a search for the id; no table and no extra launch.  The count of a
// sequence uses min(seq_len, n_splits x split_tokens), so no split index
// reaches n_splits whatever the lengths hold.
#pragma once

#include <hip/hip_runtime.h>

namespace tq {

struct SplitItem {
  int b;      // sequence (-1: no work)
  int split;  // split index within the sequence
  int g;      // KV head
};

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_prefix_sum(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    x += lane >= d ? y : 0;
  }
  return x;
}

// Item of this workgroup (wave-uniform; every lane of the wave must call it).
__device__ __forceinline__ SplitItem split_item(const int* __restrict__ seq_lens, int batch, int Hkv,
                                                int split_tokens, int n_splits, bool work_list) {
  const unsigned id = blockIdx.x;
  SplitItem it;
  it.g = static_cast<int>(id % static_cast<unsigned>(Hkv));
  const unsigned p = id / static_cast<unsigned>(Hkv);
  if (!work_list) {
    it.split = static_cast<int>(p % static_cast<unsigned>(n_splits));
    it.b = static_cast<int>(p / static_cast<unsigned>(n_splits));
    return it;
  }
  constexpr int kPer = 4;              // sequences per lane and pass
  constexpr int kSpan = 64 * kPer;     // sequences per pass
  const int lane = threadIdx.x & 63;
  // n_splits x split_tokens < 2^31 + split_tokens: fits 32 unsigned bits
  const unsigned S = static_cast<unsigned>(split_tokens);
  const unsigned cap = static_cast<unsigned>(n_splits) * S;
  // whole and last-split counts of the lane's sequences base + kPer lane + k
  auto counts = [&](int base, int* whole, int* last) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = base + kPer * lane + k;
      const int t0 = i < batch ? seq_lens[i] : 0;
      const unsigned t = t0 <= 0 ? 0u : min(static_cast<unsigned>(t0), cap);
      const unsigned w = t / S;
      whole[k] = static_cast<int>(w);
      last[k] = t != w * S ? 1 : 0;
    }
  };
  int whole[kPer], last[kPer];
  // total of whole splits (one pass when the batch fits one)
  long long n_whole = 0;
  for (int base = 0; base < batch; base += kSpan) {
    counts(base, whole, last);
    const int s = wave_prefix_sum(whole[0] + whole[1] + whole[2] + whole[3]);
    n_whole += __builtin_amdgcn_readlane(s, 63);
  }
  const bool in_whole = static_cast<long long>(p) < n_whole;
  const long long key = in_whole ? static_cast<long long>(p) : static_cast<long long>(p) - n_whole;
  long long carry = 0;
  for (int base = 0; base < batch; base += kSpan) {
    if (batch > kSpan) counts(base, whole, last);  // else still held from the first pass
    int v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) v[k] = in_whole ? whole[k] : last[k];
    const int own = v[0] + v[1] + v[2] + v[3];
    const int incl = wave_prefix_sum(own);
    const int tot = __builtin_amdgcn_readlane(incl, 63);
    if (key < carry + tot) {
      // first lane whose running count passes the key
      const unsigned long long m = __ballot(carry + incl > key);
      const int l = __builtin_amdgcn_readfirstlane(__ffsll(static_cast<long long>(m)) - 1);
      long long acc = carry + __builtin_amdgcn_readlane(incl, l) - __builtin_amdgcn_readlane(own, l);
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int vk = __builtin_amdgcn_readlane(v[k], l);
        if (key < acc + vk) {
          it.b = base + kPer * l + k;
          it.split = in_whole ? static_cast<int>(key - acc) : __builtin_amdgcn_readlane(whole[k], l);
          return it;
        }
        acc += vk;
      }
    }
    carry += tot;
  }
  it.b = -1;
  it.split = 0;
  return it;
}

}  // namespace tq
