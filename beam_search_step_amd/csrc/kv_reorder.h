// kv_reorder.h -- part of libbeamstep.so, included once by beamstep.hip.
//
// The contiguous KV-cache reorder: K3.
#pragma once

namespace {

// ---------------------------------------------------------------------------
// K3: in-place KV reorder
// ---------------------------------------------------------------------------

// One wave per workgroup. With each step's reorder on a cold cache (20 steps
// spread over the search, three runs each): 9,888-9,915 beam steps/s at the
// Llama-3-8B shape against 9,723-9,762 with 128 threads and 9,380-9,574 with
// 256; at the wide shape (W = 16) 2,153-2,158 against 2,117-2,145 and
// 2,112-2,134; Transformer-base within noise.
constexpr int kK3Threads = 64;

struct K3Args {
  char* planes[kMaxPlanesPerLaunch];
  int64_t row_stride;   // bytes
  int64_t pos_stride;   // bytes
  int64_t base_off;     // pos_offset * pos_stride, bytes
  int64_t words;        // words per row to move: gen_len * words_per_pos
  int64_t words_per_pos;
  int W;
  const int* plan;
};

template <int WORD>
struct Word;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
template <>
struct Word<16> {
  using type = u32x4;
};
template <>
struct Word<4> {
  using type = uint32_t;
};

// One thread's part of the reorder: load its words of every distinct parent,
// then store them to every slot that copies that parent. FULL: all NP words
// are in range, so no access needs a guard (and none sits in a branch).
template <int WMAX, typename WT, int NP, bool FULL>
__device__ __forceinline__ void move_words(char* base, int64_t row0, int64_t row_stride,
                                           const int64_t (&off)[NP], int64_t e0, int64_t words,
                                           int nsrc, const int (&src)[WMAX],
                                           const int (&dmask)[WMAX]) {
  bool ok[NP];
#pragma unroll
  for (int k = 0; k < NP; ++k) ok[k] = FULL || e0 + (int64_t)k * kK3Threads < words;
  WT v[NP][WMAX];
#pragma unroll
  for (int q = 0; q < WMAX; ++q) {
    if (q < nsrc) {
      const char* from = base + (row0 + src[q]) * row_stride;
#pragma unroll
      for (int k = 0; k < NP; ++k)
        if (ok[k]) v[k][q] = __builtin_nontemporal_load(reinterpret_cast<const WT*>(from + off[k]));
    }
  }
  // In place: a destination row may be another copy's parent. No other thread
  // touches this thread's words (the offsets are unique per thread, item and
  // plane), so it is enough that every load of this thread has returned before
  // its first store: s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their
  // no-wait maxima).
  __builtin_amdgcn_s_waitcnt(0x0F70);
  // Between destination slots: for W <= 4 a thread waits for its stores after
  // each slot; for wider beams the stores to all slots issue back to back.
  // Measured with each step's reorder on a cold cache: at W = 16 (V = 250000)
  // 5.69-5.74 TB/s with no wait against 5.58-5.60 after every fourth slot and
  // 5.17-5.22 after every slot; at W = 4 (Llama-3-8B shape, three runs each)
  // 5.81-5.88 TB/s waiting after every slot against 5.78-5.86 with no wait.
  // Only the wait above, before the first store, matters for correctness.
#pragma unroll
  for (int q = 0; q < WMAX; ++q) {
    for (int m = dmask[q]; m; m &= m - 1) {
      char* dst = base + (row0 + __builtin_ctz(m)) * row_stride;
      // streaming stores: the moved rows are not read again by this launch,
      // and keeping them out of the caches measured ~10% faster end to end
#pragma unroll
      for (int k = 0; k < NP; ++k)
        if (ok[k]) __builtin_nontemporal_store(v[k][q], reinterpret_cast<WT*>(dst + off[k]));
      if constexpr (WMAX <= 4) __builtin_amdgcn_s_waitcnt(0x0F70);
    }
  }
}

// Parent reads and moved-slot writes both carry the nontemporal hint: every
// word is read once and written once per launch, and in a decoder the model's
// forward pass (weights and the whole KV cache) runs between two reorders, so
// nothing a launch leaves in the 256 MB Infinity Cache is there for the next.
// Measured with every step's reorder on a cold cache (the Llama-3-8B shape,
// 20 steps spread over the 200-step search): nontemporal parent reads 5.93
// TB/s against 5.35 with plain ones; plain stores 5.11.
//
// Work order: grid order. The hardware hands consecutive workgroups (x
// fastest, then y, z) to the 8 XCDs in turn, so every XCD streams every eighth
// tile of every row span, and every item's share is spread over all XCDs.
// Giving each XCD whole planes instead (workgroup k of XCD i doing the k-th of
// the i-th eighth of the grid) measured 1.3% faster when the previous step's
// rows were still in the cache, but slower on a cold cache (5.79 against 5.93
// TB/s).
template <int WMAX, int WORD, int NP, bool CONTIG>
__global__ __launch_bounds__(kK3Threads) void k3_kv_reorder(K3Args a) {
  using WT = typename Word<WORD>::type;
  const uint32_t bx = blockIdx.x, b = blockIdx.y, bz = blockIdx.z;
  const int* plan = a.plan + b * kPlanStride;
  // the whole plan is read up front, in one batch of scalar loads: a plan read
  // after a store would be a vector load whose wait also waits for every
  // store issued before it
  const int nsrc = plan[0], ndst = plan[1];
  int src[WMAX], dmask[WMAX];
#pragma unroll
  for (int q = 0; q < WMAX; ++q) {
    const int s0 = plan[2 + q], m0 = plan[2 + kMaxBeam + q];
    src[q] = q < nsrc ? s0 : 0;
    dmask[q] = q < nsrc ? m0 : 0;
  }
  if (ndst == 0) return;
  char* base = a.planes[bz] + a.base_off;
  const int64_t row0 = (int64_t)b * a.W;

  int64_t off[NP];
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    const int64_t e = ((int64_t)bx * NP + k) * kK3Threads + threadIdx.x;
    if (CONTIG) {
      off[k] = e * WORD;
    } else {
      const int64_t pos = e / a.words_per_pos;
      off[k] = pos * a.pos_stride + (e - pos * a.words_per_pos) * WORD;
    }
  }
  // every word of the tile is in range (uniform), except in the last tile
  const int64_t e0 = (int64_t)bx * NP * kK3Threads + threadIdx.x;
  if ((int64_t)(bx + 1) * NP * kK3Threads <= a.words)
    move_words<WMAX, WT, NP, true>(base, row0, a.row_stride, off, e0, a.words, nsrc, src, dmask);
  else
    move_words<WMAX, WT, NP, false>(base, row0, a.row_stride, off, e0, a.words, nsrc, src,
                                    dmask);
}

}  // namespace
