// kv_reorder.h -- part of libbeamstep.so, included once by beamstep.hip.
//
// The contiguous KV-cache reorder: K3.
#pragma once

namespace {

// ---------------------------------------------------------------------------
// K3: in-place KV reorder
// ---------------------------------------------------------------------------

struct K3Args {
  char* planes[kMaxPlanesPerLaunch];
  int64_t row_stride;   // bytes
  int64_t pos_stride;   // bytes
  int64_t base_off;     // pos_offset * pos_stride, bytes
  int64_t words;        // words per row to move: gen_len * words_per_pos
  int64_t words_per_pos;
  int W;
  const int* plan;
  int whole_planes;     // 1: XCD i takes the i-th eighth of the planes
  int stream_loads;     // 1: parent words are read with the nontemporal hint
  int64_t region_bytes_per_plane;  // rows x gen_len x bytes_per_pos (host side)
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
                                           const int (&dmask)[WMAX], bool stream_loads) {
  bool ok[NP];
#pragma unroll
  for (int k = 0; k < NP; ++k) ok[k] = FULL || e0 + (int64_t)k * kK3Threads < words;
  WT v[NP][WMAX];
  if (stream_loads) {  // uniform: one loop each way, so no load waits on a branch
#pragma unroll
    for (int q = 0; q < WMAX; ++q) {
      if (q < nsrc) {
        const char* from = base + (row0 + src[q]) * row_stride;
#pragma unroll
        for (int k = 0; k < NP; ++k)
          if (ok[k]) v[k][q] = __builtin_nontemporal_load(reinterpret_cast<const WT*>(from + off[k]));
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < WMAX; ++q) {
      if (q < nsrc) {
        const char* from = base + (row0 + src[q]) * row_stride;
#pragma unroll
        for (int k = 0; k < NP; ++k)
          if (ok[k]) v[k][q] = *reinterpret_cast<const WT*>(from + off[k]);
      }
    }
  }
  // In place: a destination row may be another copy's parent. No other thread
  // touches this thread's words (the offsets are unique per thread, item and
  // plane), so it is enough that every load of this thread has returned before
  // its first store: s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their
  // no-wait maxima).
  __builtin_amdgcn_s_waitcnt(0x0F70);
  // Between destination slots a thread waits for its stores: after every slot
  // for W <= 4 (measured faster than keeping them all in flight), after every
  // fourth for wider beams, whose many destinations otherwise serialise on
  // the store round trip (measured 2% faster at W = 16, 2% slower at W = 4).
  // Only the wait above, before the first store, matters for correctness.
  constexpr int kSlotsPerWait = WMAX >= 8 ? 4 : 1;
  int nst = 0;
#pragma unroll
  for (int q = 0; q < WMAX; ++q) {
    for (int m = dmask[q]; m; m &= m - 1) {
      char* dst = base + (row0 + __builtin_ctz(m)) * row_stride;
      // streaming stores: the moved rows are not read again by this launch,
      // and keeping them out of the caches measured ~10% faster end to end
#pragma unroll
      for (int k = 0; k < NP; ++k)
        if (ok[k]) __builtin_nontemporal_store(v[k][q], reinterpret_cast<WT*>(dst + off[k]));
      if (++nst % kSlotsPerWait == 0) __builtin_amdgcn_s_waitcnt(0x0F70);
    }
  }
}

// Parent reads. Plain loads let a launch reuse what the previous step's
// launch left in the 256 MB Infinity Cache (the rows it wrote are often this
// step's parents): at the Llama-3-8B shape, t = 50..100, they ran at 6.7-7.5
// TB/s against 5.3-5.6 with the nontemporal hint. When the launch's region
// (rows x positions x planes) is several times the cache nothing survives to
// the next launch, and reads that do not allocate leave the launch's own
// lines in place: 4.5-7% faster per launch at the wide shape, t >= 128. The
// host sets stream_loads when that region exceeds 1 GiB.
//
// Work order. The hardware hands consecutive workgroups (x fastest, then y,
// z) to the 8 XCDs in turn, so in grid order every XCD takes every eighth
// tile of every row span. With whole_planes set (the launch's plane count a
// multiple of 8, its workgroups fewer than 2^32), the workgroup that XCD i
// receives k-th does the k-th workgroup of the i-th eighth of the grid
// instead: XCD i streams planes [i*planes/8, (i+1)*planes/8) from end to end,
// all items of each, and every XCD still gets the same share of every item.
// Measured 1.3% faster than grid order with 64 planes of 8 items; an eighth
// that does not end on a plane boundary lets some XCDs take most of the
// heavy or unfinished items, and was slower (12 planes: 1.5% with 16 items,
// 9% when many items had finished).
template <int WMAX, int WORD, int NP, bool CONTIG>
__global__ __launch_bounds__(kK3Threads) void k3_kv_reorder(K3Args a) {
  using WT = typename Word<WORD>::type;
  uint32_t bx = blockIdx.x, b = blockIdx.y, bz = blockIdx.z;
  if (a.whole_planes) {
    const uint32_t gx = gridDim.x, gy = gridDim.y;
    const uint32_t lin = bx + gx * (b + gy * bz);
    const uint32_t eighth = (gx * gy * gridDim.z) >> 3;
    const uint32_t l2 = (lin & 7) * eighth + (lin >> 3);
    const uint32_t pl = l2 / gx;
    bx = l2 - pl * gx;
    bz = pl / gy;
    b = pl - bz * gy;
  }
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
    move_words<WMAX, WT, NP, true>(base, row0, a.row_stride, off, e0, a.words, nsrc, src, dmask,
                                   a.stream_loads);
  else
    move_words<WMAX, WT, NP, false>(base, row0, a.row_stride, off, e0, a.words, nsrc, src,
                                    dmask, a.stream_loads);
}

}  // namespace
