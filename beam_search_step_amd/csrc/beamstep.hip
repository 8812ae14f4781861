// beamstep.hip -- HIP kernels and host runtime of libbeamstep.so (gfx950).
//
// One decode step of batched beam search ("llm_internals" 9.2.2: expand,
// score, prune, finalize; the batched section of "Transformers中的Beam
// Search高效实现") as three kernels per step, plus the verify step of
// blockwise parallel decoding ("Blockwise Parallel Decoding", section 3):
//
//   K1 expand_select   grid (tiles, rows). Streams each live row's logits once
//                      with 16-byte loads. Per (row, tile) it leaves the
//                      online softmax partial (max m, sum exp(x - m)) and the
//                      tile's W best raw logits ordered by (x desc, v asc).
//                      Log-softmax is monotone within a row, so the union of
//                      the tile lists holds the row's top-W candidates (the
//                      same argument as the coarse-to-fine selection in the
//                      LightSeq article, "层级式解码计算").
//   K2 merge_finalize  grid (B). Combines the partials into lse per row,
//                      forms cand = fp32(s + fp32(x - lse)) for the W*tiles*W
//                      listed candidates, takes the top-W by (cand desc, j
//                      asc), then runs the finalize sub-step: EOS selections
//                      into the finished set with the length penalty,
//                      compaction of live slots in rank order, backpointers,
//                      the stop rule, and the plan for the KV reorder.
//   K3 kv_reorder      grid (tiles, B, planes). Each thread reads one 16-byte
//                      word of every distinct parent row, waits, and writes it
//                      to every slot that moved, so swaps and cycles are safe
//                      in place and a shared parent is read once.
//   K4 verify          grid (tiles, rows) argmax partials (and, for the top-k
//                      criterion, counts of logits beating the proposal), then
//                      one wave per item merges them and forms the accepted
//                      prefix.
//   K5 finalize        grid (B). Final ranking and backtrace of the tokens.
//
// No matrix cores: nothing here is a dense contraction. Every kernel is bound
// by HBM bandwidth.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "beamstep.h"

#pragma clang fp contract(off)

namespace {

constexpr int kThreads = 256;           // workgroup size of K1, K2, K3, K4
constexpr int kWaves = kThreads / 64;   // wave64
constexpr int kMaxBeam = 16;
constexpr int kListCap = 1024;          // LDS candidate list of the top-W
constexpr int kGroups = kThreads / 16;  // 16-lane groups for the selection bound
constexpr int kMergeNE = 8;             // K2 candidates per thread per batch
constexpr int kPlanStride = 64;         // int32 words per item of the KV plan
constexpr int kK3Threads = 256;         // threads per KV-reorder workgroup
constexpr int kMaxPlanesPerLaunch = 128;
constexpr float kInf = __builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------

// Selection order: larger key first; equal keys go to the smaller index.
__device__ __forceinline__ bool better(float xa, int ia, float xb, int ib) {
  return xa > xb || (xa == xb && ia < ib);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Combine two (max, sum of exp(x - max)) partials of a log-sum-exp.
__device__ __forceinline__ void lse_combine(float& m, float& s, float m2, float s2) {
  float M = fmaxf(m, m2);
  if (M == -kInf) {
    m = -kInf;
    s = 0.0f;
    return;
  }
  float a = (m == -kInf) ? 0.0f : s * exp2f((m - M) * kLog2e);
  float c = (m2 == -kInf) ? 0.0f : s2 * exp2f((m2 - M) * kLog2e);
  m = M;
  s = a + c;
}

// ---------------------------------------------------------------------------
// wave reductions
// ---------------------------------------------------------------------------


// Candidate keys packed into one unsigned 64-bit word so that a plain unsigned
// maximum picks (score desc, index asc): the score's bits, mapped to an
// order-preserving unsigned code (-0 folded into +0 first, as fp compare
// treats them equal), above the inverted index. 0 is "no candidate" (below
// the code of every real score, -inf included).
__device__ __forceinline__ uint64_t pack_key(float x, int idx) {
  const uint32_t u = __float_as_uint(x + 0.0f);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)o << 32) | (uint32_t)(0xffffffffu - (uint32_t)idx);
}
__device__ __forceinline__ float key_score(uint64_t k) {
  const uint32_t o = (uint32_t)(k >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
__device__ __forceinline__ int key_index(uint64_t k) {
  return (int)(0xffffffffu - (uint32_t)k);
}

// One DPP step of a wave maximum: combine with the lane the control selects.
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max(uint64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xf, 0xf, false);
  const uint64_t o = ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
  return o > v ? o : v;
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}

// Maximum over the 64 lanes of a wave (uniform result). Within each row of 16
// lanes: quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror and
// row_mirror leave every lane with its row's maximum; the four rows are then
// combined through readlane.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max<0xb1>(v);
  v = dpp_max<0x4e>(v);
  v = dpp_max<0x141>(v);
  v = dpp_max<0x140>(v);
  uint64_t m = readlane_u64(v, 0);
  const uint64_t m1 = readlane_u64(v, 16), m2 = readlane_u64(v, 32), m3 = readlane_u64(v, 48);
  m = m1 > m ? m1 : m;
  m = m2 > m ? m2 : m;
  m = m3 > m ? m3 : m;
  return m;
}

// Float maximum and sum over a wave with the same DPP row steps, the four
// row results combined through readlane in a fixed order (uniform result;
// the sum is reproducible).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float wave_max_f(float v) {
  v = fmaxf(v, dpp_f<0xb1>(v));
  v = fmaxf(v, dpp_f<0x4e>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
__device__ __forceinline__ float wave_sum_f(float v) {
  v = v + dpp_f<0xb1>(v);
  v = v + dpp_f<0x4e>(v);
  v = v + dpp_f<0x141>(v);
  v = v + dpp_f<0x140>(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// The w_keep best keys (unique, 0 = none) held by a wave's lanes, C per lane:
// w_keep rounds of a wave maximum, each round over the keys below the
// previous round's winner. out[r] receives rank r (0 where there is none).
// Call with every lane of the wave; out is written by lane 0.
template <int C>
__device__ __forceinline__ void wave_topw(const uint64_t (&k)[C], int w_keep, uint64_t* out) {
  uint64_t prev = ~(uint64_t)0;
  for (int r = 0; r < w_keep; ++r) {
    uint64_t best = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) best = (k[c] < prev && k[c] > best) ? k[c] : best;
    best = wave_max_u64(best);
    if ((threadIdx.x & 63) == 0) out[r] = best;
    prev = best;
  }
}

// ---------------------------------------------------------------------------
// logits loading: EPT elements per thread, 16-byte vectors when aligned
// ---------------------------------------------------------------------------

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kVec = 4;
  __device__ static float load1(const float* p) { return *p; }
  __device__ static void loadv(const float* p, float* out) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    out[0] = v.x;
    out[1] = v.y;
    out[2] = v.z;
    out[3] = v.w;
  }
  __device__ static void unpack(const uint4& v, float* out) {  // 16 bytes: 4 elements
    out[0] = __uint_as_float(v.x);
    out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z);
    out[3] = __uint_as_float(v.w);
  }
};
template <>
struct Elem<uint16_t> {
  static constexpr int kVec = 8;
  __device__ static float load1(const uint16_t* p) { return bf16_to_f32(*p); }
  __device__ static void loadv(const uint16_t* p, float* out) {
    unpack(*reinterpret_cast<const uint4*>(p), out);
  }
  __device__ static void unpack(const uint4& v, float* out) {  // 16 bytes: 8 elements
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      out[2 * k] = __uint_as_float(w[k] << 16);
      out[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  }
};

// Element i of this thread's tile slice, with its column index:
//   aligned:   v = v0 + ((i / VEC) * kThreads + tid) * VEC + i % VEC
//   unaligned: v = v0 + i * kThreads + tid
template <typename T, bool ALIGNED>
struct TileMap {
  static constexpr int kVec = ALIGNED ? Elem<T>::kVec : 1;
  __device__ static int col(int v0, int i) {
    return v0 + ((i / kVec) * kThreads + (int)threadIdx.x) * kVec + (i % kVec);
  }
};

template <typename T, int EPT, bool ALIGNED>
__device__ __forceinline__ void load_tile_full(const T* row, int v0, float (&x)[EPT]) {
  constexpr int VEC = TileMap<T, ALIGNED>::kVec;
  // the whole tile is in range: every load is issued back to back with no
  // per-element guard, so none waits for another
#pragma unroll
  for (int q = 0; q < EPT / VEC; ++q) {
    const int v = v0 + (q * kThreads + (int)threadIdx.x) * VEC;
    if (ALIGNED) {
      Elem<T>::loadv(row + v, &x[q * VEC]);
    } else {
      x[q] = Elem<T>::load1(row + v);
    }
  }
}

// the ragged last tile of a row: columns at or past vend read as -inf
template <typename T, int EPT, bool ALIGNED>
__device__ __forceinline__ void load_tile_ragged(const T* row, int v0, int vend, float (&x)[EPT]) {
  constexpr int VEC = TileMap<T, ALIGNED>::kVec;
#pragma unroll
  for (int q = 0; q < EPT / VEC; ++q) {
    const int v = v0 + (q * kThreads + (int)threadIdx.x) * VEC;
    if (ALIGNED && v + VEC <= vend) {
      Elem<T>::loadv(row + v, &x[q * VEC]);
    } else {
#pragma unroll
      for (int k = 0; k < VEC; ++k)
        x[q * VEC + k] = (v + k < vend) ? Elem<T>::load1(row + v + k) : -kInf;
    }
  }
}

template <typename T, int EPT, bool ALIGNED>
__device__ __forceinline__ void load_tile(const T* row, int v0, int vend, float (&x)[EPT]) {
  if (v0 + kThreads * EPT <= vend)  // uniform
    load_tile_full<T, EPT, ALIGNED>(row, v0, x);
  else
    load_tile_ragged<T, EPT, ALIGNED>(row, v0, vend, x);
}

// ---------------------------------------------------------------------------
// K1: expand + local top-W per (row, tile)
// ---------------------------------------------------------------------------

struct K1Args {
  const void* logits;
  int64_t stride;       // elements between rows
  int V;
  int W;                // beam width: rows per item
  int K;                // candidates kept per tile (W, or 2W), <= WMAX
  int tile;             // elements per tile (kThreads * EPT)
  int tiles;            // tiles per row
  const float* s;       // running scores [B*W]
  const uint8_t* done;  // [B]
  float* pm;            // [rows][tiles] tile maximum
  float* ps;            // [rows][tiles] sum of exp(x - tile maximum)
  float* px;            // [rows][tiles][WMAX] tile top-K logits
  int* pv;              // [rows][tiles][WMAX] their columns
};

// tau for a tile: the w_keep-th largest of the kGroups group maxima, which is
// a lower bound on the tile's w_keep-th best logit (the group maxima are
// distinct elements). Every wave computes it on its own: lane l of each
// 16-lane row holds gmax[l % 16] and counts, over the 15 DPP row rotations,
// how many of the others are larger (gt) and at least as large (ge). A value
// with gt <= w-1 and ge+1 >= w is the w-th largest; all such lanes hold the
// same value, so the rotation direction does not matter.
template <int R>
__device__ __forceinline__ void rank_rotations(float g, int& gt, int& ge) {
  if constexpr (R <= 15) {
    const float o = dpp_f<0x120 + R>(g);  // row_ror:R
    gt += o > g ? 1 : 0;
    ge += o >= g ? 1 : 0;
    rank_rotations<R + 1>(g, gt, ge);
  }
}

__device__ __forceinline__ float tile_tau(const float* gmax, int w_keep) {
  const int lane = threadIdx.x & 63;
  const float g = gmax[lane & 15];
  int gt = 0, ge = 0;
  rank_rotations<1>(g, gt, ge);
  const uint64_t q = __ballot(lane < 16 && gt <= w_keep - 1 && ge + 1 >= w_keep);
  const int l = __builtin_ctzll(q);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g), l));
}

template <int WMAX, typename T, int EPT, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void k1_expand_select(K1Args a) {
  constexpr int kRegion = kListCap / kWaves;  // candidate slots of one wave
  __shared__ float gmax[kGroups];
  __shared__ float wm[kWaves], ws[kWaves];
  __shared__ int wn[kWaves];
  __shared__ float rx[kWaves];
  __shared__ int ri[kWaves];
  __shared__ alignas(16) uint64_t lk[kListCap];  // candidate keys (logit, column)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = blockIdx.y, c = blockIdx.x;
  const int b = r / a.W;
  const T* row = reinterpret_cast<const T*>(a.logits) + (int64_t)r * a.stride;
  const int v0 = c * a.tile;
  const int vend = min(a.V, v0 + a.tile);
  const int K = a.K;  // candidates kept per tile

  // The row's state and the tile are requested together, and the test waits
  // for both: a dead row or a finished item costs its (wasted) tile loads, but
  // a live row's logits are not held back by the state's round trip. An empty
  // asm with a memory clobber keeps the compiler from sinking the state loads
  // below the tile's waits. The flag byte is read through its aligned 32-bit
  // word, a scalar load (the flags array is 256-byte aligned and padded to a
  // multiple of 256 bytes).
  const uint32_t done_word = reinterpret_cast<const uint32_t*>(a.done)[b >> 2];
  const float sr = a.s[r];
  __asm__ volatile("" ::: "memory");
  float x[EPT];
  load_tile<T, EPT, ALIGNED>(row, v0, vend, x);
  if (((done_word >> (8 * (b & 3))) & 0xff) != 0 || sr == -kInf) return;  // nothing to expand

  // expand, per wave: the wave maximum mw and sum of exp(x - mw); the 16-lane
  // row maxima double as the group maxima for tau
  float m = -kInf;
#pragma unroll
  for (int i = 0; i < EPT; ++i) m = fmaxf(m, x[i]);
  m = fmaxf(m, dpp_f<0xb1>(m));   // quad_perm [1,0,3,2]
  m = fmaxf(m, dpp_f<0x4e>(m));   // quad_perm [2,3,0,1]
  m = fmaxf(m, dpp_f<0x141>(m));  // row_half_mirror
  m = fmaxf(m, dpp_f<0x140>(m));  // row_mirror: every lane has its row's max
  if ((lane & 15) == 0) gmax[tid >> 4] = m;
  const float mw = fmaxf(
      fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 0)),
            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 16))),
      fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 32)),
            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 48))));
  float s = 0.0f;
  if (mw > -kInf) {
    // exp(x - mw) = 2^(x log2e - mw log2e); terms below 2^-126 flush to zero,
    // far below the sum's own rounding (the sum is at least 1)
    const float off = -mw * kLog2e;
#pragma unroll
    for (int i = 0; i < EPT; ++i) s += __builtin_amdgcn_exp2f(fmaf(x[i], kLog2e, off));
  }
  s = wave_sum_f(s);
  if (lane == 0) {
    wm[wave] = mw;
    ws[wave] = s;
  }
  __syncthreads();

  // prune, stage 1: list every logit >= tau in this wave's LDS region as a
  // key that orders by (logit desc, column asc) (ballot + mbcnt compaction, no
  // atomics); -inf is never a candidate
  float tau = tile_tau(gmax, K);
  if (!(tau > -kInf)) tau = -3.402823466e38f;
  int woff = 0;
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const bool cand = x[i] >= tau;
    const uint64_t bm = __ballot(cand);
    if (bm) {
      const int pos = woff + (int)__builtin_amdgcn_mbcnt_hi(
                                 (uint32_t)(bm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0));
      if (cand && pos < kRegion)
        lk[wave * kRegion + pos] = pack_key(x[i], TileMap<T, ALIGNED>::col(v0, i));
      woff += __popcll(bm);
    }
  }
  if (lane == 0) wn[wave] = woff;
  __syncthreads();

  const int64_t pt = (int64_t)r * a.tiles + c;
  if (tid == 0) {  // the tile's (max, sum exp) from the four waves, in order
    float M = wm[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, wm[w]);
    float S = 0.0f;
    if (M > -kInf) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w)
        if (wm[w] > -kInf) S += ws[w] * exp2f((wm[w] - M) * kLog2e);
    }
    a.pm[pt] = M;
    a.ps[pt] = S;
  }
  // the list lengths are the same in every lane: keep them in scalar registers
  int n[kWaves], ntot = 0;
  bool overflow = false;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    n[w] = __builtin_amdgcn_readfirstlane(wn[w]);
    overflow |= n[w] > kRegion;
    ntot += n[w];
  }
  float* ox = a.px + pt * WMAX;
  int* oi = a.pv + pt * WMAX;
  if (tid < WMAX && tid >= min(ntot, K)) {  // ranks without a candidate
    ox[tid] = -kInf;
    oi[tid] = 0x7fffffff;
  }
  if (!overflow) {
    // rank every listed candidate by counting the larger keys (keys are
    // unique), one candidate per thread over the concatenated regions, two
    // keys per LDS read; the ranks below K go straight to the tile's output
    int pre[kWaves];
    pre[0] = 0;
#pragma unroll
    for (int w = 1; w < kWaves; ++w) pre[w] = pre[w - 1] + n[w - 1];
    for (int e = tid; e < ntot; e += kThreads) {
      int w = 0;
#pragma unroll
      for (int u = 1; u < kWaves; ++u) w = e >= pre[u] ? u : w;
      const uint64_t mine = lk[w * kRegion + e - pre[w]];
      int rank = 0;
#pragma unroll
      for (int u = 0; u < kWaves; ++u) {
        const uint64_t* bl = lk + u * kRegion;
        int f = 0;
        for (; f + 2 <= n[u]; f += 2) {
          const ulonglong2 two = *reinterpret_cast<const ulonglong2*>(bl + f);
          rank += (two.x > mine ? 1 : 0) + (two.y > mine ? 1 : 0);
        }
        if (f < n[u]) rank += bl[f] > mine ? 1 : 0;
      }
      if (rank < K) {
        ox[rank] = key_score(mine);
        oi[rank] = key_index(mine);
      }
    }
    return;
  }
  // A wave listed more candidates than its region holds (massive ties):
  // K rounds of a workgroup argmax over the registers, each round taking the
  // best key strictly worse than the previous one. Uniform control flow.
  float px = kInf;
  int pi = -1;
  for (int rk = 0; rk < K; ++rk) {
    float bx = -kInf;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int ii = TileMap<T, ALIGNED>::col(v0, i);
      if (x[i] > -kInf && better(px, pi, x[i], ii) && better(x[i], ii, bx, bi)) {
        bx = x[i];
        bi = ii;
      }
    }
    for (int o = 32; o >= 1; o >>= 1) {
      const float oxv = __shfl_xor(bx, o);
      const int oiv = __shfl_xor(bi, o);
      if (better(oxv, oiv, bx, bi)) {
        bx = oxv;
        bi = oiv;
      }
    }
    __syncthreads();
    if (lane == 0) {
      rx[wave] = bx;
      ri[wave] = bi;
    }
    __syncthreads();
    bx = rx[0];
    bi = ri[0];
    for (int w = 1; w < kWaves; ++w)
      if (better(rx[w], ri[w], bx, bi)) {
        bx = rx[w];
        bi = ri[w];
      }
    if (bx == -kInf) break;
    if (tid == 0) {
      ox[rk] = bx;
      oi[rk] = bi;
    }
    px = bx;
    pi = bi;
  }
}

// ---------------------------------------------------------------------------
// K2: merge + score + prune + finalize, one workgroup per batch item
// ---------------------------------------------------------------------------

struct DevState {
  float* s;            // [B*W] running scores, -inf = dead slot
  int* slot_rank;      // [B*W] rank of the slot's last selection
  uint8_t* done;       // [B]
  float* hnorm;        // [B*W] finished set
  float* hraw;
  int* hlen;
  int* hstep;
  int* hrank;
  int* hpar;           // parent slot at step-1
  int* htok;           // last token
  int* hcount;         // [B]
  int* bp_par;         // [T][B][W]
  int* bp_tok;         // [T][B][W]
  int* sel_j;          // [B][W]
  float* sel_c;        // [B][W]
  int* plan;           // [B][kPlanStride]
  const double* lpt;   // [T+1] length penalty per length
};

struct K2Args {
  DevState st;
  const float* pm;
  const float* ps;
  const float* px;
  const int* pv;
  int B, W, V, T, tiles, eos, pad, stop;
  int K;               // candidates ranked per item: W, or 2W (Hugging Face fill)
  double alpha;
  int t;               // this step, 1-based
  int32_t* out_beam;
  int32_t* out_tok;
  float* out_score;
  uint8_t* out_done;
};

__device__ __forceinline__ bool hyp_better(float na, int sa, int ra, float nb, int sb, int rb) {
  if (na != nb) return na > nb;
  if (sa != sb) return sa < sb;
  return ra < rb;
}

// The finished set of one item, staged in LDS for the finalize.
template <int WMAX>
struct HypSmem {
  float norm[WMAX], raw[WMAX];
  int len[WMAX], step[WMAX], rank[WMAX], par[WMAX], tok[WMAX];
  int count;
};

// BeamHypotheses.add of the batched section: append while fewer than W are
// kept, else replace the worst kept hypothesis when strictly better.
template <int WMAX>
__device__ void hyp_insert(HypSmem<WMAX>& h, int W, float norm, float raw, int len, int step,
                           int rank, int par, int tok) {
  int slot;
  if (h.count < W) {
    slot = h.count++;
  } else {
    int worst = 0;
    for (int i = 1; i < W; ++i)
      if (hyp_better(h.norm[worst], h.step[worst], h.rank[worst], h.norm[i], h.step[i],
                     h.rank[i]))
        worst = i;
    if (!hyp_better(norm, step, rank, h.norm[worst], h.step[worst], h.rank[worst])) return;
    slot = worst;
  }
  h.norm[slot] = norm;
  h.raw[slot] = raw;
  h.len[slot] = len;
  h.step[slot] = step;
  h.rank[slot] = rank;
  h.par[slot] = par;
  h.tok[slot] = tok;
}

// A finished item's step: no selection, every slot keeps itself, nothing to
// reorder.
__device__ __forceinline__ void noop_item(const K2Args& a, int b, int tid) {
  const int W = a.W, K = a.K;
  const DevState& st = a.st;
  const int bpbase = ((a.t - 1) * a.B + b) * W;
  if (tid < W) {
    a.out_beam[b * W + tid] = tid;
    a.out_tok[b * W + tid] = a.pad;
    a.out_score[b * W + tid] = -kInf;
    st.bp_par[bpbase + tid] = tid;
    st.bp_tok[bpbase + tid] = a.pad;
  }
  if (tid < K) {
    st.sel_j[b * K + tid] = -1;
    st.sel_c[b * K + tid] = -kInf;
  }
  if (tid == 0) {
    a.out_done[b] = 1;
    st.plan[b * kPlanStride + 1] = 0;
  }
}

// The finalize sub-step of item b, run by wave 0 with lane k holding the
// rank-k selected key (0 = none): EOS selections into the finished set in rank
// order, compaction of the live slots, the stop rule, the KV reorder plan, and
// the write-back of outputs, state and backpointers.
template <int WMAX>
__device__ __forceinline__ void finalize_item(const K2Args& a, HypSmem<WMAX>& hy, int* plan, int b,
                                              int lane, uint64_t key, double lp_t, double lp_T) {
  const int W = a.W, K = a.K, V = a.V, t = a.t;
  const DevState& st = a.st;
  const int bpbase = ((t - 1) * a.B + b) * W;
  const bool valid = key != 0;
  const float c = key_score(key);
  const int j = key_index(key);
  const int p = valid ? j / V : lane;
  const int tok = valid ? j - p * V : a.pad;
  const bool eos_tok = valid && a.eos >= 0 && tok == a.eos;
  // an EOS ranked W or below is dropped (only possible with 2W candidates)
  const bool is_eos = eos_tok && lane < W;
  const uint64_t lt = (lane == 0) ? 0 : (~(uint64_t)0 >> (64 - lane));  // lanes below
  const uint64_t cand_mask = __ballot(valid && !eos_tok);
  const int slot = __popcll(cand_mask & lt);  // compacted slot of a live selection
  // the first W non-EOS candidates in rank order fill the live slots
  const bool is_live = valid && !eos_tok && slot < W;
  const uint64_t live_mask = __ballot(is_live);
  const uint64_t eos_mask = __ballot(is_eos);
  const int nlive = __popcll(live_mask);

  // EOS selections enter the finished set in rank order
  const float norm = (float)((double)c / lp_t);
  for (uint64_t m = eos_mask; m; m &= m - 1) {
    const int e = __builtin_ctzll(m);
    const float ne = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(norm), e));
    const float ce = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), e));
    const int pe = __builtin_amdgcn_readlane(p, e);
    if (lane == 0) hyp_insert(hy, W, ne, ce, t, t, e, pe, a.eos);
  }

  // stop rule
  int d = 0;
  if (nlive == 0) {
    d = 1;
  } else if (hy.count == W) {
    float worst = kInf;
    for (int i = 0; i < W; ++i) worst = fminf(worst, hy.norm[i]);
    const float best_raw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), 0));
    if (a.stop == BS_STOP_TRUE) {
      d = 1;
    } else if (a.stop == BS_STOP_HEURISTIC) {
      d = worst >= (float)((double)best_raw / lp_t);
    } else {
      const int first = __builtin_ctzll(live_mask);
      const float best_live = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), first));
      const double lp = (a.alpha > 0.0 && best_live <= 0.0f) ? lp_T : lp_t;
      d = worst >= (float)((double)best_live / lp);
    }
  }

  // reorder plan: the distinct parents of moved slots (in parent order), each
  // with the bit mask of the slots it is copied to
  const bool moved = is_live && p != slot && !d;
  int nsrc = 0, ndst = 0;
  for (int q = 0; q < W; ++q) {
    uint64_t m = __ballot(moved && p == q);
    if (!m) continue;
    int dmask = 0;
    for (; m; m &= m - 1) {
      dmask |= 1 << __builtin_amdgcn_readlane(slot, __builtin_ctzll(m));
      ++ndst;
    }
    if (lane == 0) {
      plan[2 + nsrc] = q;
      plan[2 + kMaxBeam + nsrc] = dmask;
    }
    ++nsrc;
  }
  if (lane == 0) {
    plan[0] = nsrc;
    plan[1] = ndst;
    st.done[b] = (uint8_t)d;
    a.out_done[b] = (uint8_t)d;
    st.hcount[b] = hy.count;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

  // write back: plan, finished set, selection, slots, backpointers
  if (lane < 2 + 2 * kMaxBeam) st.plan[b * kPlanStride + lane] = plan[lane];
  if (lane < K) {
    st.sel_j[b * K + lane] = valid ? j : -1;
    st.sel_c[b * K + lane] = valid ? c : -kInf;
  }
  if (is_live) {  // rank `lane` becomes slot `slot`
    const int r = b * W + slot;
    st.s[r] = c;
    st.slot_rank[r] = lane;
    a.out_beam[r] = p;
    a.out_tok[r] = tok;
    a.out_score[r] = c;
    st.bp_par[bpbase + slot] = p;
    st.bp_tok[bpbase + slot] = tok;
  }
  if (lane < W) {
    const int e = b * W + lane;
    st.hnorm[e] = hy.norm[lane];
    st.hraw[e] = hy.raw[lane];
    st.hlen[e] = hy.len[lane];
    st.hstep[e] = hy.step[lane];
    st.hrank[e] = hy.rank[lane];
    st.hpar[e] = hy.par[lane];
    st.htok[e] = hy.tok[lane];
    if (lane >= nlive) {  // dead slot `lane`
      st.s[e] = -kInf;
      st.slot_rank[e] = W;
      a.out_beam[e] = lane;
      a.out_tok[e] = a.pad;
      a.out_score[e] = -kInf;
      st.bp_par[bpbase + lane] = lane;
      st.bp_tok[bpbase + lane] = a.pad;
    }
  }
}

// K2 for any tile count (the path for rows of more than 64 tiles): every
// listed candidate is scored, and each wave keeps its lanes' top-K by K rounds
// of a wave maximum, batch by batch; wave 0 merges the four lists.
template <int WMAX>
__global__ __launch_bounds__(kThreads) void k2_merge_finalize(K2Args a) {
  constexpr int kStage = 4 * kThreads;  // tile partials staged per pass
  __shared__ HypSmem<WMAX> hy;
  __shared__ float lse[WMAX];
  __shared__ float srow[WMAX];
  __shared__ float stage_m[kStage], stage_s[kStage];
  __shared__ float lse_m[WMAX], lse_s[WMAX];
  __shared__ uint64_t wave_best[kWaves][WMAX];
  __shared__ uint64_t final_best[WMAX];
  __shared__ int plan[kPlanStride];
  __shared__ int done_sh;
  __shared__ double lp_t, lp_T;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int W = a.W, K = a.K, V = a.V, t = a.t;
  const DevState& st = a.st;
  const int n_part = W * a.tiles;
  const int per_row = a.tiles * WMAX;
  const int n_entries = W * per_row;
  const float* px = a.px + (int64_t)b * n_entries;
  const int* pv = a.pv + (int64_t)b * n_entries;

  // every load of the item's state and of the first batch is issued up front
  float lx[kMergeNE];
  int lv[kMergeNE];
#pragma unroll
  for (int q = 0; q < kMergeNE; ++q) {
    const int e = q * kThreads + tid;
    lx[q] = e < n_entries ? px[e] : -kInf;
    lv[q] = e < n_entries ? pv[e] : 0;
  }
  for (int k = 0; k < kStage / kThreads; ++k) {
    const int e = k * kThreads + tid;
    if (e < n_part) {
      stage_m[e] = a.pm[(int64_t)b * n_part + e];
      stage_s[e] = a.ps[(int64_t)b * n_part + e];
    }
  }
  if (tid < W) {
    const int e = b * W + tid;
    srow[tid] = st.s[e];
    hy.norm[tid] = st.hnorm[e];
    hy.raw[tid] = st.hraw[e];
    hy.len[tid] = st.hlen[e];
    hy.step[tid] = st.hstep[e];
    hy.rank[tid] = st.hrank[e];
    hy.par[tid] = st.hpar[e];
    hy.tok[tid] = st.htok[e];
    lse_m[tid] = -kInf;
    lse_s[tid] = 0.0f;
  }
  if (tid == 0) {
    done_sh = st.done[b];
    hy.count = st.hcount[b];
    lp_t = st.lpt[t];
    lp_T = st.lpt[a.T];
  }
  __syncthreads();

  if (done_sh) {  // finished items: no-op outputs
    noop_item(a, b, tid);
    return;
  }

  // expand: lse of every live row from its tile partials. One wave per row,
  // lanes over tiles: the row maximum, then sum of S_tile * exp(M_tile - M),
  // both with fixed reduction trees.
  for (int base = 0; base < n_part; base += kStage) {
    if (base > 0) {
      __syncthreads();
      for (int k = 0; k < kStage / kThreads; ++k) {
        const int e = base + k * kThreads + tid;
        if (e < n_part) {
          stage_m[e - base] = a.pm[(int64_t)b * n_part + e];
          stage_s[e - base] = a.ps[(int64_t)b * n_part + e];
        }
      }
      __syncthreads();
    }
    for (int w = wave; w < W; w += kWaves) {
      if (!(srow[w] > -kInf)) continue;
      const int lo = max(base, w * a.tiles), hi = min(base + kStage, (w + 1) * a.tiles);
      float m = -kInf;
      for (int e = lo + lane; e < hi; e += 64) m = fmaxf(m, stage_m[e - base]);
      m = wave_max_f(m);
      float sum = 0.0f;
      if (m > -kInf)
        for (int e = lo + lane; e < hi; e += 64) {
          const float mt = stage_m[e - base];
          if (mt > -kInf) sum += stage_s[e - base] * exp2f((mt - m) * kLog2e);
        }
      sum = wave_sum_f(sum);
      if (lane == 0) {  // combine with the previous pass (tiles beyond kStage)
        float pm = lse_m[w], ps = lse_s[w];
        lse_combine(pm, ps, m, sum);
        lse_m[w] = pm;
        lse_s[w] = ps;
      }
    }
  }
  __syncthreads();
  if (tid < W) lse[tid] = (srow[tid] > -kInf && lse_m[tid] > -kInf) ? lse_m[tid] + logf(lse_s[tid])
                                                                   : -kInf;
  __syncthreads();

  // score + prune: each wave keeps the top-K of its lanes' candidates, batch by
  // batch (the running top-K rides along as one more candidate of lanes < K);
  // then wave 0 merges the waves' lists
  uint64_t carry = 0;
  for (int base = 0; base < n_entries; base += kThreads * kMergeNE) {
    if (base > 0) {
#pragma unroll
      for (int q = 0; q < kMergeNE; ++q) {
        const int e = base + q * kThreads + tid;
        lx[q] = e < n_entries ? px[e] : -kInf;
        lv[q] = e < n_entries ? pv[e] : 0;
      }
    }
    uint64_t key[kMergeNE + 1];
#pragma unroll
    for (int q = 0; q < kMergeNE; ++q) {
      const int e = base + q * kThreads + tid;
      key[q] = 0;
      if (e < n_entries) {
        const int w = e / per_row;
        const float lw = lse[w];
        if (lx[q] > -kInf && lw > -kInf) {
          const float logp = lx[q] - lw;   // fp32 log-probability
          const float c = srow[w] + logp;  // fp32 candidate score
          if (c > -kInf) key[q] = pack_key(c, w * V + lv[q]);
        }
      }
    }
    key[kMergeNE] = carry;
    wave_topw<kMergeNE + 1>(key, K, wave_best[wave]);
    carry = lane < K ? wave_best[wave][lane] : 0;
  }
  __syncthreads();

  if (wave != 0) return;

  // --- wave 0: final top-K, then the finalize sub-step
  uint64_t key;
  {
    uint64_t k4[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) k4[w] = lane < K ? wave_best[w][lane] : 0;
    wave_topw<kWaves>(k4, K, final_best);
    key = lane < K ? final_best[lane] : 0;
  }
  finalize_item<WMAX>(a, hy, plan, b, lane, key, lp_t, lp_T);
}

template <int CTRL>
__device__ __forceinline__ float dpp_max_f(float v) { return fmaxf(v, dpp_f<CTRL>(v)); }
template <int CTRL>
__device__ __forceinline__ float dpp_add_f(float v) { return v + dpp_f<CTRL>(v); }

// Maximum over each aligned group of 16 lanes (a DPP row); every lane of the
// row ends with it.
__device__ __forceinline__ float row16_max_f(float v) {
  v = dpp_max_f<0xb1>(v);   // quad_perm [1,0,3,2]
  v = dpp_max_f<0x4e>(v);   // quad_perm [2,3,0,1]
  v = dpp_max_f<0x141>(v);  // row_half_mirror
  v = dpp_max_f<0x140>(v);  // row_mirror
  return v;
}
__device__ __forceinline__ float row16_sum_f(float v) {
  v = dpp_add_f<0xb1>(v);
  v = dpp_add_f<0x4e>(v);
  v = dpp_add_f<0x141>(v);
  v = dpp_add_f<0x140>(v);
  return v;
}

// K2 for tiles <= 64: merge + score + prune + finalize, one workgroup per item.
//
// Stage A, per row: every tile list is ordered by logit, hence by candidate
// score, so K rounds of a merge of the row's tile lists give the row's best K.
// A 16-lane row of the wave serves one beam row; lane l holds the lists of
// tiles l*H .. l*H+H-1 as scores and columns in registers. Each round takes
// the maximum head score over the 16 lanes (DPP), the ballot of the lanes
// holding it, and the lowest such lane: lower lanes hold lower tiles, hence
// lower columns, so ties go to the lower flat index. That lane emits its head
// and moves to its next entry.
// Stage B, wave 0: the W row lists are merged the same way (lane w holds row
// w's list; a lower row means a lower flat index), and the K winners are put
// in exact (score desc, flat index asc) order before the finalize.
template <int WMAX, int H>
__global__ __launch_bounds__(kThreads) void k2_select_finalize(K2Args a) {
  __shared__ HypSmem<WMAX> hy;
  __shared__ float row_sc[kMaxBeam][WMAX];  // each row's best K, merge order
  __shared__ int row_j[kMaxBeam][WMAX];
  __shared__ uint64_t ordered[WMAX];
  __shared__ int plan[kPlanStride];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int W = a.W, K = a.K, V = a.V, tiles = a.tiles;
  const DevState& st = a.st;
  const int w = tid >> 4;   // beam row of this lane's 16-lane group
  const int gl = tid & 15;  // lane within the group
  const int c0 = gl * H;    // first tile of this lane

  // every load of the item is issued before the first wait: the finished set,
  // the flags and length penalties, and the partials of the lane's tiles.
  // The loads are unconditional, at indices clamped into range (what a lane
  // has no use for is masked afterwards): a load under a branch would make
  // the compiler wait for it before the next one.
  const int ws = min(tid, W - 1);
  const int eh = b * W + ws;
  const float h_norm = st.hnorm[eh], h_raw = st.hraw[eh];
  const int h_len = st.hlen[eh], h_step = st.hstep[eh], h_rank = st.hrank[eh];
  const int h_par = st.hpar[eh], h_tok = st.htok[eh];
  const int done = st.done[b];
  const int hcount = st.hcount[b];
  const double lp_t = st.lpt[a.t], lp_T = st.lpt[a.T];

  const int wr = min(w, W - 1);
  float sr = st.s[b * W + wr];
  float tm[H], ts[H];
  float sc[H][WMAX];
  int col[H][WMAX];
#pragma unroll
  for (int h = 0; h < H; ++h) {
    const int64_t pt = (int64_t)(b * W + wr) * tiles + min(c0 + h, tiles - 1);
    tm[h] = a.pm[pt];
    ts[h] = a.ps[pt];
#pragma unroll
    for (int i = 0; i < WMAX; ++i) {
      sc[h][i] = a.px[pt * WMAX + i];
      col[h][i] = a.pv[pt * WMAX + i];
    }
  }
  if (w >= W) sr = -kInf;  // a group beyond the item's rows
#pragma unroll
  for (int h = 0; h < H; ++h)
    if (c0 + h >= tiles) {  // a lane beyond the row's tiles
      tm[h] = -kInf;
      ts[h] = 0.0f;
#pragma unroll
      for (int i = 0; i < WMAX; ++i) sc[h][i] = -kInf;
    }
  // dead rows (and rows the expand pass skipped) take no part
  const bool live = w < W && sr > -kInf;
  // lse of row w from its tiles' (max, sum exp) partials
  float m = -kInf;
#pragma unroll
  for (int h = 0; h < H; ++h) m = fmaxf(m, live ? tm[h] : -kInf);
  m = row16_max_f(m);
  float e = 0.0f;
#pragma unroll
  for (int h = 0; h < H; ++h)
    if (live && tm[h] > -kInf) e += ts[h] * exp2f((tm[h] - m) * kLog2e);
  e = row16_sum_f(e);
  const float lse = m > -kInf ? m + logf(e) : -kInf;
  // candidate scores cand = fp32(s + fp32(x - lse)); -inf is no candidate.
  // Entries K.. of a tile list are -inf; K rounds could not reach them anyway
  // (K better entries of the same tile come first).
#pragma unroll
  for (int h = 0; h < H; ++h)
#pragma unroll
    for (int i = 0; i < WMAX; ++i) {
      float c = -kInf;
      if (live && lse > -kInf && sc[h][i] > -kInf) {
        const float logp = sc[h][i] - lse;
        c = sr + logp;
      }
      sc[h][i] = c;
    }

  // stage A: K rounds per row
  {
    const uint64_t below = ((uint64_t)1 << (lane & 15)) - 1;  // lower lanes of the group
    const int gshift = lane & 48;
    float hs[H];
    int hc[H];
#pragma unroll
    for (int h = 0; h < H; ++h) {
      hs[h] = sc[h][0];
      hc[h] = col[h][0];
    }
    for (int r = 0; r < K; ++r) {
      // this lane's best head: the first of its tiles holding the maximum
      int bh = 0;
      float bs = hs[0];
#pragma unroll
      for (int h = 1; h < H; ++h)
        if (hs[h] > bs) {
          bs = hs[h];
          bh = h;
        }
      const float M = row16_max_f(bs);
      const uint64_t holders = __ballot(bs == M && M > -kInf);
      const bool win = bs == M && M > -kInf && ((holders >> gshift) & below) == 0;
      if (gl == 0 && w < W && !(M > -kInf)) {  // the row has no candidate left
        row_sc[w][r] = -kInf;
        row_j[w][r] = 0;
      }
      if (win) {
        int hcol = hc[0];
#pragma unroll
        for (int h = 1; h < H; ++h) hcol = bh == h ? hc[h] : hcol;
        row_sc[w][r] = M;
        row_j[w][r] = w * V + hcol;
        // the winning list moves up by one entry (register moves: the lists
        // are never indexed at run time)
#pragma unroll
        for (int h = 0; h < H; ++h) {
          if (bh == h) {
#pragma unroll
            for (int i = 0; i + 1 < WMAX; ++i) {
              sc[h][i] = sc[h][i + 1];
              col[h][i] = col[h][i + 1];
            }
            sc[h][WMAX - 1] = -kInf;
            hs[h] = sc[h][0];
            hc[h] = col[h][0];
          }
        }
      }
    }
  }
  if (tid < W) {
    hy.norm[tid] = h_norm;
    hy.raw[tid] = h_raw;
    hy.len[tid] = h_len;
    hy.step[tid] = h_step;
    hy.rank[tid] = h_rank;
    hy.par[tid] = h_par;
    hy.tok[tid] = h_tok;
  }
  if (tid == 0) hy.count = hcount;
  __syncthreads();

  if (done) {  // finished items: no-op outputs
    noop_item(a, b, tid);
    return;
  }
  if (wave != 0) return;

  // stage B: lane w < W holds row w's list; lane r keeps round r's winner
  float rs[WMAX];
  int rj[WMAX];
#pragma unroll
  for (int i = 0; i < WMAX; ++i) {
    const bool in = lane < W && i < K;
    rs[i] = in ? row_sc[lane < W ? lane : 0][i] : -kInf;
    rj[i] = in ? row_j[lane < W ? lane : 0][i] : 0;
  }
  float hs = rs[0], fs = -kInf;
  int hj = rj[0], fj = 0;
  for (int r = 0; r < K; ++r) {
    const float M = row16_max_f(hs);  // lanes 0..15 hold every row
    const uint64_t holders = __ballot(lane < 16 && hs == M && M > -kInf);
    if (holders == 0) break;  // uniform: no candidate left
    const int l = __builtin_ctzll(holders);
    const int wj = __builtin_amdgcn_readlane(hj, l);
    if (lane == r) {
      fs = M;
      fj = wj;
    }
    if (lane == l) {  // the winning row's list moves up by one entry
#pragma unroll
      for (int i = 0; i + 1 < WMAX; ++i) {
        rs[i] = rs[i + 1];
        rj[i] = rj[i + 1];
      }
      rs[WMAX - 1] = -kInf;
      hs = rs[0];
      hj = rj[0];
    }
  }
  // exact order of the K winners: rank = number of better winners (the empty
  // ranks come last and keep their places)
  const uint64_t fk = fs > -kInf ? pack_key(fs, fj) : 0;
  int rank = 0;
  for (int q = 0; q < K; ++q) rank += readlane_u64(fk, q) > fk ? 1 : 0;
  if (fk == 0) rank = lane;
  if (lane < K) ordered[rank] = fk;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  const uint64_t key = lane < K ? ordered[lane] : 0;
  finalize_item<WMAX>(a, hy, plan, b, lane, key, lp_t, lp_T);
}

// ---------------------------------------------------------------------------
// L1-L3: the two-pass (coarse-to-fine) selection of the LightSeq article
// ("层级式解码计算"), a measured alternative to K1/K2
// ---------------------------------------------------------------------------

struct CFArgs {
  const void* logits;
  int64_t stride;       // elements between rows
  int V, W, K, KP;      // KP: groups per row, a power of two >= K (<= 16)
  int tile, tiles;
  const float* s;       // [B*W] running scores
  const uint8_t* done;  // [B]
  float* pm;            // [rows][tiles] tile maximum
  float* ps;            // [rows][tiles] sum of exp(x - tile maximum)
  float* gm;            // [rows][tiles][KP] the tile's group maxima
  float* qc;            // [B][cap] queued candidate scores
  int* qj;              // [B][cap] their flat indices
  int* qn;              // [B] queue lengths (a length above cap: overflow)
  int cap;
};

// The row state and the tile, requested together (as in K1).
template <typename T, int EPT, bool ALIGNED>
__device__ __forceinline__ bool cf_load(const CFArgs& a, int r, int v0, int vend,
                                        float (&x)[EPT], float& sr) {
  const int b = r / a.W;
  const T* row = reinterpret_cast<const T*>(a.logits) + (int64_t)r * a.stride;
  const uint32_t done_word = reinterpret_cast<const uint32_t*>(a.done)[b >> 2];
  sr = a.s[r];
  __asm__ volatile("" ::: "memory");
  load_tile<T, EPT, ALIGNED>(row, v0, vend, x);
  return ((done_word >> (8 * (b & 3))) & 0xff) == 0 && sr > -kInf;
}

// L1, grid (tiles, rows): the tile's (max, sum exp) and the maxima of its KP
// groups (lane mod KP: every group of the row takes elements from every tile).
template <typename T, int EPT, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void l1_coarse(CFArgs a) {
  __shared__ float wm[kWaves], ws[kWaves];
  __shared__ float wg[kWaves][kMaxBeam];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = blockIdx.y, c = blockIdx.x;
  const int v0 = c * a.tile, vend = min(a.V, v0 + a.tile);
  float x[EPT], sr;
  if (!cf_load<T, EPT, ALIGNED>(a, r, v0, vend, x, sr)) return;
  float m = -kInf;
#pragma unroll
  for (int i = 0; i < EPT; ++i) m = fmaxf(m, x[i]);
  float g = m;  // lanes l and l ^ st share l mod KP for st >= KP
  for (int st = a.KP; st < 64; st <<= 1) g = fmaxf(g, __shfl_xor(g, st));
  if (lane < a.KP) wg[wave][lane] = g;
  const float mw = wave_max_f(m);
  float sum = 0.0f;
  if (mw > -kInf) {
    const float off = -mw * kLog2e;
#pragma unroll
    for (int i = 0; i < EPT; ++i) sum += __builtin_amdgcn_exp2f(fmaf(x[i], kLog2e, off));
  }
  sum = wave_sum_f(sum);
  if (lane == 0) {
    wm[wave] = mw;
    ws[wave] = sum;
  }
  __syncthreads();
  const int64_t pt = (int64_t)r * a.tiles + c;
  if (tid == 0) {
    float M = wm[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, wm[w]);
    float S = 0.0f;
    if (M > -kInf) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w)
        if (wm[w] > -kInf) S += ws[w] * exp2f((wm[w] - M) * kLog2e);
    }
    a.pm[pt] = M;
    a.ps[pt] = S;
  }
  if (tid < a.KP)
    a.gm[pt * a.KP + tid] = fmaxf(fmaxf(wg[0][tid], wg[1][tid]), fmaxf(wg[2][tid], wg[3][tid]));
}

// L2, grid (tiles, rows): the row's lse and threshold R (the K-th largest of
// its KP group maxima: KP distinct elements, so R is at most the row's K-th
// best logit), then the second read of the tile queues every logit >= R with
// its candidate score fp32(s + fp32(x - lse)), one queue slot range per wave
// (one device-scope atomic).
template <typename T, int EPT, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void l2_fine(CFArgs a) {
  __shared__ float sh_R, sh_lse;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = blockIdx.y, c = blockIdx.x, b = r / a.W, w = r - b * a.W;
  const int v0 = c * a.tile, vend = min(a.V, v0 + a.tile);
  float x[EPT], sr;
  if (!cf_load<T, EPT, ALIGNED>(a, r, v0, vend, x, sr)) return;
  if (wave == 0) {
    const int64_t p0 = (int64_t)r * a.tiles;
    float M = -kInf;
    for (int t = lane; t < a.tiles; t += 64) M = fmaxf(M, a.pm[p0 + t]);
    M = wave_max_f(M);
    float S = 0.0f;
    if (M > -kInf)
      for (int t = lane; t < a.tiles; t += 64) {
        const float mt = a.pm[p0 + t];
        if (mt > -kInf) S += a.ps[p0 + t] * exp2f((mt - M) * kLog2e);
      }
    S = wave_sum_f(S);
    // group g's maximum over the row: lane l reads entries l, l+64, ... of
    // the row's [tiles][KP] maxima, all of group l mod KP (64 is a multiple
    // of KP), four unconditional loads at a time; then lanes of one group
    // combine (xor strides >= KP)
    const int ng = a.tiles * a.KP;
    const float* gr = a.gm + p0 * a.KP;
    float gv = -kInf;
    for (int e0 = lane; e0 < ng; e0 += 4 * 64) {
      float g4[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) g4[u] = gr[min(e0 + u * 64, ng - 1)];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (e0 + u * 64 < ng) gv = fmaxf(gv, g4[u]);
    }
    for (int st = a.KP; st < 64; st <<= 1) gv = fmaxf(gv, __shfl_xor(gv, st));
    int gt = 0, ge = 0;
    for (int q = 0; q < a.KP; ++q) {
      const float o = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gv), q));
      gt += o > gv ? 1 : 0;
      ge += o >= gv ? 1 : 0;
    }
    // the K-th largest: at most K-1 larger and at least K not smaller (self included)
    const uint64_t hit = __ballot(lane < a.KP && gt <= a.K - 1 && ge >= a.K);
    const int hl = hit ? __builtin_ctzll(hit) : 0;
    const float R = hit ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gv), hl))
                        : -kInf;
    if (lane == 0) {
      sh_R = R;
      sh_lse = M > -kInf ? M + logf(S) : -kInf;
    }
  }
  __syncthreads();
  float R = sh_R;
  const float lse = sh_lse;
  if (!(lse > -kInf)) return;
  if (!(R > -kInf)) R = -3.402823466e38f;  // -inf is never a candidate
  int n = 0;
#pragma unroll
  for (int i = 0; i < EPT; ++i) n += __popcll(__ballot(x[i] >= R));
  if (n == 0) return;
  int base = 0;
  if (lane == 0) base = atomicAdd(&a.qn[b], n);
  base = __builtin_amdgcn_readfirstlane(base);
  float* qc = a.qc + (int64_t)b * a.cap;
  int* qj = a.qj + (int64_t)b * a.cap;
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const bool cand = x[i] >= R;
    const uint64_t bm = __ballot(cand);
    if (bm) {
      const int pos = base + (int)__builtin_amdgcn_mbcnt_hi(
                                 (uint32_t)(bm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0));
      if (cand && pos < a.cap) {
        const float logp = x[i] - lse;
        qc[pos] = sr + logp;
        qj[pos] = w * a.V + TileMap<T, ALIGNED>::col(v0, i);
      }
      base += __popcll(bm);
    }
  }
}

// The best K keys of an item over per-thread key arrays: K rounds of a
// workgroup maximum over the keys below the previous round's winner.
// out[r] (LDS) gets round r's key (0: none). Call with every thread.
template <int N>
__device__ __forceinline__ void block_topk(const uint64_t (&k)[N], int K, uint64_t* wbest,
                                           uint64_t* out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint64_t prev = ~(uint64_t)0;
  for (int r = 0; r < K; ++r) {
    uint64_t best = 0;
#pragma unroll
    for (int q = 0; q < N; ++q) best = (k[q] < prev && k[q] > best) ? k[q] : best;
    best = wave_max_u64(best);
    if (lane == 0) wbest[wave] = best;
    __syncthreads();
    uint64_t m = wbest[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = wbest[w] > m ? wbest[w] : m;
    if (threadIdx.x == 0) out[r] = m;
    __syncthreads();
    prev = m;
  }
}

struct L3Args {
  K2Args k2;
  CFArgs cf;
};

// L3, one workgroup per item: the K best queued candidates, exactly ordered by
// (score desc, flat index asc), then the finalize of K2. A queue that
// overflowed (massive ties above R) falls back to an exact scan of the item's
// logits: K rounds of a workgroup maximum over all W*V candidates.
template <int WMAX, typename T>
__global__ __launch_bounds__(kThreads) void l3_sort_finalize(L3Args args) {
  constexpr int kPer = kMaxBeam;  // queue entries per thread: cap = 256 * KP <= 256 * 16
  __shared__ HypSmem<WMAX> hy;
  __shared__ uint64_t wbest[kWaves];
  __shared__ uint64_t best[WMAX];
  __shared__ float lse_sh[kMaxBeam];
  __shared__ int plan[kPlanStride];
  const K2Args& a = args.k2;
  const CFArgs& cf = args.cf;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int W = a.W, K = a.K, V = a.V;
  const DevState& st = a.st;
  if (tid < W) {
    const int e = b * W + tid;
    hy.norm[tid] = st.hnorm[e];
    hy.raw[tid] = st.hraw[e];
    hy.len[tid] = st.hlen[e];
    hy.step[tid] = st.hstep[e];
    hy.rank[tid] = st.hrank[e];
    hy.par[tid] = st.hpar[e];
    hy.tok[tid] = st.htok[e];
  }
  if (tid == 0) hy.count = st.hcount[b];
  const int done = st.done[b];
  const double lp_t = st.lpt[a.t], lp_T = st.lpt[a.T];
  const int n = cf.qn[b];
  __syncthreads();
  if (tid == 0) cf.qn[b] = 0;  // the queue is empty for the next step
  if (done) {
    noop_item(a, b, tid);
    return;
  }
  if (n <= cf.cap) {
    // unconditional loads (the queue has cap entries; those at or past n are
    // masked), so that they are all in flight before the first wait
    float qc[kPer];
    int qj[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int e = min(q * kThreads + tid, cf.cap - 1);
      qc[q] = cf.qc[(int64_t)b * cf.cap + e];
      qj[q] = cf.qj[(int64_t)b * cf.cap + e];
    }
    uint64_t k[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) k[q] = (q * kThreads + tid < n) ? pack_key(qc[q], qj[q]) : 0;
    block_topk<kPer>(k, K, wbest, best);
  } else {
    // exact fallback: the lse of each live row, then K rounds over all of the
    // item's candidates
    if (wave == 0) {
      for (int w = 0; w < W; ++w) {
        const int64_t p0 = (int64_t)(b * W + w) * cf.tiles;
        float M = -kInf;
        for (int t = lane; t < cf.tiles; t += 64) M = fmaxf(M, cf.pm[p0 + t]);
        M = wave_max_f(M);
        float S = 0.0f;
        if (M > -kInf)
          for (int t = lane; t < cf.tiles; t += 64) {
            const float mt = cf.pm[p0 + t];
            if (mt > -kInf) S += cf.ps[p0 + t] * exp2f((mt - M) * kLog2e);
          }
        S = wave_sum_f(S);
        if (lane == 0)
          lse_sh[w] = (st.s[b * W + w] > -kInf && M > -kInf) ? M + logf(S) : -kInf;
      }
    }
    __syncthreads();
    uint64_t prev = ~(uint64_t)0;
    for (int r = 0; r < K; ++r) {
      uint64_t bk = 0;
      for (int w = 0; w < W; ++w) {
        const float lw = lse_sh[w];
        if (!(lw > -kInf)) continue;
        const float sw = st.s[b * W + w];
        const T* row = reinterpret_cast<const T*>(cf.logits) + (int64_t)(b * W + w) * cf.stride;
        for (int v = tid; v < V; v += kThreads) {
          const float xv = Elem<T>::load1(row + v);
          if (!(xv > -kInf)) continue;
          const float logp = xv - lw;
          const float cv = sw + logp;
          if (!(cv > -kInf)) continue;
          const uint64_t kk = pack_key(cv, w * V + v);
          bk = (kk < prev && kk > bk) ? kk : bk;
        }
      }
      bk = wave_max_u64(bk);
      if (lane == 0) wbest[wave] = bk;
      __syncthreads();
      uint64_t m = wbest[0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) m = wbest[w] > m ? wbest[w] : m;
      if (tid == 0) best[r] = m;
      __syncthreads();
      prev = m;
    }
  }
  if (wave != 0) return;
  const uint64_t key = lane < K ? best[lane] : 0;
  finalize_item<WMAX>(a, hy, plan, b, lane, key, lp_t, lp_T);
}

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
        if (ok[k]) v[k][q] = *reinterpret_cast<const WT*>(from + off[k]);
    }
  }
  // In place: a destination row may be another copy's parent. No other thread
  // touches this thread's words (the offsets are unique per thread, item and
  // plane), so it is enough that every load of this thread has returned before
  // its first store: s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their
  // no-wait maxima).
  __builtin_amdgcn_s_waitcnt(0x0F70);
#pragma unroll
  for (int q = 0; q < WMAX; ++q) {
    for (int m = dmask[q]; m; m &= m - 1) {
      char* dst = base + (row0 + __builtin_ctz(m)) * row_stride;
      // streaming stores: the moved rows are not read again by this launch,
      // and keeping them out of the caches measured ~10% faster end to end
#pragma unroll
      for (int k = 0; k < NP; ++k)
        if (ok[k]) __builtin_nontemporal_store(v[k][q], reinterpret_cast<WT*>(dst + off[k]));
      // one destination slot at a time: waiting for this slot's stores before
      // issuing the next measured faster than keeping all of them in flight
      __builtin_amdgcn_s_waitcnt(0x0F70);
    }
  }
}

template <int WMAX, int WORD, int NP, bool CONTIG>
__global__ __launch_bounds__(kK3Threads) void k3_kv_reorder(K3Args a) {
  using WT = typename Word<WORD>::type;
  const int b = blockIdx.y;
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
  char* base = a.planes[blockIdx.z] + a.base_off;
  const int64_t row0 = (int64_t)b * a.W;

  int64_t off[NP];
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    const int64_t e = ((int64_t)blockIdx.x * NP + k) * kK3Threads + threadIdx.x;
    if (CONTIG) {
      off[k] = e * WORD;
    } else {
      const int64_t pos = e / a.words_per_pos;
      off[k] = pos * a.pos_stride + (e - pos * a.words_per_pos) * WORD;
    }
  }
  // every word of the tile is in range (uniform), except in the last tile
  const int64_t e0 = (int64_t)blockIdx.x * NP * kK3Threads + threadIdx.x;
  if ((int64_t)(blockIdx.x + 1) * NP * kK3Threads <= a.words)
    move_words<WMAX, WT, NP, true>(base, row0, a.row_stride, off, e0, a.words, nsrc, src, dmask);
  else
    move_words<WMAX, WT, NP, false>(base, row0, a.row_stride, off, e0, a.words, nsrc, src,
                                    dmask);
}

// ---------------------------------------------------------------------------
// K4: blockwise verify
// ---------------------------------------------------------------------------

struct K4Args {
  const void* logits;
  int64_t stride;
  int V, tile, tiles, k, B;
  float* px;   // [rows][tiles] tile maximum
  int* pv;     // [rows][tiles] its first column
  int* pc;     // [rows][tiles] logits of the tile that beat the proposal's
  const int32_t* proposals;
  int32_t* accept;
  int32_t* argmax;
  int32_t* rank;       // optional [rows]
  int top_k, min_block;
};

// The accept sub-step of item b, run by one wave: lane i merges the tiles of
// position i. Without counts a position passes when its proposal is the
// argmax; with counts, when the proposal's rank (logits that beat it, summed
// over tiles) is below top_k.
template <bool COUNT>
__device__ void accept_item(const K4Args& a, int b, int i) {
  bool pass = false;
  if (i < a.k) {
    const int64_t r = (int64_t)b * a.k + i;
    float bx = -kInf;
    int bi = 0x7fffffff;
    int rank = 0;
    for (int c = 0; c < a.tiles; ++c) {
      const float x = a.px[r * a.tiles + c];
      const int v = a.pv[r * a.tiles + c];
      if (better(x, v, bx, bi)) {
        bx = x;
        bi = v;
      }
      if (COUNT) rank += a.pc[r * a.tiles + c];
    }
    a.argmax[r] = bi;
    const int prop = a.proposals[r];
    if (COUNT) {
      if (prop < 0 || prop >= a.V) rank = a.V;
      if (a.rank) a.rank[r] = rank;
      pass = rank < a.top_k;
    } else {
      pass = (prop == bi);
    }
  }
  const uint64_t m = __ballot(pass);
  if (i == 0) {
    // accepted prefix: number of trailing ones of the pass mask, at most k,
    // and at least the minimum block
    const uint64_t miss = ~m;
    int acc = (miss == 0) ? 64 : __ffsll((long long)miss) - 1;
    acc = acc < a.k ? acc : a.k;
    a.accept[b] = acc > a.min_block ? acc : a.min_block;
  }
}

template <typename T, int EPT, bool ALIGNED, bool COUNT>
__global__ __launch_bounds__(kThreads) void k4_verify(K4Args a) {
  __shared__ float rx[kWaves];
  __shared__ int ri[kWaves];
  __shared__ int rc[kWaves];
  const int r = blockIdx.y, c = blockIdx.x;
  const T* row = reinterpret_cast<const T*>(a.logits) + (int64_t)r * a.stride;
  const int v0 = c * a.tile;
  const int vend = min(a.V, v0 + a.tile);
  const int prop = COUNT ? a.proposals[r] : -1;
  float x[EPT];
  load_tile<T, EPT, ALIGNED>(row, v0, vend, x);
  // the proposal's own logit (top-k criterion); an out-of-range proposal is
  // never read and beaten by nothing here (its rank is set to V at the merge)
  float xp = kInf;
  if (COUNT && prop >= 0 && prop < a.V) xp = Elem<T>::load1(row + prop);
  // first index of the maximum; -inf logits take part (padding is excluded)
  float bx = -kInf;
  int bi = 0x7fffffff;
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int v = TileMap<T, ALIGNED>::col(v0, i);
    if (v < vend && better(x[i], v, bx, bi)) {
      bx = x[i];
      bi = v;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    float ox = __shfl_xor(bx, o);
    int oi = __shfl_xor(bi, o);
    if (better(ox, oi, bx, bi)) {
      bx = ox;
      bi = oi;
    }
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    rx[wave] = bx;
    ri[wave] = bi;
  }
  __syncthreads();
  int cnt = 0;
  if (COUNT && prop >= 0 && prop < a.V) {
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int v = TileMap<T, ALIGNED>::col(v0, i);
      cnt += (v < vend && better(x[i], v, xp, prop)) ? 1 : 0;
    }
  }
  if (COUNT) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) cnt += __shfl_xor(cnt, o);
    if (lane == 0) rc[wave] = cnt;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < kWaves; ++w)
      if (better(rx[w], ri[w], bx, bi)) {
        bx = rx[w];
        bi = ri[w];
      }
    a.px[(int64_t)r * a.tiles + c] = bx;
    a.pv[(int64_t)r * a.tiles + c] = bi;
    if (COUNT) a.pc[(int64_t)r * a.tiles + c] = rc[0] + rc[1] + rc[2] + rc[3];
  }
}

// Verify with one workgroup per row (used when there are enough rows to fill
// the chip): each thread streams its share of the row, kRowLoads 16-byte
// loads per batch, all unconditional (indices clamped into the row, so no
// branch stands between the loads and the compiler waits for a batch only
// once). A thread visits its columns in increasing order, so a strictly
// larger logit is the only one that moves its running maximum and the first
// index of the maximum is kept; a row that is -inf throughout has its first
// index, 0. For the top-k criterion, logits that beat the proposal's (larger,
// or equal at a lower index) are counted, in the rare vectors whose maximum
// reaches it. The row's result goes to the partials as a single tile, for the
// same accept step.
constexpr int kRowLoads = 16;
template <typename T, bool ALIGNED, bool COUNT>
__global__ __launch_bounds__(kThreads) void k4_row(K4Args a) {
  __shared__ float rx[kWaves];
  __shared__ int ri[kWaves];
  __shared__ int rc[kWaves];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const T* row = reinterpret_cast<const T*>(a.logits) + (int64_t)r * a.stride;
  const int V = a.V;
  const int prop = COUNT ? a.proposals[r] : -1;
  float xp = kInf;  // an out-of-range proposal is beaten by nothing here
  if (COUNT && prop >= 0 && prop < V) xp = Elem<T>::load1(row + prop);
  float bx = -kInf;
  int bi = 0x7fffffff;
  int cnt = 0;
  auto count = [&](float x, int v) {
    if (COUNT) cnt += better(x, v, xp, prop) ? 1 : 0;
  };
  if (ALIGNED) {
    constexpr int VEC = Elem<T>::kVec;
    const int nvec = V / VEC;
    const uint4* rv = reinterpret_cast<const uint4*>(row);
    if (nvec > 0) {  // uniform; a row shorter than one vector has only a tail
      const int qmax = nvec - 1;
      for (int q0 = tid; q0 < nvec; q0 += kThreads * kRowLoads) {
        uint4 raw[kRowLoads];
#pragma unroll
        for (int u = 0; u < kRowLoads; ++u) raw[u] = rv[min(q0 + u * kThreads, qmax)];
#pragma unroll
        for (int u = 0; u < kRowLoads; ++u) {
          const int q = q0 + u * kThreads;
          if (q < nvec) {
            float x[VEC];
            Elem<T>::unpack(raw[u], x);
            float vm = x[0];
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
              if (x[k] > bx) {
                bx = x[k];
                bi = q * VEC + k;
              }
              if (COUNT) vm = fmaxf(vm, x[k]);
            }
            if (COUNT && vm >= xp) {
#pragma unroll
              for (int k = 0; k < VEC; ++k) count(x[k], q * VEC + k);
            }
          }
        }
      }
    }
    const int v = nvec * VEC + tid;  // the ragged tail, under one vector
    if (v < V) {  // the tail columns come after every vector column
      const float x = Elem<T>::load1(row + v);
      if (x > bx) {
        bx = x;
        bi = v;
      }
      count(x, v);
    }
  } else {
    for (int v0 = tid; v0 < V; v0 += kThreads * kRowLoads) {
      float x[kRowLoads];
#pragma unroll
      for (int u = 0; u < kRowLoads; ++u) x[u] = Elem<T>::load1(row + min(v0 + u * kThreads, V - 1));
#pragma unroll
      for (int u = 0; u < kRowLoads; ++u) {
        const int v = v0 + u * kThreads;
        if (v < V) {
          if (x[u] > bx) {
            bx = x[u];
            bi = v;
          }
          count(x[u], v);
        }
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ox = __shfl_xor(bx, o);
    const int oi = __shfl_xor(bi, o);
    if (better(ox, oi, bx, bi)) {
      bx = ox;
      bi = oi;
    }
    if (COUNT) cnt += __shfl_xor(cnt, o);
  }
  if (lane == 0) {
    rx[wave] = bx;
    ri[wave] = bi;
    rc[wave] = cnt;
  }
  __syncthreads();
  if (tid == 0) {
#pragma unroll
    for (int w = 1; w < kWaves; ++w)
      if (better(rx[w], ri[w], bx, bi)) {
        bx = rx[w];
        bi = ri[w];
      }
    a.px[r] = bx;
    a.pv[r] = bi == 0x7fffffff ? 0 : bi;  // every logit -inf: the first index
    if (COUNT) a.pc[r] = rc[0] + rc[1] + rc[2] + rc[3];
  }
}

// the merge as its own launch, one wave per item (a device-scope release and
// acquire per workgroup, to let the last one merge, cost far more than the
// second launch on this chip)
template <bool COUNT>
__global__ __launch_bounds__(64) void k4_accept(K4Args a) {
  accept_item<COUNT>(a, blockIdx.x, threadIdx.x);
}


// ---------------------------------------------------------------------------
// K5: final selection and backtrace
// ---------------------------------------------------------------------------

struct K5Args {
  DevState st;
  int B, W, T, pad, R, steps;
  int32_t* tokens;     // [B][R][T]
  int32_t* lengths;    // [B][R]
  float* norms;        // [B][R]
};

template <int WMAX>
__global__ __launch_bounds__(64) void k5_finalize(K5Args a) {
  __shared__ float hn[2 * WMAX];
  __shared__ int hs[2 * WMAX], hr[2 * WMAX], hl[2 * WMAX], hp[2 * WMAX], ht[2 * WMAX];
  __shared__ int order[2 * WMAX];
  __shared__ int nh;
  const int b = blockIdx.x, tid = threadIdx.x, W = a.W;
  const DevState& st = a.st;
  if (tid == 0) {
    // a copy of the finished set, then the live beams of an unfinished item
    int n = st.hcount[b];
    for (int i = 0; i < n; ++i) {
      hn[i] = st.hnorm[b * W + i];
      hs[i] = st.hstep[b * W + i];
      hr[i] = st.hrank[b * W + i];
      hl[i] = st.hlen[b * W + i];
      hp[i] = st.hpar[b * W + i];
      ht[i] = st.htok[b * W + i];
    }
    if (!st.done[b]) {
      const int T1 = a.steps;
      const int bp = ((T1 - 1) * a.B + b) * W;
      for (int i = 0; i < W; ++i) {
        const float s = st.s[b * W + i];
        if (!(s > -kInf)) continue;
        const float norm = (float)((double)s / st.lpt[T1]);
        const int rank = st.slot_rank[b * W + i];
        int slot;
        if (n < W) {
          slot = n++;
        } else {
          int worst = 0;
          for (int q = 1; q < W; ++q)
            if (hyp_better(hn[worst], hs[worst], hr[worst], hn[q], hs[q], hr[q])) worst = q;
          if (!hyp_better(norm, T1, rank, hn[worst], hs[worst], hr[worst])) continue;
          slot = worst;
        }
        hn[slot] = norm;
        hs[slot] = T1;
        hr[slot] = rank;
        hl[slot] = T1;
        hp[slot] = st.bp_par[bp + i];
        ht[slot] = st.bp_tok[bp + i];
      }
    }
    // best first
    for (int i = 0; i < n; ++i) order[i] = i;
    for (int i = 1; i < n; ++i) {
      int x = order[i], k = i;
      while (k > 0 && hyp_better(hn[x], hs[x], hr[x], hn[order[k - 1]], hs[order[k - 1]],
                                 hr[order[k - 1]])) {
        order[k] = order[k - 1];
        --k;
      }
      order[k] = x;
    }
    nh = n;
  }
  __syncthreads();
  for (int r = tid; r < a.R; r += blockDim.x) {
    int32_t* out = a.tokens + ((int64_t)b * a.R + r) * a.T;
    for (int i = 0; i < a.T; ++i) out[i] = a.pad;
    if (r < nh) {
      const int h = order[r];
      const int len = hl[h];
      out[len - 1] = ht[h];
      int slot = hp[h];
      for (int u = hs[h] - 1; u >= 1; --u) {
        const int bp = ((u - 1) * a.B + b) * W + slot;
        out[u - 1] = st.bp_tok[bp];
        slot = st.bp_par[bp];
      }
      a.lengths[b * a.R + r] = len;
      a.norms[b * a.R + r] = hn[h];
    } else {
      a.lengths[b * a.R + r] = 0;
      a.norms[b * a.R + r] = -kInf;
    }
  }
}

// ---------------------------------------------------------------------------
// K6/K7: paged KV cache -- block tables with copy on write
// ---------------------------------------------------------------------------

constexpr int kPagedMaxBlocks = 4096;  // blocks per item (LDS reference counts)
constexpr int kPagedMaxTable = 2048;   // W * max_blocks (LDS table copies)

struct PagedDev {
  int* table;     // [B*W][mb] global block ids, -1 = none
  int* refc;      // [B*bpi] live-row references of each block
  int* freel;     // [B][bpi] stack of free global block ids
  int* nfree;     // [B]
  int* overflow;  // [1]
  int* cpy;       // [B*W][3] copy list of the step: source block, destination block, positions
  int* ncpy;      // [2] entries of the list, by step parity
};

struct K6Args {
  PagedDev pg;
  const float* s;       // [B*W] running scores after the step
  const uint8_t* done;  // [B] after the step
  const int* plan;      // [B][kPlanStride] the step's reorder plan
  int W, bs, bpi, mb, t;
};

// One workgroup per item. The item's table, reference counts and free list
// are staged in LDS; the new table is formed from the old one and the plan,
// references are added before old ones are dropped (a block both gains and
// loses references without being freed in between), and a block whose count
// reaches zero goes back to the free list. Then wave 0 makes position t
// writable for every live slot.
__global__ __launch_bounds__(kThreads) void k6_paged_reorder(K6Args a) {
  __shared__ int refc[kPagedMaxBlocks];
  __shared__ int fstack[kPagedMaxBlocks];
  __shared__ int told[kPagedMaxTable];
  __shared__ int tnew[kPagedMaxTable];
  __shared__ int par[kMaxBeam];
  __shared__ int plan_sh[2 + 2 * kMaxBeam];
  __shared__ int nfree_sh;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int W = a.W, mb = a.mb, bpi = a.bpi, t = a.t, bs = a.bs;
  const int base = b * bpi;          // the item's first global block id
  const int nb = (t + bs - 1) / bs;  // blocks holding positions [0, t)
  const int nt = W * mb;
  const PagedDev& pg = a.pg;
  const int* plan = a.plan + b * kPlanStride;
  const bool item_done = a.done[b] != 0;
  const int nf = min(max(pg.nfree[b], 0), bpi);
  for (int e = tid; e < bpi; e += kThreads) refc[e] = pg.refc[base + e];
  for (int e = tid; e < nf; e += kThreads) fstack[e] = pg.freel[base + e];
  for (int e = tid; e < nt; e += kThreads) {
    const int v = pg.table[(int64_t)b * nt + e];
    told[e] = (v >= base && v < base + bpi) ? v : -1;  // only the item's own blocks
  }
  if (tid < 2 + 2 * kMaxBeam) plan_sh[tid] = plan[tid];  // staged with the other loads
  if (tid == 0) nfree_sh = nf;
  __syncthreads();
  if (tid < W) {  // parent of each slot: itself unless the plan moves it
    int pp = tid;
    if (plan_sh[1] > 0)
      for (int q = 0; q < plan_sh[0]; ++q)
        if ((plan_sh[2 + kMaxBeam + q] >> tid) & 1) pp = plan_sh[2 + q];
    par[tid] = pp;
  }
  __syncthreads();

  // new table: a live slot of a running item takes its parent's blocks
  // [0, nb); rows of dead slots and of finished items hold nothing
  for (int e = tid; e < nt; e += kThreads) {
    const int i = e / mb, k = e - i * mb;
    int v = -1;
    if (!item_done && a.s[b * W + i] > -kInf && k < nb) v = told[par[i] * mb + k];
    tnew[e] = v;
  }
  __syncthreads();
  for (int e = tid; e < nt; e += kThreads)
    if (tnew[e] >= 0) atomicAdd(&refc[tnew[e] - base], 1);
  __syncthreads();
  for (int e = tid; e < nt; e += kThreads)
    if (told[e] >= 0 && atomicSub(&refc[told[e] - base], 1) == 1) {
      const int slot = atomicAdd(&nfree_sh, 1);
      if (slot < kPagedMaxBlocks) fstack[slot] = told[e];
    }
  __syncthreads();

  // position t: a fresh block at a block boundary; inside a block that a
  // lower live slot also holds, a private copy of its first t % bs positions
  if (tid < 64) {
    const int lane = tid;
    const int blk = t / bs, off = t - blk * bs;
    const bool live = lane < W && !item_done && a.s[b * W + lane] > -kInf;
    const int cur = live ? tnew[lane * mb + blk] : -1;
    bool shared = false;
    for (int j = 0; j < W; ++j) {
      const bool lj = !item_done && a.s[b * W + j] > -kInf;
      if (j < lane && lj && cur >= 0 && tnew[j * mb + blk] == cur) shared = true;
    }
    const bool alloc = live && (off == 0 || cur < 0 || shared);
    const bool copy = live && off > 0 && cur >= 0 && shared;
    const uint64_t below = (lane == 0) ? 0 : (~(uint64_t)0 >> (64 - lane));
    const uint64_t am = __ballot(alloc);
    const int rank = __popcll(am & below);
    const int avail = min(nfree_sh, bpi);
    int nbk = -1;
    if (alloc && rank < avail) nbk = fstack[avail - 1 - rank];
    if (nbk < base || nbk >= base + bpi) nbk = -1;  // only the item's own blocks
    const bool got = nbk >= 0;
    if (alloc && !got) {  // out of blocks: the slot is left without one
      pg.overflow[0] = 1;
      if (cur >= 0) {
        tnew[lane * mb + blk] = -1;
        atomicSub(&refc[cur - base], 1);  // still held by a lower slot
      }
    }
    const uint64_t cm = __ballot(copy && got);
    // the item's copies go to the step's global list (one atomic per item);
    // the other parity's count is cleared for the next step
    int cbase = 0;
    if (lane == 0 && cm) cbase = atomicAdd(&pg.ncpy[t & 1], __popcll(cm));
    cbase = __builtin_amdgcn_readfirstlane(cbase);
    if (b == 0 && lane == 0) pg.ncpy[(t + 1) & 1] = 0;
    __builtin_amdgcn_wave_barrier();
    if (got) {
      tnew[lane * mb + blk] = nbk;
      refc[nbk - base] = 1;
      if (copy) {
        atomicSub(&refc[cur - base], 1);
        int* c = pg.cpy + ((int64_t)cbase + __popcll(cm & below)) * 3;
        c[0] = cur;
        c[1] = nbk;
        c[2] = off;
      }
    }
    if (lane == 0) {
      const int used = __popcll(am) < avail ? __popcll(am) : avail;
      nfree_sh = avail - used;
    }
  }
  __syncthreads();

  for (int e = tid; e < bpi; e += kThreads) pg.refc[base + e] = refc[e];
  const int nf2 = min(nfree_sh, bpi);
  for (int e = tid; e < nf2; e += kThreads) pg.freel[base + e] = fstack[e];
  for (int e = tid; e < nt; e += kThreads) pg.table[(int64_t)b * nt + e] = tnew[e];
  if (tid == 0) pg.nfree[b] = nf2;
}

struct K7Args {
  char* pools[kMaxPlanesPerLaunch];
  int n_planes;
  int64_t block_stride, pos_stride;
  int words_per_pos;
  int tiles;             // word tiles of a copy of block_size - 1 positions
  int groups;            // groups of kCopyPlanes pools
  const int* cpy;
  const int* ncpy;
  int parity;
  int max_copies;        // capacity of the list: B*W
};

// The copies on write of the step: a fixed grid walks the units (copy, word
// tile, group of kCopyPlanes pools) of the step's list; a thread moves one
// word of each pool of its unit's group, all loads issued before the first
// store.
constexpr int kCopyPlanes = 8;
constexpr int kCopyGrid = 256;
template <int WORD>
__global__ __launch_bounds__(kThreads) void k7_paged_copy(K7Args a) {
  using WT = typename Word<WORD>::type;
  const int units = min(a.ncpy[a.parity], a.max_copies) * a.tiles * a.groups;
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int f = u / (a.tiles * a.groups);
    const int rest = u - f * a.tiles * a.groups;
    const int tile = rest / a.groups, grp = rest - tile * a.groups;
    const int* c = a.cpy + (int64_t)f * 3;
    const int src = c[0], dst = c[1], npos = c[2];
    const int e = tile * kThreads + threadIdx.x;
    if (e >= npos * a.words_per_pos) continue;
    const int pos = e / a.words_per_pos;
    const int64_t off = pos * a.pos_stride + (int64_t)(e - pos * a.words_per_pos) * WORD;
    const int64_t so = src * a.block_stride + off, d = dst * a.block_stride + off;
    const int p0 = grp * kCopyPlanes;
    const int np = min(kCopyPlanes, a.n_planes - p0);
    WT v[kCopyPlanes];
#pragma unroll
    for (int k = 0; k < kCopyPlanes; ++k)
      if (k < np) v[k] = *reinterpret_cast<const WT*>(a.pools[p0 + k] + so);
#pragma unroll
    for (int k = 0; k < kCopyPlanes; ++k)
      if (k < np) *reinterpret_cast<WT*>(a.pools[p0 + k] + d) = v[k];
  }
}

// Reset: row r of item b holds block b*bpi + w in logical block 0; the other
// blocks of the item are free.
__global__ void k6_paged_init(PagedDev pg, int B, int W, int bpi, int mb) {
  const int b = blockIdx.x;
  const int base = b * bpi;
  for (int e = threadIdx.x; e < bpi; e += blockDim.x) {
    pg.refc[base + e] = e < W ? 1 : 0;
    if (e < bpi - W) pg.freel[base + e] = base + bpi - 1 - e;
  }
  for (int e = threadIdx.x; e < W * mb; e += blockDim.x) {
    const int i = e / mb, k = e - i * mb;
    pg.table[(int64_t)b * W * mb + e] = k == 0 ? base + i : -1;
  }
  if (threadIdx.x == 0) {
    pg.nfree[b] = bpi - W;
    if (b == 0) {
      pg.overflow[0] = 0;
      pg.ncpy[0] = 0;
      pg.ncpy[1] = 0;
    }
  }
}

// ---------------------------------------------------------------------------
// init: running scores, finished sets, done flags, length-penalty table
// ---------------------------------------------------------------------------

struct InitArgs {
  DevState st;
  double* lpt;
  int* qn;  // two-pass queue lengths, or null
  int B, W, T, lp;
  double alpha;
};

__global__ void k0_init(InitArgs a) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < a.B * a.W) {
    a.st.s[i] = (i % a.W == 0) ? 0.0f : -kInf;
    a.st.slot_rank[i] = 0;
  }
  if (i < a.B) {
    a.st.done[i] = 0;
    a.st.hcount[i] = 0;
    a.st.plan[i * kPlanStride + 1] = 0;
    if (a.qn) a.qn[i] = 0;
  }
  if (i <= a.T) {
    double v = 1.0;
    if (a.lp == BS_LP_GNMT) v = pow((5.0 + (double)i) / 6.0, a.alpha);
    else if (a.lp == BS_LP_POW) v = pow((double)i, a.alpha);
    a.lpt[i] = v;
  }
}

}  // namespace

// ===========================================================================
// host runtime
// ===========================================================================

struct bs_state {
  bs_config cfg;
  hipStream_t stream;
  int device;
  int B, W, V, T, rows, wmax, ept, tile, tiles;
  int K, kmax;          // candidates ranked per item (W or 2W), pow2 bound
  int t;                // steps taken
  void* block;          // the one device allocation
  DevState st;
  double* lpt;
  float* pm;
  float* ps;
  float* px;
  int* pv;
  // two-pass selection
  int KP, cap;
  float* gm;
  float* qc;
  int* qj;
  int* qn;
};

struct bs_kv_paged {
  bs_state* h;
  int bs, bpi, mb;
  int last_t;  // the step last reordered (0: none since the reset)
  void* block;
  PagedDev pg;
};

struct bs_verify_state {
  hipStream_t stream;
  int device;
  int B, k, V, dtype, ept, tile, tiles;
  void* block;
  float* px;
  int* pv;
  int* pc;
};

namespace {

int pow2ceil(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

size_t align_up(size_t n) { return (n + 255) & ~(size_t)255; }

int choose_ept(int rows, int V, int hint) {
  if (hint == 16 || hint == 32 || hint == 64) return hint;
  // the largest per-thread tile that still gives >= 1024 workgroups
  for (int e : {64, 32}) {
    const int64_t tiles = (V + (int64_t)kThreads * e - 1) / ((int64_t)kThreads * e);
    if ((int64_t)rows * tiles >= 1024) return e;
  }
  return 16;
}

int launch_status() { return hipGetLastError() == hipSuccess ? BS_OK : BS_EDEVICE; }

// ---- K1 dispatch ----------------------------------------------------------
template <int WMAX, typename T, int EPT>
void launch_k1_a(const K1Args& a, bool aligned, dim3 grid, hipStream_t s) {
  if (aligned)
    hipLaunchKernelGGL((k1_expand_select<WMAX, T, EPT, true>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((k1_expand_select<WMAX, T, EPT, false>), grid, dim3(kThreads), 0, s, a);
}
template <int WMAX, typename T>
void launch_k1_e(const K1Args& a, int ept, bool aligned, dim3 grid, hipStream_t s) {
  if (ept == 64) launch_k1_a<WMAX, T, 64>(a, aligned, grid, s);
  else if (ept == 32) launch_k1_a<WMAX, T, 32>(a, aligned, grid, s);
  else launch_k1_a<WMAX, T, 16>(a, aligned, grid, s);
}
template <int WMAX>
void launch_k1_t(const K1Args& a, int dtype, int ept, bool aligned, dim3 grid, hipStream_t s) {
  if (dtype == BS_BF16) launch_k1_e<WMAX, uint16_t>(a, ept, aligned, grid, s);
  else launch_k1_e<WMAX, float>(a, ept, aligned, grid, s);
}
void launch_k1(const K1Args& a, int wmax, int dtype, int ept, bool aligned, dim3 grid,
               hipStream_t s) {
  switch (wmax) {
    case 1: launch_k1_t<1>(a, dtype, ept, aligned, grid, s); break;
    case 2: launch_k1_t<2>(a, dtype, ept, aligned, grid, s); break;
    case 4: launch_k1_t<4>(a, dtype, ept, aligned, grid, s); break;
    case 8: launch_k1_t<8>(a, dtype, ept, aligned, grid, s); break;
    default: launch_k1_t<16>(a, dtype, ept, aligned, grid, s); break;
  }
}

template <typename T, int EPT>
void launch_cf_a(const CFArgs& a, bool aligned, dim3 grid, hipStream_t s) {
  if (aligned) {
    hipLaunchKernelGGL((l1_coarse<T, EPT, true>), grid, dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL((l2_fine<T, EPT, true>), grid, dim3(kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((l1_coarse<T, EPT, false>), grid, dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL((l2_fine<T, EPT, false>), grid, dim3(kThreads), 0, s, a);
  }
}
template <typename T>
void launch_cf_t(const CFArgs& a, int ept, bool aligned, dim3 grid, hipStream_t s) {
  if (ept == 64) launch_cf_a<T, 64>(a, aligned, grid, s);
  else if (ept == 32) launch_cf_a<T, 32>(a, aligned, grid, s);
  else launch_cf_a<T, 16>(a, aligned, grid, s);
}
template <typename T>
void launch_l3_t(const L3Args& a, int wmax, hipStream_t s) {
  dim3 g(a.k2.B), blk(kThreads);
  switch (wmax) {
    case 1: hipLaunchKernelGGL((l3_sort_finalize<1, T>), g, blk, 0, s, a); break;
    case 2: hipLaunchKernelGGL((l3_sort_finalize<2, T>), g, blk, 0, s, a); break;
    case 4: hipLaunchKernelGGL((l3_sort_finalize<4, T>), g, blk, 0, s, a); break;
    case 8: hipLaunchKernelGGL((l3_sort_finalize<8, T>), g, blk, 0, s, a); break;
    default: hipLaunchKernelGGL((l3_sort_finalize<16, T>), g, blk, 0, s, a); break;
  }
}

void launch_k2(const K2Args& a, int wmax, hipStream_t s) {
  dim3 g(a.B), blk(kThreads);
  if (a.tiles <= 64) {
    const int H = a.tiles <= 16 ? 1 : (a.tiles <= 32 ? 2 : 4);  // tiles per lane
    switch (wmax * 8 + H) {
#define K2SEL(WM, HH) \
  case WM * 8 + HH: hipLaunchKernelGGL((k2_select_finalize<WM, HH>), g, blk, 0, s, a); break;
      K2SEL(1, 1) K2SEL(1, 2) K2SEL(1, 4)
      K2SEL(2, 1) K2SEL(2, 2) K2SEL(2, 4)
      K2SEL(4, 1) K2SEL(4, 2) K2SEL(4, 4)
      K2SEL(8, 1) K2SEL(8, 2) K2SEL(8, 4)
      K2SEL(16, 1) K2SEL(16, 2) K2SEL(16, 4)
#undef K2SEL
      default: break;
    }
    return;
  }
  switch (wmax) {
    case 1: hipLaunchKernelGGL((k2_merge_finalize<1>), g, blk, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k2_merge_finalize<2>), g, blk, 0, s, a); break;
    case 4: hipLaunchKernelGGL((k2_merge_finalize<4>), g, blk, 0, s, a); break;
    case 8: hipLaunchKernelGGL((k2_merge_finalize<8>), g, blk, 0, s, a); break;
    default: hipLaunchKernelGGL((k2_merge_finalize<16>), g, blk, 0, s, a); break;
  }
}

// ---- K3 dispatch ----------------------------------------------------------
template <int WMAX, int WORD, bool CONTIG>
void launch_k3_c(const K3Args& a, int64_t tiles_per_row, int B, int nplanes, hipStream_t s) {
  // one 16-byte word per thread and parent: more threads with fewer stores in
  // flight each measured faster than 2, 4 or 8 words per thread
  constexpr int NP = 1;
  const int64_t tiles = (a.words + (int64_t)kK3Threads * NP - 1) / ((int64_t)kK3Threads * NP);
  (void)tiles_per_row;
  dim3 g((unsigned)tiles, B, nplanes);
  hipLaunchKernelGGL((k3_kv_reorder<WMAX, WORD, NP, CONTIG>), g, dim3(kK3Threads), 0, s, a);
}
template <int WMAX>
void launch_k3_w(const K3Args& a, int word, bool contig, int B, int nplanes, hipStream_t s) {
  if (word == 16) {
    if (contig) launch_k3_c<WMAX, 16, true>(a, 0, B, nplanes, s);
    else launch_k3_c<WMAX, 16, false>(a, 0, B, nplanes, s);
  } else {
    if (contig) launch_k3_c<WMAX, 4, true>(a, 0, B, nplanes, s);
    else launch_k3_c<WMAX, 4, false>(a, 0, B, nplanes, s);
  }
}
void launch_k3(const K3Args& a, int wmax, int word, bool contig, int B, int nplanes,
               hipStream_t s) {
  switch (wmax) {
    case 1: launch_k3_w<1>(a, word, contig, B, nplanes, s); break;
    case 2: launch_k3_w<2>(a, word, contig, B, nplanes, s); break;
    case 4: launch_k3_w<4>(a, word, contig, B, nplanes, s); break;
    case 8: launch_k3_w<8>(a, word, contig, B, nplanes, s); break;
    default: launch_k3_w<16>(a, word, contig, B, nplanes, s); break;
  }
}

void launch_k5(const K5Args& a, int wmax, hipStream_t s) {
  dim3 g(a.B), blk(64);
  switch (wmax) {
    case 1: hipLaunchKernelGGL((k5_finalize<1>), g, blk, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k5_finalize<2>), g, blk, 0, s, a); break;
    case 4: hipLaunchKernelGGL((k5_finalize<4>), g, blk, 0, s, a); break;
    case 8: hipLaunchKernelGGL((k5_finalize<8>), g, blk, 0, s, a); break;
    default: hipLaunchKernelGGL((k5_finalize<16>), g, blk, 0, s, a); break;
  }
}

// ---- K4 dispatch ----------------------------------------------------------
template <typename T, int EPT, bool COUNT>
void launch_k4_a(const K4Args& a, bool aligned, dim3 grid, hipStream_t s) {
  if (aligned)
    hipLaunchKernelGGL((k4_verify<T, EPT, true, COUNT>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((k4_verify<T, EPT, false, COUNT>), grid, dim3(kThreads), 0, s, a);
}

void fill_k2_args(K2Args& a2, bs_state* h, int t, int32_t* beam_idx, int32_t* token_id,
                  float* scores, uint8_t* done) {
  a2.st = h->st;
  a2.pm = h->pm;
  a2.ps = h->ps;
  a2.px = h->px;
  a2.pv = h->pv;
  a2.B = h->B;
  a2.W = h->W;
  a2.K = h->K;
  a2.V = h->V;
  a2.T = h->T;
  a2.tiles = h->tiles;
  a2.eos = h->cfg.eos_id;
  a2.pad = h->cfg.pad_id;
  a2.stop = h->cfg.stop;
  a2.alpha = h->cfg.alpha;
  a2.t = t;
  a2.out_beam = beam_idx;
  a2.out_tok = token_id;
  a2.out_score = scores;
  a2.out_done = done;
}

constexpr int kRowVerifyMinRows = 256;

template <typename T, bool COUNT>
void launch_k4_row(const K4Args& a, bool aligned, int rows, hipStream_t s) {
  if (aligned)
    hipLaunchKernelGGL((k4_row<T, true, COUNT>), dim3(rows), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((k4_row<T, false, COUNT>), dim3(rows), dim3(kThreads), 0, s, a);
}

void launch_k4_tiles(const K4Args& a, int dtype, bool count, bool aligned, dim3 grid,
                     hipStream_t s) {
  if (count) {
    if (dtype == BS_BF16) launch_k4_a<uint16_t, 16, true>(a, aligned, grid, s);
    else launch_k4_a<float, 16, true>(a, aligned, grid, s);
  } else {
    if (dtype == BS_BF16) launch_k4_a<uint16_t, 16, false>(a, aligned, grid, s);
    else launch_k4_a<float, 16, false>(a, aligned, grid, s);
  }
}

int launch_init(bs_state* h) {
  InitArgs ia;
  ia.st = h->st;
  ia.lpt = h->lpt;
  ia.qn = h->qn;
  ia.B = h->B;
  ia.W = h->W;
  ia.T = h->T;
  ia.lp = h->cfg.lp;
  ia.alpha = h->cfg.alpha;
  int n = h->B * h->W;
  if (h->T + 1 > n) n = h->T + 1;
  hipLaunchKernelGGL(k0_init, dim3((n + 255) / 256), dim3(256), 0, h->stream, ia);
  return launch_status();
}

}  // namespace

extern "C" {

const char* bs_strerror(int status) {
  switch (status) {
    case BS_OK: return "ok";
    case BS_EINVAL: return "invalid argument";
    case BS_ENOMEM: return "device allocation failed";
    case BS_EDEVICE: return "HIP runtime error";
    case BS_ESTATE: return "call not valid in the current state";
    default: return "unknown status";
  }
}

int bs_create(const bs_config* cfg, void* hip_stream, bs_state** out) {
  if (!cfg || !out) return BS_EINVAL;
  *out = nullptr;
  const bs_config c = *cfg;
  if (c.batch < 1 || c.beam < 1 || c.beam > kMaxBeam || c.vocab < 1 || c.max_steps < 1)
    return BS_EINVAL;
  if ((int64_t)c.beam * c.vocab >= ((int64_t)1 << 31)) return BS_EINVAL;
  if ((int64_t)c.batch * c.beam * c.max_steps >= ((int64_t)1 << 31)) return BS_EINVAL;
  if (c.logits_dtype != BS_F32 && c.logits_dtype != BS_BF16) return BS_EINVAL;
  if (c.lp < BS_LP_NONE || c.lp > BS_LP_POW) return BS_EINVAL;
  if (c.stop < BS_STOP_TRUE || c.stop > BS_STOP_NEVER) return BS_EINVAL;
  if (c.num_return < 1 || c.num_return > c.beam) return BS_EINVAL;
  if (c.tile_elems != 0 && c.tile_elems != 16 && c.tile_elems != 32 && c.tile_elems != 64)
    return BS_EINVAL;
  if (!(c.alpha == c.alpha)) return BS_EINVAL;
  if (c.prune != BS_PRUNE_TOPW && c.prune != BS_PRUNE_TOP2W) return BS_EINVAL;
  if (c.prune == BS_PRUNE_TOP2W && 2 * c.beam > kMaxBeam) return BS_EINVAL;
  if (c.select != BS_SELECT_FUSED && c.select != BS_SELECT_TWO_PASS) return BS_EINVAL;

  bs_state* h = (bs_state*)calloc(1, sizeof(bs_state));
  if (!h) return BS_ENOMEM;
  h->cfg = c;
  h->stream = (hipStream_t)hip_stream;
  if (hipGetDevice(&h->device) != hipSuccess) {
    free(h);
    return BS_EDEVICE;
  }
  h->B = c.batch;
  h->W = c.beam;
  h->V = c.vocab;
  h->T = c.max_steps;
  h->rows = c.batch * c.beam;
  h->wmax = pow2ceil(c.beam);
  h->K = c.prune == BS_PRUNE_TOP2W ? 2 * c.beam : c.beam;
  h->kmax = pow2ceil(h->K);
  h->ept = choose_ept(h->rows, c.vocab, c.tile_elems);
  h->tile = kThreads * h->ept;
  h->tiles = (c.vocab + h->tile - 1) / h->tile;

  const size_t RW = (size_t)h->rows;
  const size_t PT = RW * h->tiles;
  const size_t BT = (size_t)h->T * RW;
  const bool two = c.select == BS_SELECT_TWO_PASS;
  h->KP = pow2ceil(h->K);
  h->cap = kThreads * h->KP;
  size_t sizes[] = {
      RW * 4,                 // s
      RW * 4,                 // slot_rank
      (size_t)h->B,           // done
      RW * 4, RW * 4, RW * 4, RW * 4, RW * 4, RW * 4, RW * 4,  // finished set
      (size_t)h->B * 4,       // hcount
      BT * 4, BT * 4,         // backpointers
      (size_t)h->B * h->K * 4, (size_t)h->B * h->K * 4,  // selection
      (size_t)h->B * kPlanStride * 4,  // plan
      ((size_t)h->T + 1) * 8, // lpt
      PT * 4, PT * 4,         // pm, ps
      PT * h->kmax * 4, PT * h->kmax * 4,  // px, pv
      two ? PT * h->KP * 4 : 0,            // two-pass: group maxima
      two ? (size_t)h->B * h->cap * 4 : 0, two ? (size_t)h->B * h->cap * 4 : 0,  // queue
      two ? (size_t)h->B * 4 : 0,          // queue lengths
  };
  const int n = sizeof(sizes) / sizeof(sizes[0]);
  size_t total = 0;
  for (int i = 0; i < n; ++i) total += align_up(sizes[i]);
  if (hipMalloc(&h->block, total) != hipSuccess) {
    (void)hipGetLastError();
    free(h);
    return BS_ENOMEM;
  }
  char* p = (char*)h->block;
  void* ptr[n];
  for (int i = 0; i < n; ++i) {
    ptr[i] = p;
    p += align_up(sizes[i]);
  }
  int i = 0;
  h->st.s = (float*)ptr[i++];
  h->st.slot_rank = (int*)ptr[i++];
  h->st.done = (uint8_t*)ptr[i++];
  h->st.hnorm = (float*)ptr[i++];
  h->st.hraw = (float*)ptr[i++];
  h->st.hlen = (int*)ptr[i++];
  h->st.hstep = (int*)ptr[i++];
  h->st.hrank = (int*)ptr[i++];
  h->st.hpar = (int*)ptr[i++];
  h->st.htok = (int*)ptr[i++];
  h->st.hcount = (int*)ptr[i++];
  h->st.bp_par = (int*)ptr[i++];
  h->st.bp_tok = (int*)ptr[i++];
  h->st.sel_j = (int*)ptr[i++];
  h->st.sel_c = (float*)ptr[i++];
  h->st.plan = (int*)ptr[i++];
  h->lpt = (double*)ptr[i++];
  h->st.lpt = h->lpt;
  h->pm = (float*)ptr[i++];
  h->ps = (float*)ptr[i++];
  h->px = (float*)ptr[i++];
  h->pv = (int*)ptr[i++];
  h->gm = two ? (float*)ptr[i] : nullptr;
  ++i;
  h->qc = two ? (float*)ptr[i] : nullptr;
  ++i;
  h->qj = two ? (int*)ptr[i] : nullptr;
  ++i;
  h->qn = two ? (int*)ptr[i] : nullptr;
  ++i;

  int rc = launch_init(h);
  if (rc == BS_OK && hipStreamSynchronize(h->stream) != hipSuccess) rc = BS_EDEVICE;
  if (rc != BS_OK) {
    (void)hipFree(h->block);
    free(h);
    return rc;
  }
  *out = h;
  return BS_OK;
}

int bs_reset(bs_state* h) {
  if (!h) return BS_EINVAL;
  int rc = launch_init(h);
  if (rc == BS_OK) h->t = 0;
  return rc;
}

int bs_step(bs_state* h, const void* logits, int64_t row_stride_elems, int32_t* beam_idx,
            int32_t* token_id, float* scores, uint8_t* done) {
  if (!h || !logits || !beam_idx || !token_id || !scores || !done) return BS_EINVAL;
  if (row_stride_elems < h->V) return BS_EINVAL;
  if (h->t >= h->T) return BS_ESTATE;
  const int t = h->t + 1;
  const int esize = h->cfg.logits_dtype == BS_BF16 ? 2 : 4;
  const bool aligned = ((uintptr_t)logits % 16 == 0) && ((row_stride_elems * esize) % 16 == 0);

  if (h->cfg.select == BS_SELECT_TWO_PASS) {
    CFArgs cf;
    cf.logits = logits;
    cf.stride = row_stride_elems;
    cf.V = h->V;
    cf.W = h->W;
    cf.K = h->K;
    cf.KP = h->KP;
    cf.tile = h->tile;
    cf.tiles = h->tiles;
    cf.s = h->st.s;
    cf.done = h->st.done;
    cf.pm = h->pm;
    cf.ps = h->ps;
    cf.gm = h->gm;
    cf.qc = h->qc;
    cf.qj = h->qj;
    cf.qn = h->qn;
    cf.cap = h->cap;
    const dim3 grid(h->tiles, h->rows);
    if (h->cfg.logits_dtype == BS_BF16) launch_cf_t<uint16_t>(cf, h->ept, aligned, grid, h->stream);
    else launch_cf_t<float>(cf, h->ept, aligned, grid, h->stream);
    int rc = launch_status();
    if (rc != BS_OK) return rc;
    L3Args a3;
    a3.cf = cf;
    fill_k2_args(a3.k2, h, t, beam_idx, token_id, scores, done);
    if (h->cfg.logits_dtype == BS_BF16) launch_l3_t<uint16_t>(a3, h->kmax, h->stream);
    else launch_l3_t<float>(a3, h->kmax, h->stream);
    rc = launch_status();
    if (rc != BS_OK) return rc;
    h->t = t;
    return BS_OK;
  }

  K1Args a1;
  a1.logits = logits;
  a1.stride = row_stride_elems;
  a1.V = h->V;
  a1.W = h->W;
  a1.K = h->K;
  a1.tile = h->tile;
  a1.tiles = h->tiles;
  a1.s = h->st.s;
  a1.done = h->st.done;
  a1.pm = h->pm;
  a1.ps = h->ps;
  a1.px = h->px;
  a1.pv = h->pv;
  launch_k1(a1, h->kmax, h->cfg.logits_dtype, h->ept, aligned, dim3(h->tiles, h->rows),
            h->stream);
  int rc = launch_status();
  if (rc != BS_OK) return rc;

  K2Args a2;
  fill_k2_args(a2, h, t, beam_idx, token_id, scores, done);
  launch_k2(a2, h->kmax, h->stream);
  rc = launch_status();
  if (rc != BS_OK) return rc;
  h->t = t;
  return BS_OK;
}

int bs_reorder_kv(bs_state* h, const bs_kv_desc* kv, int32_t gen_len) {
  if (!h || !kv || !kv->planes || kv->n_planes < 1 || gen_len < 0) return BS_EINVAL;
  if (kv->bytes_per_pos <= 0 || kv->row_stride <= 0 || kv->pos_stride <= 0 || kv->pos_offset < 0)
    return BS_EINVAL;
  if (h->t == 0) return BS_ESTATE;
  if (gen_len == 0) return BS_OK;
  const int64_t base_off = kv->pos_offset * kv->pos_stride;
  bool a16 = (kv->bytes_per_pos % 16 == 0) && (kv->row_stride % 16 == 0) &&
             (kv->pos_stride % 16 == 0) && (base_off % 16 == 0);
  bool a4 = (kv->bytes_per_pos % 4 == 0) && (kv->row_stride % 4 == 0) &&
            (kv->pos_stride % 4 == 0) && (base_off % 4 == 0);
  for (int i = 0; i < kv->n_planes; ++i) {
    if (!kv->planes[i]) return BS_EINVAL;
    a16 = a16 && ((uintptr_t)kv->planes[i] % 16 == 0);
    a4 = a4 && ((uintptr_t)kv->planes[i] % 4 == 0);
  }
  if (!a4) return BS_EINVAL;
  const int word = a16 ? 16 : 4;
  const bool contig = kv->pos_stride == kv->bytes_per_pos;
  K3Args a;
  a.row_stride = kv->row_stride;
  a.pos_stride = kv->pos_stride;
  a.base_off = base_off;
  a.words_per_pos = kv->bytes_per_pos / word;
  a.words = (int64_t)gen_len * a.words_per_pos;
  a.W = h->W;
  a.plan = h->st.plan;
  for (int p0 = 0; p0 < kv->n_planes; p0 += kMaxPlanesPerLaunch) {
    const int np = kv->n_planes - p0 < kMaxPlanesPerLaunch ? kv->n_planes - p0
                                                           : kMaxPlanesPerLaunch;
    for (int i = 0; i < np; ++i) a.planes[i] = (char*)kv->planes[p0 + i];
    launch_k3(a, h->wmax, word, contig, h->B, np, h->stream);
    const int rc = launch_status();
    if (rc != BS_OK) return rc;
  }
  return BS_OK;
}

int bs_kv_paged_create(bs_state* h, int32_t block_size, int32_t blocks_per_item,
                       bs_kv_paged** out) {
  if (!h || !out) return BS_EINVAL;
  *out = nullptr;
  if (block_size < 1 || blocks_per_item < h->W || blocks_per_item > kPagedMaxBlocks)
    return BS_EINVAL;
  const int mb = h->T / block_size + 1;
  if ((int64_t)h->W * mb > kPagedMaxTable) return BS_EINVAL;
  if ((int64_t)h->B * blocks_per_item >= ((int64_t)1 << 31)) return BS_EINVAL;
  bs_kv_paged* p = (bs_kv_paged*)calloc(1, sizeof(bs_kv_paged));
  if (!p) return BS_ENOMEM;
  p->h = h;
  p->bs = block_size;
  p->bpi = blocks_per_item;
  p->mb = mb;
  const size_t B = (size_t)h->B;
  const size_t sizes[] = {
      B * h->W * mb * 4,            // table
      B * blocks_per_item * 4,      // reference counts
      B * blocks_per_item * 4,      // free lists
      B * 4,                        // free counts
      4,                            // overflow flag
      B * h->W * 3 * 4,             // the step's copy list
      2 * 4,                        // its length, by step parity
  };
  const int n = sizeof(sizes) / sizeof(sizes[0]);
  size_t total = 0;
  for (int i = 0; i < n; ++i) total += align_up(sizes[i]);
  if (hipMalloc(&p->block, total) != hipSuccess) {
    (void)hipGetLastError();
    free(p);
    return BS_ENOMEM;
  }
  char* q = (char*)p->block;
  int* ptr[n];
  for (int i = 0; i < n; ++i) {
    ptr[i] = (int*)q;
    q += align_up(sizes[i]);
  }
  p->pg.table = ptr[0];
  p->pg.refc = ptr[1];
  p->pg.freel = ptr[2];
  p->pg.nfree = ptr[3];
  p->pg.overflow = ptr[4];
  p->pg.cpy = ptr[5];
  p->pg.ncpy = ptr[6];
  int rc = bs_kv_paged_reset(p);
  if (rc == BS_OK && hipStreamSynchronize(h->stream) != hipSuccess) rc = BS_EDEVICE;
  if (rc != BS_OK) {
    (void)hipFree(p->block);
    free(p);
    return rc;
  }
  *out = p;
  return BS_OK;
}

int bs_kv_paged_reset(bs_kv_paged* p) {
  if (!p) return BS_EINVAL;
  hipLaunchKernelGGL(k6_paged_init, dim3(p->h->B), dim3(kThreads), 0, p->h->stream, p->pg,
                     p->h->B, p->h->W, p->bpi, p->mb);
  const int rc = launch_status();
  if (rc == BS_OK) p->last_t = 0;
  return rc;
}

int bs_kv_paged_table(const bs_kv_paged* p, int32_t** table, int32_t* max_blocks) {
  if (!p || !table || !max_blocks) return BS_EINVAL;
  *table = p->pg.table;
  *max_blocks = p->mb;
  return BS_OK;
}

int bs_kv_paged_reorder(bs_kv_paged* p, const bs_kv_pool* pool, int32_t gen_len) {
  if (!p || !pool || !pool->pools || pool->n_planes < 1) return BS_EINVAL;
  if (pool->block_stride <= 0 || pool->pos_stride <= 0 || pool->bytes_per_pos <= 0)
    return BS_EINVAL;
  if (pool->bytes_per_pos > pool->pos_stride ||
      (int64_t)(p->bs - 1) * pool->pos_stride + pool->bytes_per_pos > pool->block_stride)
    return BS_EINVAL;
  bs_state* h = p->h;
  // every step is reordered once, in order: the table of step t is built on
  // that of step t-1
  if (h->t == 0 || gen_len != h->t || p->last_t + 1 != h->t) return BS_ESTATE;
  bool a16 = (pool->bytes_per_pos % 16 == 0) && (pool->pos_stride % 16 == 0) &&
             (pool->block_stride % 16 == 0);
  bool a4 = (pool->bytes_per_pos % 4 == 0) && (pool->pos_stride % 4 == 0) &&
            (pool->block_stride % 4 == 0);
  for (int i = 0; i < pool->n_planes; ++i) {
    if (!pool->pools[i]) return BS_EINVAL;
    a16 = a16 && ((uintptr_t)pool->pools[i] % 16 == 0);
    a4 = a4 && ((uintptr_t)pool->pools[i] % 4 == 0);
  }
  if (!a4) return BS_EINVAL;
  K6Args a6;
  a6.pg = p->pg;
  a6.s = h->st.s;
  a6.done = h->st.done;
  a6.plan = h->st.plan;
  a6.W = h->W;
  a6.bs = p->bs;
  a6.bpi = p->bpi;
  a6.mb = p->mb;
  a6.t = gen_len;
  hipLaunchKernelGGL(k6_paged_reorder, dim3(h->B), dim3(kThreads), 0, h->stream, a6);
  int rc = launch_status();
  if (rc != BS_OK) return rc;
  const int word = a16 ? 16 : 4;
  K7Args a7;
  a7.block_stride = pool->block_stride;
  a7.pos_stride = pool->pos_stride;
  a7.words_per_pos = (int)(pool->bytes_per_pos / word);
  a7.cpy = p->pg.cpy;
  a7.ncpy = p->pg.ncpy;
  a7.parity = gen_len & 1;
  a7.max_copies = h->B * h->W;
  const int64_t words = (int64_t)(p->bs - 1) * a7.words_per_pos;  // at most bs-1 positions
  a7.tiles = (int)((words + kThreads - 1) / kThreads);
  if (a7.tiles > 0) {
    for (int p0 = 0; p0 < pool->n_planes; p0 += kMaxPlanesPerLaunch) {
      const int np = pool->n_planes - p0 < kMaxPlanesPerLaunch ? pool->n_planes - p0
                                                                : kMaxPlanesPerLaunch;
      a7.n_planes = np;
      a7.groups = (np + kCopyPlanes - 1) / kCopyPlanes;
      for (int i = 0; i < np; ++i) a7.pools[i] = (char*)pool->pools[p0 + i];
      if (word == 16)
        hipLaunchKernelGGL(k7_paged_copy<16>, dim3(kCopyGrid), dim3(kThreads), 0, h->stream, a7);
      else
        hipLaunchKernelGGL(k7_paged_copy<4>, dim3(kCopyGrid), dim3(kThreads), 0, h->stream, a7);
      rc = launch_status();
      if (rc != BS_OK) return rc;
    }
  }
  p->last_t = h->t;
  return BS_OK;
}

int bs_kv_paged_status(bs_kv_paged* p, int32_t* overflow, int32_t* free_blocks) {
  if (!p || !overflow) return BS_EINVAL;
  hipStream_t s = p->h->stream;
  if (hipStreamSynchronize(s) != hipSuccess) return BS_EDEVICE;
  if (hipMemcpy(overflow, p->pg.overflow, 4, hipMemcpyDeviceToHost) != hipSuccess)
    return BS_EDEVICE;
  if (free_blocks &&
      hipMemcpy(free_blocks, p->pg.nfree, (size_t)p->h->B * 4, hipMemcpyDeviceToHost) !=
          hipSuccess)
    return BS_EDEVICE;
  return BS_OK;
}

void bs_kv_paged_destroy(bs_kv_paged* p) {
  if (!p) return;
  (void)hipStreamSynchronize(p->h->stream);
  (void)hipFree(p->block);
  free(p);
}

int bs_finalize(bs_state* h, int32_t* tokens, int32_t* lengths, float* norm_scores) {
  if (!h || !tokens || !lengths || !norm_scores) return BS_EINVAL;
  if (h->t == 0) return BS_ESTATE;
  K5Args a;
  a.st = h->st;
  a.B = h->B;
  a.W = h->W;
  a.T = h->T;
  a.pad = h->cfg.pad_id;
  a.R = h->cfg.num_return;
  a.steps = h->t;
  a.tokens = tokens;
  a.lengths = lengths;
  a.norms = norm_scores;
  launch_k5(a, h->wmax, h->stream);
  return launch_status();
}

int bs_last_selection(bs_state* h, int32_t* flat_idx, float* cand_score) {
  if (!h || !flat_idx || !cand_score) return BS_EINVAL;
  if (h->t == 0) return BS_ESTATE;
  const size_t n = (size_t)h->B * h->K;
  if (hipMemcpyAsync(flat_idx, h->st.sel_j, n * 4, hipMemcpyDeviceToDevice, h->stream) !=
          hipSuccess ||
      hipMemcpyAsync(cand_score, h->st.sel_c, n * 4, hipMemcpyDeviceToDevice, h->stream) !=
          hipSuccess)
    return BS_EDEVICE;
  return BS_OK;
}

int bs_get_finished(bs_state* h, float* norm, float* raw, int32_t* len, int32_t* step,
                    int32_t* rank, int32_t* count) {
  if (!h || !norm || !raw || !len || !step || !rank || !count) return BS_EINVAL;
  const size_t n = (size_t)h->rows * 4;
  const hipMemcpyKind k = hipMemcpyDeviceToDevice;
  if (hipMemcpyAsync(norm, h->st.hnorm, n, k, h->stream) != hipSuccess ||
      hipMemcpyAsync(raw, h->st.hraw, n, k, h->stream) != hipSuccess ||
      hipMemcpyAsync(len, h->st.hlen, n, k, h->stream) != hipSuccess ||
      hipMemcpyAsync(step, h->st.hstep, n, k, h->stream) != hipSuccess ||
      hipMemcpyAsync(rank, h->st.hrank, n, k, h->stream) != hipSuccess ||
      hipMemcpyAsync(count, h->st.hcount, (size_t)h->B * 4, k, h->stream) != hipSuccess)
    return BS_EDEVICE;
  return BS_OK;
}

int bs_steps_taken(const bs_state* h) { return h ? h->t : BS_EINVAL; }

void bs_destroy(bs_state* h) {
  if (!h) return;
  (void)hipStreamSynchronize(h->stream);
  (void)hipFree(h->block);
  free(h);
}

int bs_verify_create(int32_t batch, int32_t k, int32_t vocab, int32_t logits_dtype,
                     void* hip_stream, bs_verify_state** out) {
  if (!out) return BS_EINVAL;
  *out = nullptr;
  if (batch < 1 || k < 1 || k > 64 || vocab < 1) return BS_EINVAL;
  if (logits_dtype != BS_F32 && logits_dtype != BS_BF16) return BS_EINVAL;
  bs_verify_state* h = (bs_verify_state*)calloc(1, sizeof(bs_verify_state));
  if (!h) return BS_ENOMEM;
  h->stream = (hipStream_t)hip_stream;
  if (hipGetDevice(&h->device) != hipSuccess) {
    free(h);
    return BS_EDEVICE;
  }
  h->B = batch;
  h->k = k;
  h->V = vocab;
  h->dtype = logits_dtype;
  // 16 logits per thread: measured faster than 32 or 64 per thread on the
  // verify shapes (more, shorter workgroups in flight)
  h->ept = 16;
  h->tile = kThreads * h->ept;
  h->tiles = (vocab + h->tile - 1) / h->tile;
  const size_t pt = (size_t)batch * k * h->tiles;
  if (hipMalloc(&h->block, 3 * align_up(pt * 4)) != hipSuccess) {
    (void)hipGetLastError();
    free(h);
    return BS_ENOMEM;
  }
  h->px = (float*)h->block;
  h->pv = (int*)((char*)h->block + align_up(pt * 4));
  h->pc = (int*)((char*)h->block + 2 * align_up(pt * 4));
  *out = h;
  return BS_OK;
}

int bs_verify_ex(bs_verify_state* h, const void* logits, int64_t row_stride_elems,
                 const int32_t* proposals, int32_t top_k, int32_t min_block,
                 int32_t* accept_len, int32_t* argmax, int32_t* prop_rank) {
  if (!h || !logits || !proposals || !accept_len || !argmax) return BS_EINVAL;
  if (row_stride_elems < h->V || top_k < 1 || min_block < 0 || min_block > h->k)
    return BS_EINVAL;
  const int esize = h->dtype == BS_BF16 ? 2 : 4;
  const bool aligned = ((uintptr_t)logits % 16 == 0) && ((row_stride_elems * esize) % 16 == 0);
  const bool count = top_k > 1 || prop_rank != nullptr;
  K4Args a;
  a.logits = logits;
  a.stride = row_stride_elems;
  a.V = h->V;
  a.tile = h->tile;
  a.tiles = h->tiles;
  a.k = h->k;
  a.B = h->B;
  a.px = h->px;
  a.pv = h->pv;
  a.pc = h->pc;
  a.proposals = proposals;
  a.accept = accept_len;
  a.argmax = argmax;
  a.rank = prop_rank;
  a.top_k = top_k;
  a.min_block = min_block;
  const int rows = h->B * h->k;
  if (rows >= kRowVerifyMinRows) {
    // enough rows to fill the chip: one workgroup per row, results as one tile
    a.tiles = 1;
    if (h->dtype == BS_BF16) {
      if (count) launch_k4_row<uint16_t, true>(a, aligned, rows, h->stream);
      else launch_k4_row<uint16_t, false>(a, aligned, rows, h->stream);
    } else {
      if (count) launch_k4_row<float, true>(a, aligned, rows, h->stream);
      else launch_k4_row<float, false>(a, aligned, rows, h->stream);
    }
  } else {
    launch_k4_tiles(a, h->dtype, count, aligned, dim3(h->tiles, rows), h->stream);
  }
  int rc = launch_status();
  if (rc != BS_OK) return rc;
  if (count)
    hipLaunchKernelGGL((k4_accept<true>), dim3(h->B), dim3(64), 0, h->stream, a);
  else
    hipLaunchKernelGGL((k4_accept<false>), dim3(h->B), dim3(64), 0, h->stream, a);
  return launch_status();
}

int bs_verify(bs_verify_state* h, const void* logits, int64_t row_stride_elems,
              const int32_t* proposals, int32_t* accept_len, int32_t* argmax) {
  return bs_verify_ex(h, logits, row_stride_elems, proposals, 1, 0, accept_len, argmax, nullptr);
}

void bs_verify_destroy(bs_verify_state* h) {
  if (!h) return;
  (void)hipStreamSynchronize(h->stream);
  (void)hipFree(h->block);
  free(h);
}

}  // extern "C"
