// device_common.h -- part of libbeamstep.so, included once by beamstep.hip.
//
// Shared device code: constants, selection-order keys, wave and DPP reductions,
// and the 16-byte logits loads used by every streaming kernel.
#pragma once

namespace {

constexpr int kThreads = 256;           // workgroup size of K1, K2, K4
constexpr int kWaves = kThreads / 64;   // wave64
constexpr int kMaxBeam = 16;
constexpr int kMaxGridRows = 65535;     // rows per launch: the grid's y extent
constexpr int kListCap = 1024;          // LDS candidate list of the top-W
constexpr int kMergeNE = 8;             // K2 candidates per thread per batch
constexpr int kPlanStride = 64;         // int32 words per item of the KV plan
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

// 16 bytes of logits with the nontemporal hint: the logits of a step are
// read once, so keeping them out of the caches leaves room for what is
// reused (measured 8% more verify calls per second)
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16_stream(const void* p) {
  const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kVec = 4;
  __device__ static float load1(const float* p) { return *p; }
  __device__ static void loadv(const float* p, float* out) { unpack(load16_stream(p), out); }
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
  __device__ static void loadv(const uint16_t* p, float* out) { unpack(load16_stream(p), out); }
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

}  // namespace
