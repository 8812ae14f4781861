// verify.h -- part of libbeamstep.so, included once by beamstep.hip.
//
// The verify sub-step of blockwise parallel decoding: K4.
#pragma once

namespace {

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

// Verify by row segments (used when there are enough rows to fill the chip):
// grid (segments, rows), a workgroup streams one contiguous segment of a row,
// kRowLoads 16-byte loads per thread per batch, all unconditional (indices
// clamped into the segment, so no branch stands between the loads and the
// compiler waits for a batch only once). A thread visits its columns in
// increasing order, so a strictly larger logit is the only one that moves its
// running maximum and the first index of the maximum is kept; a segment that
// is -inf throughout reports its first column, so that a row that is -inf
// throughout has its first index, 0, after the merge. For the top-k criterion,
// logits that beat the proposal's (larger, or equal at a lower index) are
// counted, in the rare vectors whose maximum reaches it. Segment s of row r
// is tile s of the partials, for the same accept step.
constexpr int kRowLoads = 16;
template <typename T, bool ALIGNED, bool COUNT>
__global__ __launch_bounds__(kThreads) void k4_row(K4Args a) {
  __shared__ float rx[kWaves];
  __shared__ int ri[kWaves];
  __shared__ int rc[kWaves];
  const int r = blockIdx.y, seg = blockIdx.x, nseg = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const T* row = reinterpret_cast<const T*>(a.logits) + (int64_t)r * a.stride;
  const int V = a.V;
  int first;  // the segment's first column
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
    // vectors [qs, qe) of the row; the ragged tail goes with the last segment
    const int qs = (int)((int64_t)nvec * seg / nseg), qe = (int)((int64_t)nvec * (seg + 1) / nseg);
    first = qs * VEC;
    const uint4* rv = reinterpret_cast<const uint4*>(row);
    if (qe > qs) {  // uniform; an empty segment (a row of few vectors) has none
      const int qmax = qe - 1;
      for (int q0 = qs + tid; q0 < qe; q0 += kThreads * kRowLoads) {
        uint4 raw[kRowLoads];
#pragma unroll
        for (int u = 0; u < kRowLoads; ++u) raw[u] = load16_stream(&rv[min(q0 + u * kThreads, qmax)]);
#pragma unroll
        for (int u = 0; u < kRowLoads; ++u) {
          const int q = q0 + u * kThreads;
          if (q < qe) {
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
    if (seg == nseg - 1 && v < V) {  // the tail columns come after every vector column
      const float x = Elem<T>::load1(row + v);
      if (x > bx) {
        bx = x;
        bi = v;
      }
      count(x, v);
    }
  } else {
    // columns [vs, ve) of the row
    const int vs = (int)((int64_t)V * seg / nseg), ve = (int)((int64_t)V * (seg + 1) / nseg);
    first = vs;
    for (int v0 = vs + tid; v0 < ve; v0 += kThreads * kRowLoads) {
      float x[kRowLoads];
#pragma unroll
      for (int u = 0; u < kRowLoads; ++u) x[u] = Elem<T>::load1(row + min(v0 + u * kThreads, ve - 1));
#pragma unroll
      for (int u = 0; u < kRowLoads; ++u) {
        const int v = v0 + u * kThreads;
        if (v < ve) {
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
    const int64_t pt = (int64_t)r * nseg + seg;
    a.px[pt] = bx;
    a.pv[pt] = bi == 0x7fffffff ? first : bi;  // every logit -inf: the first column
    if (COUNT) a.pc[pt] = rc[0] + rc[1] + rc[2] + rc[3];
  }
}

// the merge as its own launch, one wave per item (a device-scope release and
// acquire per workgroup, to let the last one merge, cost far more than the
// second launch on this chip)
template <bool COUNT>
__global__ __launch_bounds__(64) void k4_accept(K4Args a) {
  accept_item<COUNT>(a, blockIdx.x, threadIdx.x);
}

}  // namespace
