// select_two_pass.h -- part of libbeamstep.so, included once by beamstep.hip.
//
// The two-pass (coarse-to-fine) selection: L1, L2, L3.
#pragma once

namespace {

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

// The row state, then (for a live row of an item still running) the tile, as
// in K1: a dead row or a finished item loads nothing.
template <typename T, int EPT, bool ALIGNED>
__device__ __forceinline__ bool cf_load(const CFArgs& a, int r, int v0, int vend,
                                        float (&x)[EPT], float& sr) {
  const int b = r / a.W;
  const T* row = reinterpret_cast<const T*>(a.logits) + (int64_t)r * a.stride;
  const uint32_t done_word = reinterpret_cast<const uint32_t*>(a.done)[b >> 2];
  sr = a.s[r];
  if (((done_word >> (8 * (b & 3))) & 0xff) != 0 || !(sr > -kInf)) return false;
  load_tile<T, EPT, ALIGNED>(row, v0, vend, x);
  return true;
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

}  // namespace
