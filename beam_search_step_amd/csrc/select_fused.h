// select_fused.h -- part of libbeamstep.so, included once by beamstep.hip.
//
// The fused selection (one pass over the logits): K1 expand + per-tile top-K,
// K2 merge + score + prune + finalize, and the finalize sub-step they share.
#pragma once

namespace {

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

// tau for a tile: the w_keep-th largest of the tile's G group maxima (16
// groups of 16 lanes, or 32 groups of 8 lanes), which is a lower bound on the
// tile's w_keep-th best logit (the group maxima are distinct elements). Every
// wave computes it on its own: lane l holds gmax[l % G] and counts, over the
// 15 DPP rotations of its 16-lane row (and for G = 32 over the 16 rotations
// of the other half's values, gmax[(l % 32) ^ 16]), how many of the others
// are larger (gt) and at least as large (ge). A value with gt <= w-1 and
// ge+1 >= w is the w-th largest; all such lanes hold the same value, so the
// rotation direction does not matter.
template <int R>
__device__ __forceinline__ void count_rotations(float h, float g, int& gt, int& ge) {
  if constexpr (R <= 15) {
    const float o = dpp_f<0x120 + R>(h);  // row_ror:R
    gt += o > g ? 1 : 0;
    ge += o >= g ? 1 : 0;
    count_rotations<R + 1>(h, g, gt, ge);
  }
}

template <int G>
__device__ __forceinline__ float tile_tau(const float* gmax, int w_keep) {
  static_assert(G == 16 || G == 32, "16 or 32 group maxima");
  const int lane = threadIdx.x & 63;
  const float g = gmax[lane & (G - 1)];
  int gt = 0, ge = 0;
  count_rotations<1>(g, g, gt, ge);
  if constexpr (G == 32) {
    const float h = gmax[(lane & 31) ^ 16];
    gt += h > g ? 1 : 0;
    ge += h >= g ? 1 : 0;
    count_rotations<1>(h, g, gt, ge);
  }
  const uint64_t q = __ballot(lane < G && gt <= w_keep - 1 && ge + 1 >= w_keep);
  const int l = __builtin_ctzll(q);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g), l));
}

template <int WMAX, typename T, int EPT, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void k1_expand_select(K1Args a) {
  constexpr int kRegion = kListCap / kWaves;  // candidate slots of one wave
  // group maxima for tau: 16 groups of 256 threads / 16 lanes, or 32 of 8
  // lanes when up to 16 candidates are kept. At K = 16 a bound from 16 maxima
  // is their minimum and lets ~54 logits of a 16384-logit tile through to the
  // ranking (Gaussian logits); from 32 maxima ~22. Measured at W = 16, V =
  // 250000: K1 + K2 65.2 us against 69.9 per step. For K <= 4 the count is
  // ~4.4 with 16 groups already.
  constexpr int kG = WMAX >= 16 ? 32 : 16;
  __shared__ float gmax[kG];
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

  // The row's state first: a dead row or a finished item loads nothing. The
  // flag byte is read through its aligned 32-bit word, a scalar load (the
  // flags array is 256-byte aligned and padded to a multiple of 256 bytes).
  // Requesting the tile together with the state instead, so that a live row
  // never waits for the state's round trip, measured no faster (Llama-3-8B
  // and Transformer-base shapes) and read every finished row's logits.
  const uint32_t done_word = reinterpret_cast<const uint32_t*>(a.done)[b >> 2];
  const float sr = a.s[r];
  if (((done_word >> (8 * (b & 3))) & 0xff) != 0 || sr == -kInf) return;  // nothing to expand
  float x[EPT];
  load_tile<T, EPT, ALIGNED>(row, v0, vend, x);

  // expand, per wave: the wave maximum mw and sum of exp(x - mw); the 16-lane
  // row maxima double as the group maxima for tau
  float m = -kInf;
#pragma unroll
  for (int i = 0; i < EPT; ++i) m = fmaxf(m, x[i]);
  m = fmaxf(m, dpp_f<0xb1>(m));   // quad_perm [1,0,3,2]
  m = fmaxf(m, dpp_f<0x4e>(m));   // quad_perm [2,3,0,1]
  m = fmaxf(m, dpp_f<0x141>(m));  // row_half_mirror: every lane has its 8-lane half's max
  if constexpr (kG == 32) {
    if ((lane & 7) == 0) gmax[tid >> 3] = m;
  }
  m = fmaxf(m, dpp_f<0x140>(m));  // row_mirror: every lane has its row's max
  if constexpr (kG == 16) {
    if ((lane & 15) == 0) gmax[tid >> 4] = m;
  }
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
  float tau = tile_tau<kG>(gmax, K);
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
// For W <= 4 (K <= 4) one wave holds every row, and K rounds of the same
// merge over the whole wave replace both stages.
// The workgroup has 256 threads, or 64 when W <= 4 (one wave holds the row
// groups of 4 rows; every use of the thread index stays below 64 then).
template <int WMAX, int H>
__device__ __forceinline__ void select_finalize_item(const K2Args& a) {
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

  // W <= 4: wave 0 holds every row of the item, and lane order is (row, tile)
  // order, so K rounds of a wave-wide merge give the item's best K in exact
  // (score desc, flat index asc) order, with no per-row stage and no LDS
  // round trip; lane r keeps round r's winner. Measured against stages A and
  // B: K1 + K2 13.8-14.1 against 14.8-15.1 us per step at the Llama-3-8B
  // shape, 32,767-33,108 against 31,783-32,177 beam steps/s at
  // Transformer-base (three runs each).
  float fs_w = -kInf;
  int fj_w = 0;
  if constexpr (WMAX <= 4) {
    if (wave == 0) {
      float hs[H];
      int hc[H];
#pragma unroll
      for (int h = 0; h < H; ++h) {
        hs[h] = sc[h][0];
        hc[h] = col[h][0];
      }
      for (int r = 0; r < K; ++r) {
        int bh = 0;
        float bs = hs[0];
#pragma unroll
        for (int h = 1; h < H; ++h)
          if (hs[h] > bs) {
            bs = hs[h];
            bh = h;
          }
        const float M = wave_max_f(bs);
        const uint64_t holders = __ballot(bs == M && M > -kInf);
        if (holders == 0) break;  // uniform: no candidate left
        const int l = __builtin_ctzll(holders);
        int hcol = hc[0];
#pragma unroll
        for (int h = 1; h < H; ++h) hcol = bh == h ? hc[h] : hcol;
        const int wj = __builtin_amdgcn_readlane(w * V + hcol, l);
        if (lane == r) {
          fs_w = M;
          fj_w = wj;
        }
        if (lane == l) {
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
  } else {  // stage A (W > 4): K rounds per row
    const uint64_t below = ((uint64_t)1 << (lane & 15)) - 1;  // lower lanes of the group
    const int gshift = lane & 48;
    // The lane's lists wait in LDS (lane-fastest, 64 KB at most) and only each
    // list's head is in registers: the winning lane reads its next entry, where
    // a register shift of its lists took ~120 moves a round as compiled. K1 + K2
    // 58.7 against 60.8 us per step at the wide shape (three runs each). Lists
    // of H * WMAX > 32 entries (64 tiles of 16 candidates) keep the shift.
    constexpr bool kLdsLists = H * WMAX <= 32;
    __shared__ float lsc[kLdsLists ? H * WMAX : 1][kLdsLists ? kThreads : 1];
    __shared__ int lcol[kLdsLists ? H * WMAX : 1][kLdsLists ? kThreads : 1];
    int ph[H];
    float hs[H];
    int hc[H];
#pragma unroll
    for (int h = 0; h < H; ++h) {
      ph[h] = 0;
      hs[h] = sc[h][0];
      hc[h] = col[h][0];
      if constexpr (kLdsLists) {
#pragma unroll
        for (int i = 1; i < WMAX; ++i) {
          lsc[h * WMAX + i][tid] = sc[h][i];
          lcol[h * WMAX + i][tid] = col[h][i];
        }
      }
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
        if constexpr (kLdsLists) {
          // the winning list's next entry, read from LDS
#pragma unroll
          for (int h = 0; h < H; ++h) {
            if (bh == h) {
              const int q = ++ph[h];
              hs[h] = q < WMAX ? lsc[h * WMAX + q][tid] : -kInf;
              hc[h] = q < WMAX ? lcol[h * WMAX + q][tid] : 0;
            }
          }
        } else {
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
  if constexpr (WMAX <= 4) {
    const uint64_t key = lane < K && fs_w > -kInf ? pack_key(fs_w, fj_w) : 0;
    finalize_item<WMAX>(a, hy, plan, b, lane, key, lp_t, lp_T);
    return;
  }

  // stage B: lane w < W holds the head of row w's list, which stays in LDS;
  // lane r keeps round r's winner
  int pw = 0;
  float hs = lane < W ? row_sc[lane < W ? lane : 0][0] : -kInf, fs = -kInf;
  int hj = lane < W ? row_j[lane < W ? lane : 0][0] : 0, fj = 0;
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
    if (lane == l) {  // the winning row's next entry
      ++pw;
      hs = pw < K ? row_sc[lane][pw] : -kInf;
      hj = pw < K ? row_j[lane][pw] : 0;
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

template <int WMAX, int H>
__global__ __launch_bounds__(kThreads) void k2_select_finalize(K2Args a) {
  select_finalize_item<WMAX, H>(a);
}

}  // namespace
