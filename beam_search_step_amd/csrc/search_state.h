// search_state.h -- part of libbeamstep.so, included once by beamstep.hip.
//
// The final selection and backtrace (K5).
#pragma once

namespace {

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

}  // namespace
