// init.h -- part of libbeamstep.so, included once by beamstep.hip.
//
// Initialisation of a search's state (k0_init).
#pragma once

namespace {

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
